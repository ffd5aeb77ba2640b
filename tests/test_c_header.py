"""The C ABI from C: a C11 program that includes include/mcsparse.h (warnings
as errors) links against libmcsparse.so and calls the entry points that need
no GPU. These are the version, workspace sizes, and argument validation,
which rejects every call below before anything is enqueued. This checks that
the header is plain C, and that its declarations match the exported symbols
at link time."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_attention_diffusion_pddp_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "mcsparse.h"

#define CHECK(cond) do { if (!(cond)) { printf("FAIL line %d: %s\n", __LINE__, #cond); return 1; } } while (0)

int main(void) {
  mcs_attn_desc_t d;
  size_t n = 0;
  int32_t perm_dummy[4];
  char ws[64];
  memset(&d, 0, sizeof d);
  d.batch = 1; d.heads = 12; d.seqlen = 32760; d.head_dim = 128;
  d.stride_n = 12 * 128; d.stride_h = 128; d.stride_b = 32760LL * 12 * 128;
  d.scale = 0.08838834764831845f;

  CHECK(mcs_version() == 100);
  CHECK(mcs_pddp_group_workspace_size(&d, 128, &n) == MCS_OK && n > 0);
  CHECK(mcs_anchor_select_topk_workspace_size(&d, 128, 4914, &n) == MCS_OK);
  CHECK(n == (size_t)12 * 256 * 32760 * 4);
  CHECK(mcs_kv_idx_bitmap_bytes(&d, 128, &n) == MCS_OK && n == (size_t)12 * 256 * 1024 * 4);
  /* validation: unsupported head_dim, bad group size, NULL and short buffers */
  d.head_dim = 96;
  CHECK(mcs_pddp_group_workspace_size(&d, 128, &n) == MCS_ERR_UNSUPPORTED);
  d.head_dim = 128;
  CHECK(mcs_pddp_group_workspace_size(&d, 96, &n) == MCS_ERR_UNSUPPORTED);
  CHECK(mcs_pddp_group(&d, NULL, 128, 16, perm_dummy, ws, sizeof ws, NULL) == MCS_ERR_INVALID_ARGUMENT);
  CHECK(strlen(mcs_last_error()) > 0);
  CHECK(mcs_pddp_group_ex(&d, ws, 128, 16, 0x10u, perm_dummy, ws, sizeof ws, NULL) == MCS_ERR_INVALID_ARGUMENT);
  CHECK(mcs_pddp_group_ex(&d, ws, 128, 16, MCS_PDDP_WHITEN, perm_dummy, ws, sizeof ws, NULL) == MCS_ERR_WORKSPACE);
  CHECK(mcs_sparse_apply(&d, ws, ws, ws, perm_dummy, 128, perm_dummy, 0, NULL, ws, NULL) == MCS_ERR_INVALID_ARGUMENT);
  CHECK(mcs_rcache_create(0, 16, NULL) == MCS_ERR_INVALID_ARGUMENT);
  printf("ok\n");
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_header_is_c11_and_links(tmp_path):
    lib = os.path.join(PKG, "libmcsparse.so")
    assert os.path.exists(lib), "build the library first (__graft_entry__.build())"
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    cc = subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                         str(src), "-o", str(exe), "-L", PKG, "-lmcsparse", f"-Wl,-rpath,{PKG}"],
                        capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.strip().endswith("ok"), run.stdout + run.stderr
