"""Host-side argument validation under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU: the two host-only sources of the
library are rebuilt with both sanitizers on their host code (the kernels'
objects are reused from the normal build), and a C program calls every entry
point with random and extreme descriptors, sizes, flags and pointers (the
pointers are never dereferenced on the host). It runs only on a machine
without a GPU, with every device hidden as well: calls that pass validation
stop at the first HIP call with MCS_ERR_HIP. Any sanitizer report fails the
test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_attention_diffusion_pddp_amd")
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
KERNEL_OBJS = ["mcs_attention.o", "mcs_select.o", "mcs_pddp.o", "mcs_idxcode.o", "mcs_scratch.o"]

PROGRAM = r"""
#include <stdint.h>
#include <stdio.h>
#include "mcsparse.h"

static uint64_t st = 88172645463325252ull;
static uint64_t rnd(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return st; }
static int64_t pick64(void) {
  static const int64_t v[] = {0, 1, -1, 8, 64, 128, 1536, 32760, 98304, 1 << 20, INT32_MAX, (int64_t)INT32_MAX + 1,
                              INT64_MAX, INT64_MIN, -8, 4096LL * 4096 * 4096, 3, 7, 16, 24};
  return v[rnd() % (sizeof v / sizeof v[0])];
}
static int32_t pick32(void) {
  static const int32_t v[] = {0, 1, -1, 64, 128, 96, 256, 32760, 65536, 524288, 524289, INT32_MAX, INT32_MIN, 2, 16};
  return v[rnd() % (sizeof v / sizeof v[0])];
}
static void *ptr(void) {
  static char buf[4096] __attribute__((aligned(256)));
  switch (rnd() % 4) {
    case 0: return NULL;
    case 1: return buf + 8 * (rnd() % 64);
    case 2: return buf + 1;
    default: return (void *)(uintptr_t)(0x7f0000000000ull + 256 * (rnd() % 1024));
  }
}
int main(void) {
  size_t n;
  int counts[8] = {0};
  for (int it = 0; it < 12000; ++it) {
    mcs_attn_desc_t d;
    d.batch = pick32(); d.heads = pick32(); d.seqlen = pick32(); d.head_dim = (rnd() & 1) ? 128 : pick32();
    d.stride_b = pick64(); d.stride_n = pick64(); d.stride_h = pick64();
    d.scale = (rnd() & 1) ? 0.088f : (float)(int64_t)pick64();
    const int32_t T = (rnd() & 1) ? 128 : pick32(), K = pick32(), iters = pick32();
    mcs_status_t s = 0;
    switch (rnd() % 14) {
      case 0: s = mcs_pddp_group_workspace_size(&d, T, &n); break;
      case 1: s = mcs_anchor_select_topk_workspace_size(&d, T, K, &n); break;
      case 2: s = mcs_kv_idx_bitmap_bytes(&d, T, &n); break;
      case 3: s = mcs_pddp_group(&d, ptr(), T, iters, ptr(), ptr(), (size_t)pick64(), NULL); break;
      case 4: s = (rnd() & 1) ? mcs_pddp_group_ex(&d, ptr(), T, iters, (uint32_t)rnd() & 3u, ptr(), ptr(), (size_t)pick64(), NULL)
                              : mcs_pddp_group_noalloc(&d, ptr(), T, iters, (uint32_t)rnd() & 3u, ptr(), NULL); break;
      case 5: s = mcs_anchor_dense_lse(&d, ptr(), ptr(), ptr(), ptr(), ptr(), NULL); break;
      case 6: s = mcs_anchor_select_topk(&d, ptr(), ptr(), ptr(), ptr(), T, K, ptr(), ptr(), ptr(), (size_t)pick64(), NULL); break;
      case 7: s = mcs_residual(&d, ptr(), ptr(), ptr(), ptr(), ptr(), T, ptr(), K, ptr(), NULL); break;
      case 8: s = mcs_sparse_apply(&d, ptr(), ptr(), ptr(), ptr(), T, ptr(), K, ptr(), ptr(), NULL); break;
      case 9: s = mcs_kv_idx_encode(&d, T, ptr(), K, ptr(), NULL); break;
      case 10: s = mcs_kv_idx_decode(&d, T, ptr(), K, ptr(), NULL); break;
      case 11: { mcs_rcache_t *c = NULL;
                 s = mcs_rcache_create(pick32(), (size_t)pick64() & ((1ull << 20) - 1), (rnd() & 1) ? &c : NULL);
                 if (s == MCS_OK && c) mcs_rcache_destroy(c);
                 break; }
      case 12: { mcs_rcache_t *c = NULL;
                 s = mcs_rcache_create(pick32(), (size_t)pick64(), &c);
                 if (s == MCS_OK && c) mcs_rcache_destroy(c);
                 break; }
      default: { const void *pp;
                 s = mcs_rcache_store(NULL, pick32(), ptr(), NULL) | mcs_rcache_prefetch(NULL, 0, NULL) |
                     mcs_rcache_acquire(NULL, 0, NULL, &pp) | mcs_rcache_host_ptr(NULL, 0, &pp) |
                     mcs_rcache_destroy(NULL);
                 s &= 7; }
    }
    counts[s & 7]++;
    if (s != MCS_OK && mcs_last_error()[0] == 0) { printf("empty error message for status %d\n", s); return 1; }
  }
  printf("ok %d %d %d %d %d %d\n", counts[0], counts[1], counts[2], counts[3], counts[4], counts[5]);
  return 0;
}
"""


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="no ROCm toolchain")
# the program hands made-up device pointers to entry points that would launch
# kernels on them if a GPU were present: it runs only where there is none
@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU driver is present")
def test_entry_points_under_asan_ubsan(tmp_path):
    for o in KERNEL_OBJS:
        assert os.path.exists(os.path.join(BUILD, o)), "build the library first (__graft_entry__.build())"
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    objs = []
    for src in ("mcs_api.cpp", "mcs_rcache.cpp"):
        obj = str(tmp_path / (src[:-4] + ".o"))
        r = subprocess.run([HIPCC, *flags, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        objs.append(obj)
    lib = str(tmp_path / "libmcsparse.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined", "-o", lib, *objs,
                        *[os.path.join(BUILD, o) for o in KERNEL_OBJS]], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    (tmp_path / "fuzz.c").write_text(PROGRAM)
    exe = str(tmp_path / "fuzz")
    r = subprocess.run([CLANG, "-std=c11", "-g", "-O1", "-fsanitize=address,undefined",
                        f"-I{os.path.join(ROOT, 'include')}", str(tmp_path / "fuzz.c"), "-o", exe,
                        f"-L{tmp_path}", "-lmcsparse", f"-Wl,-rpath,{tmp_path}"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               ASAN_OPTIONS="detect_leaks=0:allocator_may_return_null=1", HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    out = run.stdout + run.stderr
    assert run.returncode == 0 and "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-3000:]
    assert run.stdout.strip().startswith("ok")
