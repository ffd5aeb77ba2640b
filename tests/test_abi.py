"""The C-ABI library loads, exports every symbol include/mcsparse.h declares,
and rejects bad arguments before anything reaches the GPU (these calls make
no HIP call, so they run on a host without a GPU)."""
import ctypes
import os
import re

import pytest

from sparse_attention_diffusion_pddp_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    txt = open(os.path.join(ROOT, "include", "mcsparse.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(mcs_[a-z0-9_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def lib():
    return B.load()


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert len(names) == 22
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(s[0] for s in B.SIGNATURES) == names
    assert lib.mcs_version() == 100


def desc(B_=1, H=2, N=1000, d=128, scale=0.088):
    return B.Desc(B_, H, N, d, N * H * d, H * d, d, scale)


FAKE = ctypes.c_void_p(1 << 20)  # 16-byte aligned, never dereferenced: validation fails first


def status(lib, fn, *args):
    return getattr(lib, fn)(*args)


def test_validation_codes(lib):
    d = desc()
    null = None
    s = lib.mcs_sparse_apply(None, FAKE, FAKE, FAKE, FAKE, 128, FAKE, 10, None, FAKE, None)
    assert s == 1 and b"desc" in lib.mcs_last_error()
    bad = desc(d=96)
    assert lib.mcs_sparse_apply(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, 128, FAKE, 10, None, FAKE, None) == 2
    assert lib.mcs_sparse_apply(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 96, FAKE, 10, None, FAKE, None) == 2
    assert lib.mcs_sparse_apply(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 128, FAKE, 0, None, FAKE, None) == 1
    assert lib.mcs_sparse_apply(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 128, FAKE, 1001, None, FAKE, None) == 1
    assert b"topk" in lib.mcs_last_error()
    mis = ctypes.c_void_p((1 << 20) + 8)
    assert lib.mcs_sparse_apply(ctypes.byref(d), mis, FAKE, FAKE, FAKE, 128, FAKE, 10, None, FAKE, None) == 1
    assert b"aligned" in lib.mcs_last_error()
    # output aliasing an input
    assert lib.mcs_sparse_apply(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 128, FAKE, 10, None, FAKE, None) == 1
    assert b"overlaps" in lib.mcs_last_error()
    assert lib.mcs_anchor_dense_lse(ctypes.byref(d), FAKE, FAKE, FAKE, null, None, None) == 1
    bad_stride = B.Desc(1, 2, 1000, 128, 1000 * 2 * 128, 2 * 128 + 4, 128, 0.1)
    assert lib.mcs_anchor_dense_lse(ctypes.byref(bad_stride), FAKE, FAKE, FAKE, FAKE, None, None) == 1
    assert lib.mcs_pddp_group(ctypes.byref(d), FAKE, 128, 0, FAKE, FAKE, 1 << 30, None) == 1
    assert lib.mcs_pddp_group(ctypes.byref(d), FAKE, 128, 16, FAKE, FAKE, 16, None) == 3
    assert lib.mcs_pddp_group_ex(ctypes.byref(d), FAKE, 128, 16, 2, FAKE, FAKE, 1 << 30, None) == 1
    assert b"flag" in lib.mcs_last_error()
    assert lib.mcs_pddp_group_ex(ctypes.byref(d), FAKE, 128, 16, 1, FAKE, FAKE, 16, None) == 3
    assert lib.mcs_anchor_select_topk(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 128, 10, FAKE, None, FAKE, 16, None) == 3
    assert lib.mcs_residual(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 64, FAKE, 0, FAKE, None) == 1



def test_descriptor_layout_checks(lib):
    """Strided layouts: rows that overlap, strides whose extent overflows and
    dimensions whose product overflows are rejected before any arithmetic
    can wrap; a packed-qkv view and a heads-major layout are accepted."""
    n = ctypes.c_size_t()

    def ws(d):
        return lib.mcs_pddp_group_workspace_size(ctypes.byref(d), 128, ctypes.byref(n))

    H, N, dd = 12, 32760, 128
    assert ws(B.Desc(1, H, N, dd, N * 3 * H * dd, 3 * H * dd, dd, 0.1)) == 0  # q of a packed qkv
    assert ws(B.Desc(2, H, N, dd, H * N * dd, dd, N * dd, 0.1)) == 0  # [B, H, N, d] storage
    # heads interleaved into one token's row: (n=1, h=0) and (n=0, h=1) share memory
    assert ws(B.Desc(1, H, N, dd, N * H * dd, dd, dd, 0.1)) == 1
    assert b"overlap" in lib.mcs_last_error()
    assert ws(B.Desc(1, H, N, dd, N * H * dd, 0, dd, 0.1)) == 1  # every token on one row
    big = (1 << 63) - 8
    assert ws(B.Desc(2, 2, 2, dd, big, big // 2 - 4, dd, 0.1)) == 1
    assert ws(B.Desc(2, H, N, dd, 1 << 40, H * dd, dd, 0.1)) == 0  # a wide batch stride is fine
    i32 = (1 << 31) - 1
    assert ws(B.Desc(i32, i32, 1, dd, 8, 8, 8, 0.1)) == 1
    assert b"2^31" in lib.mcs_last_error()
    assert ws(B.Desc(1, 1, i32, dd, 8, dd, 8, 0.1)) == 2
    assert b"seqlen" in lib.mcs_last_error()
    assert ws(B.Desc(1, 1, 1, dd, 0, 0, 0, float("inf"))) == 1


def test_outputs_overlapping_other_buffers_are_rejected(lib):
    """Each output is checked against every other buffer of the call with
    both buffers' own extents (never dereferenced: validation fails first)."""
    d = desc()  # B=1, H=2, N=1000, d=128: tensors 512,000 B; per-token arrays 8,000 B
    base = 1 << 30

    def at(off):
        return ctypes.c_void_p(base + off)

    q, k, v = at(0), at(1 << 20), at(2 << 20)
    o, r = at(3 << 20), at(4 << 20)
    perm, idx = at(5 << 20), at(6 << 20)  # idx: 2 heads x 8 groups x 10 keys x 4 B = 640 B
    assert lib.mcs_sparse_apply(ctypes.byref(d), q, k, v, perm, 128, idx, 10, r, at((5 << 20) - 16), None) == 1
    assert b"o overlaps perm" in lib.mcs_last_error()
    assert lib.mcs_residual(ctypes.byref(d), q, k, v, o, perm, 128, idx, 10, at((6 << 20) - 256 * 1024), None) == 1
    assert b"r overlaps kv_idx" in lib.mcs_last_error()
    lse = at(7 << 20)
    assert lib.mcs_anchor_dense_lse(ctypes.byref(d), q, k, v, o, at((3 << 20) + 4096), None) == 1
    assert b"overlaps lse" in lib.mcs_last_error()
    # top-K output inside the mass workspace
    n = ctypes.c_size_t()
    assert lib.mcs_anchor_select_topk_workspace_size(ctypes.byref(d), 128, 10, ctypes.byref(n)) == 0
    ws = at(8 << 20)
    assert lib.mcs_anchor_select_topk(ctypes.byref(d), q, k, lse, perm, 128, 10, at((8 << 20) + 4096), None, ws,
                                      n.value, None) == 1
    assert b"overlaps kv_idx" in lib.mcs_last_error()
    # PDDP's perm inside its workspace
    assert lib.mcs_pddp_group_workspace_size(ctypes.byref(d), 128, ctypes.byref(n)) == 0
    assert lib.mcs_pddp_group(ctypes.byref(d), q, 128, 16, at((8 << 20) + 64), ws, n.value, None) == 1
    assert b"perm overlaps ws" in lib.mcs_last_error()
    # a bitmap that starts inside a long index array (the index array is the longer one)
    big = B.Desc(1, 2, 1000, 128, 1000 * 2 * 128, 2 * 128, 128, 0.088)
    assert lib.mcs_kv_idx_encode(ctypes.byref(big), 128, idx, 900, at((6 << 20) + 20000), None) == 1
    assert b"overlap" in lib.mcs_last_error()


def test_binding_refuses_host_tensors(lib):
    """The library takes bare pointers; the binding refuses tensors that do
    not live on the GPU before any call reaches it."""
    import torch
    q = torch.zeros((1, 300, 2, 128), dtype=torch.bfloat16)
    perm = torch.zeros((1, 2, 300), dtype=torch.int32)
    idx = torch.zeros((1, 2, 3, 10), dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensor"):
        B.sparse_apply(q, q, q, perm, 128, idx, 10, None, torch.empty_like(q))
    with pytest.raises(ValueError, match="GPU tensor"):
        B.anchor_dense_lse(q, q, q, torch.empty_like(q))


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    """No fallback path: without the built library every call raises."""
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        B.load(str(tmp_path / "libmcsparse.so"))

def test_workspace_sizes(lib):
    d = desc(H=12, N=32760)
    n = ctypes.c_size_t()
    assert lib.mcs_anchor_select_topk_workspace_size(ctypes.byref(d), 128, 4914, ctypes.byref(n)) == 0
    assert n.value == 12 * 256 * 32760 * 4
    assert lib.mcs_pddp_group_workspace_size(ctypes.byref(d), 128, ctypes.byref(n)) == 0
    assert n.value > 12 * 32760 * 12  # projections + scratch order at least
    small = desc(H=1, N=100)
    assert lib.mcs_pddp_group_workspace_size(ctypes.byref(small), 128, ctypes.byref(n)) == 0
    assert n.value > 0


def test_rcache_argument_checks(lib):
    h = ctypes.c_void_p()
    assert lib.mcs_rcache_create(0, 1024, ctypes.byref(h)) == 1
    assert lib.mcs_rcache_create(2, 1000, ctypes.byref(h)) == 1
    assert lib.mcs_rcache_create(2, 1024, None) == 1
    assert lib.mcs_rcache_store(None, 0, FAKE, None) == 1
    assert lib.mcs_rcache_destroy(None) == 1


def test_kv_idx_codec_argument_checks(lib):
    d = desc(H=12, N=32760)
    n = ctypes.c_size_t()
    assert lib.mcs_kv_idx_bitmap_bytes(ctypes.byref(d), 128, ctypes.byref(n)) == 0
    assert n.value == 12 * 256 * 1024 * 4  # ceil(32760 / 32) = 1024 words per group
    assert lib.mcs_kv_idx_bitmap_bytes(ctypes.byref(d), 96, ctypes.byref(n)) == 2
    other = ctypes.c_void_p((1 << 30))
    assert lib.mcs_kv_idx_encode(ctypes.byref(d), 128, FAKE, 0, other, None) == 1
    assert lib.mcs_kv_idx_decode(ctypes.byref(d), 128, other, 32761, FAKE, None) == 1
    assert lib.mcs_kv_idx_encode(ctypes.byref(d), 128, FAKE, 10, FAKE, None) == 1
    assert b"overlap" in lib.mcs_last_error()
    assert lib.mcs_kv_idx_encode(ctypes.byref(d), 128, None, 10, other, None) == 1
    mis = ctypes.c_void_p((1 << 30) + 2)
    assert lib.mcs_kv_idx_decode(ctypes.byref(d), 128, mis, 10, FAKE, None) == 1
    big = desc(H=1, N=(1 << 19) + 1)
    assert lib.mcs_kv_idx_encode(ctypes.byref(big), 128, FAKE, 10, other, None) == 2


def test_noalloc_validation_on_the_host(lib):
    """mcs_pddp_group_noalloc checks its arguments, and that one head's
    workspace fits the library's scratch, before it looks up the scratch or
    launches anything (no GPU here)."""
    d = desc(N=1000)
    assert lib.mcs_pddp_group_noalloc(ctypes.byref(d), FAKE, 128, 16, 0, None, None) == 1
    assert lib.mcs_pddp_group_noalloc(ctypes.byref(d), FAKE, 128, 16, 2, FAKE, None) == 1
    assert b"flag" in lib.mcs_last_error()
    assert lib.mcs_pddp_group_noalloc(ctypes.byref(d), FAKE, 128, 0, 0, FAKE, None) == 1
    assert lib.mcs_pddp_group_noalloc(ctypes.byref(d), FAKE, 96, 16, 0, FAKE, None) == 2
    big = desc(H=1, N=200000)
    assert lib.mcs_pddp_group_noalloc(ctypes.byref(big), FAKE, 128, 16, 0, FAKE, None) == 2
    assert b"scratch" in lib.mcs_last_error()


def test_grouping_refuses_more_heads_than_its_grid_rows(lib):
    """The grouping kernels run one grid row per (batch, head); more than
    65535 heads is refused on the host, for every grouping call."""
    d = B.Desc(2, 40000, 64, 128, 40000 * 64 * 128, 128, 64 * 128, 0.088)
    n = ctypes.c_size_t()
    assert lib.mcs_pddp_group_workspace_size(ctypes.byref(d), 128, ctypes.byref(n)) == 2
    assert b"65535" in lib.mcs_last_error()
    assert lib.mcs_pddp_group(ctypes.byref(d), FAKE, 128, 16, FAKE, FAKE, 1 << 40, None) == 2
    assert lib.mcs_pddp_group_noalloc(ctypes.byref(d), FAKE, 128, 16, 0, FAKE, None) == 2


def test_select_blocks_validation_on_the_host(lib):
    d = desc(N=1000)
    n = ctypes.c_size_t()
    assert lib.mcs_select_blocks_workspace_size(ctypes.byref(d), 128, 64, 15, ctypes.byref(n)) == 0
    assert n.value > 0
    assert lib.mcs_select_blocks_workspace_size(ctypes.byref(d), 128, 96, 2, ctypes.byref(n)) == 2  # not a multiple of 64
    assert lib.mcs_select_blocks_workspace_size(ctypes.byref(d), 128, 64, 16, ctypes.byref(n)) == 1  # 15 full blocks
    assert lib.mcs_select_blocks_workspace_size(ctypes.byref(d), 128, 64, 0, ctypes.byref(n)) == 1
    short = desc(N=50)
    assert lib.mcs_select_blocks_workspace_size(ctypes.byref(short), 128, 64, 1, ctypes.byref(n)) == 1
    assert b"full block" in lib.mcs_last_error()
    assert lib.mcs_select_blocks(ctypes.byref(d), FAKE, 128, 64, 4, FAKE, FAKE, 16, None) == 3  # workspace too small
