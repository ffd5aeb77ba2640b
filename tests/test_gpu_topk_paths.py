"""Top-K selection at every row length the library dispatches on.

The selection runs differently by row length: rows up to 98304 keys are held
in registers (six sizes, the last on 768 threads), longer rows compact the
first digit's bin into LDS when it fits and re-read the row when it does not. The inputs here make the
exact answer plain without the oracle. Every query is c * e_0 and key j is
k_j * e_0, with k_j on a grid of 257 values, so a group's mass is
exp(scale * c * k_j - L) summed over identical rows. That is strictly
increasing in k_j (adjacent grid values differ in mass by 0.8%, far above
fp32 rounding), and many keys share each value. The top-K are then the keys
of largest k_j, lowest index first among equals (the pages' tie rule as this
library reads it), stored ascending. With all keys equal, every mass ties
and the answer is the first K indices. Those rows leave keys equal to the
K-th largest out, so the partition ranks ties; rows of distinct scores
(two key dimensions) take its plain form, whose indices are staged in LDS
up to a capacity and written straight out beyond it: both are covered at
each capacity's edge."""
import numpy as np
import pytest
import torch

from sparse_attention_diffusion_pddp_amd import binding as mcs

pytestmark = pytest.mark.gpu

D, T = 64, 128


def run_select(kcol, K):
    N = kcol.shape[0]
    q = torch.zeros((1, N, 1, D), dtype=torch.bfloat16)
    q[0, :, 0, 0] = 2.0
    k = torch.zeros((1, N, 1, D), dtype=torch.bfloat16)
    k[0, :, 0, 0] = torch.from_numpy(kcol).to(torch.bfloat16)
    assert torch.equal(k[0, :, 0, 0].double(), torch.from_numpy(kcol)), "grid values are exact in bf16"
    q, k = q.cuda(), k.cuda()
    G = -(-N // T)
    lse = torch.zeros((1, 1, N), dtype=torch.float32, device="cuda")
    perm = torch.arange(N, dtype=torch.int32, device="cuda").reshape(1, 1, N)
    idx = torch.empty((1, 1, G, K), dtype=torch.int32, device="cuda")
    desc = mcs.desc_for(q)
    ws = torch.empty(mcs.select_workspace_size(desc, T, K), dtype=torch.uint8, device="cuda")
    mcs.anchor_select_topk(q, k, lse, perm, T, K, idx, ws=ws)
    torch.cuda.synchronize()
    return idx[0, 0].cpu().numpy()


def expected(kcol, K):
    N = kcol.shape[0]
    order = np.lexsort((np.arange(N), -kcol))  # largest k first, then lowest index
    return np.sort(order[:K])


# register-held rows of 8, 16, 32, 64 and 128 keys per thread on 512
# threads, then 128 per thread on 768 threads (70000 and the full 98304);
# then the long row with the first digit's bin compacted into LDS
@pytest.mark.parametrize("N", [3000, 8000, 16000, 32760, 60000, 70000, 98304, 100000])
def test_topk_graded_keys(lib, N):
    print(f"\n[topk graded N={N}]", flush=True)
    rng = np.random.default_rng(N)
    kcol = rng.integers(-128, 129, size=N).astype(np.float64) / 32.0
    K = (15 * N + 99) // 100
    got = run_select(kcol, K)
    want = expected(kcol, K)
    for g in range(got.shape[0]):
        assert np.array_equal(got[g], want), f"N={N} group {g}"


@pytest.mark.parametrize("N", [32760, 98304, 100000])
def test_topk_all_masses_tied(lib, N):
    """Every key equal: the first K indices. At N = 100000 the first digit's
    bin holds every key, more than LDS keeps, so the row is read again for
    each digit."""
    print(f"\n[topk tied N={N}]", flush=True)
    K = (20 * N + 99) // 100
    got = run_select(np.full(N, 1.5), K)
    want = np.arange(K)
    for g in range(got.shape[0]):
        assert np.array_equal(got[g], want), f"N={N} group {g}"


# one key past a whole number of the register kernel's per-wave segments
# (64 lanes x keys per lane), so the last wave holds a single valid key; the
# mass rows sit in a buffer of exactly G * N * 4 bytes from hipMalloc
@pytest.mark.parametrize("N", [7 * 64 * 8 + 1, 7 * 64 * 16 + 1, 4 * 64 * 32 + 1, 8 * 64 * 128 + 1])
def test_topk_row_one_past_segments_exact_buffer(lib, N):
    import ctypes
    print(f"\n[topk exact buffer N={N}]", flush=True)
    rng = np.random.default_rng(N)
    kcol = rng.integers(-128, 129, size=N).astype(np.float64) / 32.0
    K = (15 * N + 99) // 100
    q = torch.zeros((1, N, 1, D), dtype=torch.bfloat16)
    q[0, :, 0, 0] = 2.0
    k = torch.zeros((1, N, 1, D), dtype=torch.bfloat16)
    k[0, :, 0, 0] = torch.from_numpy(kcol).to(torch.bfloat16)
    q, k = q.cuda(), k.cuda()
    G = -(-N // T)
    lse = torch.zeros((1, 1, N), dtype=torch.float32, device="cuda")
    perm = torch.arange(N, dtype=torch.int32, device="cuda").reshape(1, 1, N)
    idx = torch.empty((1, 1, G, K), dtype=torch.int32, device="cuda")
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
    hip.hipFree.argtypes = [ctypes.c_void_p]
    mass = ctypes.c_void_p()
    assert hip.hipMalloc(ctypes.byref(mass), G * N * 4) == 0
    try:
        desc = mcs.desc_for(q)
        st = lib.mcs_anchor_select_topk(ctypes.byref(desc), ctypes.c_void_p(q.data_ptr()),
                                        ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(lse.data_ptr()),
                                        ctypes.c_void_p(perm.data_ptr()), T, K, ctypes.c_void_p(idx.data_ptr()),
                                        mass, None, 0,
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0, lib.mcs_last_error()
        torch.cuda.synchronize()
    finally:
        hip.hipFree(mass)
    got = idx[0, 0].cpu().numpy()
    want = expected(kcol, K)
    for g in range(G):
        assert np.array_equal(got[g], want), f"N={N} group {g}"


def run_select_2d(a_col, b_col, K):
    """Queries (16, 1/16, 0, ...) and keys (a_j, b_j, 0, ...): the score is
    16 a_j + b_j / 16, exact in the MFMA's fp32 sums."""
    N = a_col.shape[0]
    q = torch.zeros((1, N, 1, D), dtype=torch.bfloat16)
    q[0, :, 0, 0] = 16.0
    q[0, :, 0, 1] = 1.0 / 16.0
    k = torch.zeros((1, N, 1, D), dtype=torch.bfloat16)
    k[0, :, 0, 0] = torch.from_numpy(a_col).to(torch.bfloat16)
    k[0, :, 0, 1] = torch.from_numpy(b_col).to(torch.bfloat16)
    assert torch.equal(k[0, :, 0, 0].double(), torch.from_numpy(a_col))
    assert torch.equal(k[0, :, 0, 1].double(), torch.from_numpy(b_col))
    q, k = q.cuda(), k.cuda()
    G = -(-N // T)
    lse = torch.zeros((1, 1, N), dtype=torch.float32, device="cuda")
    perm = torch.arange(N, dtype=torch.int32, device="cuda").reshape(1, 1, N)
    idx = torch.empty((1, 1, G, K), dtype=torch.int32, device="cuda")
    desc = mcs.desc_for(q)
    ws = torch.empty(mcs.select_workspace_size(desc, T, K), dtype=torch.uint8, device="cuda")
    mcs.anchor_select_topk(q, k, lse, perm, T, K, idx, ws=ws)
    torch.cuda.synchronize()
    return idx[0, 0].cpu().numpy()


# Distinct masses at the top of the row, so the K-th largest is unique and
# the partition takes its plain u >= tau form: with the indices staged in
# LDS (K at the stage's capacity: 4096 for 8 keys a thread, 12288 on 512
# threads, 16384 on 768) and written straight out (one key more).
@pytest.mark.parametrize("N,K", [(4000, 4000), (32760, 12288), (32760, 12289), (60000, 12288), (60000, 12289),
                                 (98304, 16384), (98304, 16385)])
def test_topk_distinct_masses_both_partition_outputs(lib, N, K):
    print(f"\n[topk distinct N={N} K={K}]", flush=True)
    rng = np.random.default_rng(N + K)
    # codes 256 A + B, A in [-128, 127], B in [0, 255]: 65536 distinct scores
    # (256 A + B) / 512, 2.4e-4 apart in scale * score; rows longer than
    # 65536 repeat the lowest code, far below the K-th largest
    codes = rng.permutation(65536)[:min(N, 65536)]
    if N > 65536:
        codes = np.concatenate([codes, np.zeros(N - 65536, dtype=codes.dtype)])
        codes = codes[rng.permutation(N)]
    A, B = codes // 256 - 128, codes % 256
    got = run_select_2d(A / 32.0, B / 32.0, K)
    want = np.sort(np.argsort(-codes, kind="stable")[:K])
    assert codes[np.argsort(-codes, kind="stable")[K - 1]] > 0, "the K-th largest is above the repeated code"
    for g in range(got.shape[0]):
        assert np.array_equal(got[g], want), f"N={N} K={K} group {g}"
