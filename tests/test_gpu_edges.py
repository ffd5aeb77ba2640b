"""GPU edge cases through the C-ABI, each against the oracle or a fixed fact:
full density (sparse == dense, R at the rounding of O), a single selected
key and short sequences (N = 1, one group shorter than the tile, N = T + 1)
in 128- and 64-row groups, all-equal queries, tied keys, batch > 1 with a
strided (packed QKV) layout, bitwise run-to-run determinism, the error path,
and the offload cache's bitwise round trip."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_diffusion_pddp_amd import binding as mcs
from sparse_attention_diffusion_pddp_amd import synth
from tests import parity_util as U

pytestmark = pytest.mark.gpu


def pipeline(q, k, v, T, K, qt=None, kt=None, vt=None):
    """All five calls on GPU tensors; returns CPU copies."""
    B, N, H, d = q.shape
    G = -(-N // T)
    desc = mcs.desc_for(q)
    ws = torch.empty(mcs.pddp_workspace_size(desc, T), dtype=torch.uint8, device="cuda")
    perm = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, H, G, K), dtype=torch.int32, device="cuda")
    mass = torch.empty((B, H, G, N), dtype=torch.float32, device="cuda")
    r = torch.empty_like(q)
    ot = torch.empty_like(q)
    mcs.pddp_group(q, T, perm, ws)
    mcs.anchor_dense_lse(q, k, v, o, lse)
    mcs.anchor_select_topk(q, k, lse, perm, T, K, idx, group_mass=mass)
    mcs.residual(q, k, v, o, perm, T, idx, K, r)
    mcs.sparse_apply(qt if qt is not None else q, kt if kt is not None else k, vt if vt is not None else v,
                     perm, T, idx, K, r, ot)
    torch.cuda.synchronize()
    return dict(perm=perm.cpu().numpy(), o=o.cpu().float().numpy(), lse=lse.cpu().numpy(), idx=idx.cpu().numpy(),
                mass=mass.cpu().double().numpy(), r=r.cpu().float().numpy(), ot=ot.cpu().float().numpy())


def oracle_head(q, k, v, T, K, qt=None, kt=None, vt=None):
    qt = q if qt is None else qt
    kt = k if kt is None else kt
    vt = v if vt is None else vt
    N, d = q.shape
    scale = 1.0 / math.sqrt(d)
    perm = O.pddp_group(q, T)
    od, L = O.dense_lse(q, k, v, scale)
    od = O.round_bf16(od)
    G = -(-N // T)
    idx = np.zeros((G, K), np.int64)
    mass = np.zeros((G, N))
    r = np.zeros_like(od)
    out = np.zeros_like(od)
    for g in range(G):
        rows = perm[g * T:(g + 1) * T]
        mass[g] = O.group_mass(q[rows], k, L[rows], scale)
        idx[g] = O.topk_select(mass[g], K)
        r[rows] = O.residual(od[rows], O.sparse_attention(q[rows], k, v, idx[g], scale))
        out[rows] = O.reuse_output(qt[rows], kt, vt, idx[g], r[rows], scale)
    return dict(perm=perm, o=od, lse=L, idx=idx, mass=mass, r=r, ot=out, T=T,
                inputs=dict(q=q, k=k, v=v, qt=qt, kt=kt, vt=vt))


def compare(gpu, orc, b, h, K, N, name):
    """Groups exact, O and LSE within tolerance, indices audited; then R and
    O_t against the oracle's chain re-run on the GPU's own index rows (the
    oracle's own chain wherever the rows agree), and each of them once more
    stage-isolated on the GPU's own upstream value (O_dense for R, R for O_t)."""
    assert np.array_equal(gpu["perm"][b, h], orc["perm"]), f"{name}: groups"
    U.assert_close(gpu["o"][b, :, h], orc["o"], f"{name}: O")
    U.assert_close(gpu["lse"][b, h], orc["lse"], f"{name}: LSE", max_abs=U.LSE_ABS, rel_l2=1e-4)
    G = orc["idx"].shape[0]
    swaps = sum(U.audit_topk(gpu["idx"][b, h, g], orc["idx"][g], orc["mass"][g], K, N, f"{name} g{g}")
                for g in range(G))
    print(f"{name}: near-tie swaps {swaps}")
    x = orc["inputs"]
    T = orc["T"]
    scale = 1.0 / math.sqrt(x["q"].shape[1])
    want_r = np.zeros_like(orc["r"])
    want_ot = np.zeros_like(orc["r"])
    iso_r = np.zeros_like(orc["r"])
    iso_ot = np.zeros_like(orc["r"])
    got_od, got_r = gpu["o"][b, :, h], gpu["r"][b, :, h]
    for g in range(G):
        rows = orc["perm"][g * T:(g + 1) * T]
        sel = gpu["idx"][b, h, g].astype(np.int64)
        osp = O.sparse_attention(x["q"][rows], x["k"], x["v"], sel, scale)
        want_r[rows] = O.residual(orc["o"][rows], osp)
        want_ot[rows] = O.reuse_output(x["qt"][rows], x["kt"], x["vt"], sel, want_r[rows], scale)
        iso_r[rows] = O.residual(got_od[rows], osp)
        iso_ot[rows] = O.reuse_output(x["qt"][rows], x["kt"], x["vt"], sel, got_r[rows], scale)
    U.assert_close_residual(got_r, want_r, orc["o"], f"{name}: R")
    U.assert_close_chained_reuse(gpu["ot"][b, :, h], want_ot, want_r, f"{name}: O_t")
    U.assert_close_residual(got_r, iso_r, got_od, f"{name}: stage-isolated R")
    U.assert_close(gpu["ot"][b, :, h], iso_ot, f"{name}: stage-isolated O_t")


def head(t, b=0, h=0):
    return U.head_np(t, b, h)


@pytest.mark.parametrize("N,T,d,pct", [(300, 128, 128, 100), (300, 64, 64, 100)])
def test_full_density_sparse_equals_dense(lib, N, T, d, pct):
    w = synth.small_workload(N, heads=1, head_dim=d, group_size=T, density_pct=pct)
    q, k, v = synth.make_qkv(w, seed=11)
    K = w.topk
    assert K == N
    g = pipeline(*(x.cuda() for x in (q, k, v)), T, K)
    # every group selects every key, in order
    assert np.array_equal(g["idx"][0, 0], np.tile(np.arange(N), (w.groups, 1)))
    # R is only the bf16 storage error of O_dense, so sparse + R == dense
    assert np.all(np.abs(g["r"][0, :, 0]) <= np.abs(g["o"][0, :, 0]) * 2**-7 + 2e-3)
    U.assert_close(g["ot"][0, :, 0], g["o"][0, :, 0], "sparse + R vs dense")
    compare(g, oracle_head(head(q), head(k), head(v), T, K), 0, 0, K, N, "K=N")


@pytest.mark.parametrize("T", [128, 64])
def test_single_key(lib, T):
    w = synth.small_workload(500, heads=2, head_dim=128, group_size=T, density_pct=1)
    q, k, v = synth.make_qkv(w, seed=12)
    K = 1
    qt, kt, vt = synth.drift_qkv(w, (q, k, v), step=1, seed=12)
    g = pipeline(*(x.cuda() for x in (q, k, v)), T, K, *(x.cuda() for x in (qt, kt, vt)))
    for h in range(2):
        orc = oracle_head(head(q, 0, h), head(k, 0, h), head(v, 0, h), T, K,
                          head(qt, 0, h), head(kt, 0, h), head(vt, 0, h))
        compare(g, orc, 0, h, K, 500, f"K=1 T={T} h{h}")


@pytest.mark.parametrize("T", [128, 64])
@pytest.mark.parametrize("N", [1, 37, 100, 128, 129])
def test_short_sequences(lib, N, T):
    w = synth.small_workload(N, heads=1, head_dim=128, group_size=T, density_pct=30)
    q, k, v = synth.make_qkv(w, seed=13)
    K = w.topk
    g = pipeline(*(x.cuda() for x in (q, k, v)), T, K)
    compare(g, oracle_head(head(q), head(k), head(v), T, K), 0, 0, K, N, f"N={N} T={T}")
    if N == 1:
        assert np.array_equal(g["o"][0, 0, 0], v[0, 0, 0].float().numpy())


def test_equal_queries_and_tied_keys(lib):
    N, d, T = 600, 64, 64
    w = synth.small_workload(N, heads=1, head_dim=d, group_size=T, density_pct=10)
    q, k, v = synth.make_qkv(w, seed=14)
    q[:] = q[0, 0]                   # all queries equal: PDDP falls back to index order
    k[0, 200:, 0] = k[0, 199, 0]     # 400 identical keys: mass ties among them
    K = w.topk
    g = pipeline(*(x.cuda() for x in (q, k, v)), T, K)
    assert np.array_equal(g["perm"][0, 0], np.arange(N))
    orc = oracle_head(head(q), head(k), head(v), T, K)
    assert np.array_equal(orc["perm"], np.arange(N))
    compare(g, orc, 0, 0, K, N, "ties")


def test_batched_strided_layout(lib):
    """B = 2 with q, k, v as views into one packed [B, N, 3, H, d] buffer."""
    Bn, N, H, d, T = 2, 700, 3, 128, 128
    w = synth.small_workload(N, heads=H, head_dim=d, group_size=T, density_pct=20, batch=Bn)
    q, k, v = synth.make_qkv(w, seed=15)
    packed = torch.stack([q, k, v], dim=2).cuda()      # [B, N, 3, H, d]
    dq, dk, dv = packed[:, :, 0], packed[:, :, 1], packed[:, :, 2]
    assert dq.stride() == (N * 3 * H * d, 3 * H * d, d, 1)
    K = w.topk
    G = -(-N // T)
    desc = mcs.desc_for(dq)
    ws = torch.empty(mcs.pddp_workspace_size(desc, T), dtype=torch.uint8, device="cuda")
    perm = torch.empty((Bn, H, N), dtype=torch.int32, device="cuda")
    o = torch.empty_strided(dq.shape, dq.stride(), dtype=dq.dtype, device="cuda")
    lse = torch.empty((Bn, H, N), dtype=torch.float32, device="cuda")
    idx = torch.empty((Bn, H, G, K), dtype=torch.int32, device="cuda")
    r = torch.empty_strided(dq.shape, dq.stride(), dtype=dq.dtype, device="cuda")
    ot = torch.empty_strided(dq.shape, dq.stride(), dtype=dq.dtype, device="cuda")
    mcs.pddp_group(dq, T, perm, ws)
    mcs.anchor_dense_lse(dq, dk, dv, o, lse)
    mcs.anchor_select_topk(dq, dk, lse, perm, T, K, idx, ws=torch.empty(
        mcs.select_workspace_size(desc, T, K), dtype=torch.uint8, device="cuda"))
    mcs.residual(dq, dk, dv, o, perm, T, idx, K, r)
    mcs.sparse_apply(dq, dk, dv, perm, T, idx, K, r, ot)
    torch.cuda.synchronize()
    g = dict(perm=perm.cpu().numpy(), o=o.cpu().float().numpy(), lse=lse.cpu().numpy(), idx=idx.cpu().numpy(),
             r=r.cpu().float().numpy(), ot=ot.cpu().float().numpy())
    for b in range(Bn):
        for h in (0, H - 1):
            orc = oracle_head(head(q, b, h), head(k, b, h), head(v, b, h), T, K)
            compare(g, orc, b, h, K, N, f"b{b} h{h}")


def test_bitwise_determinism(lib):
    w = synth.small_workload(2000, heads=2, head_dim=128, group_size=128, density_pct=15)
    x = [t.cuda() for t in synth.make_qkv(w, seed=16)]
    a = pipeline(*x, 128, w.topk)
    b = pipeline(*x, 128, w.topk)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


def test_error_path_raises(lib):
    w = synth.small_workload(256, heads=1, head_dim=128, group_size=128, density_pct=10)
    q, k, v = (t.cuda() for t in synth.make_qkv(w, seed=17))
    perm = torch.zeros((1, 1, 256), dtype=torch.int32, device="cuda")
    idx = torch.zeros((1, 1, 2, 26), dtype=torch.int32, device="cuda")
    with pytest.raises(mcs.McsError) as e:
        mcs.sparse_apply(q, k, v, perm, 128, idx, 0, None, torch.empty_like(q))
    assert e.value.status == 1
    with pytest.raises(mcs.McsError) as e:
        mcs.sparse_apply(q, k, v, perm, 96, idx, 26, None, torch.empty_like(q))
    assert e.value.status == 2



def test_binding_checks_buffer_sizes(lib):
    """Index and statistics buffers of the wrong size, dtype or layout are
    refused by the binding before a kernel could run past them."""
    w = synth.small_workload(256, heads=1, head_dim=128, group_size=128, density_pct=10)
    q, k, v = (t.cuda() for t in synth.make_qkv(w, seed=18))
    o = torch.empty_like(q)
    perm = torch.zeros((1, 1, 256), dtype=torch.int32, device="cuda")
    idx = torch.zeros((1, 1, 2, 26), dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="perm"):
        mcs.sparse_apply(q, k, v, perm[..., :200], 128, idx, 26, None, o)
    with pytest.raises(ValueError, match="kv_idx"):
        mcs.sparse_apply(q, k, v, perm, 128, idx[..., :20], 26, None, o)
    with pytest.raises(ValueError, match="kv_idx"):
        mcs.sparse_apply(q, k, v, perm, 128, idx.long(), 26, None, o)
    with pytest.raises(ValueError, match="lse"):
        mcs.anchor_dense_lse(q, k, v, o, torch.empty((1, 1, 255), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError, match="kv_idx"):
        mcs.residual(q, k, v, o, perm, 128, idx.transpose(2, 3), 26, torch.empty_like(q))

def test_rcache_round_trip_and_order(lib):
    """R of 3 layers stored to pinned host memory, prefetched one layer ahead
    on a side stream, acquired on the compute stream: bitwise equal."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    n, nbytes = 3, 1 << 20
    srcs = [torch.randint(0, 2**15, (nbytes // 2,), dtype=torch.int16, device="cuda") for _ in range(n)]
    cache = mcs.RCache(n, nbytes)
    compute = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    for layer, s in enumerate(srcs):
        cache.store(layer, s, compute)
    torch.cuda.synchronize()
    with pytest.raises(mcs.McsError) as e:
        cache.acquire(0, compute)  # nothing prefetched yet
    assert e.value.status == 5
    side.wait_stream(compute)
    cache.prefetch(0, side)
    got = []
    for layer in range(n):
        ptr = cache.acquire(layer, compute)
        if layer + 1 < n:
            cache.prefetch(layer + 1, side)
        dst = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda")
        # copy out of the slot on the compute stream (the slot's reader)
        assert hip.hipMemcpyAsync(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(ptr), nbytes, 3,
                                  ctypes.c_void_p(compute.cuda_stream)) == 0
        got.append(dst)
    torch.cuda.synchronize()
    for s, d in zip(srcs, got):
        assert torch.equal(s, d)
    other = mcs.RCache(2, nbytes)
    with pytest.raises(mcs.McsError) as e:
        other.prefetch(1)  # never stored
    assert e.value.status == 5
    other.close()
    cache.close()


def test_rcache_store_and_prefetch_on_different_streams(lib):
    """A store enqueued on one stream and the prefetch of the same layer on
    another, with no wait between them in the caller: the prefetch waits for
    the store's copy itself. Then a second store of layer 0 right after its
    prefetch, again on another stream: it waits for the upload to finish."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    nbytes = 8 << 20
    first = torch.randint(0, 2**15, (nbytes // 2,), dtype=torch.int16, device="cuda")
    second = torch.randint(0, 2**15, (nbytes // 2,), dtype=torch.int16, device="cuda")
    torch.cuda.synchronize()
    cache = mcs.RCache(2, nbytes)
    compute = torch.cuda.current_stream()
    s_store, s_fetch = torch.cuda.Stream(), torch.cuda.Stream()
    cache.store(0, first, s_store)
    cache.prefetch(0, s_fetch)
    cache.store(0, second, s_store)  # must not overwrite the blob under the upload
    ptr = cache.acquire(0, compute)
    got = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda")
    assert hip.hipMemcpyAsync(ctypes.c_void_p(got.data_ptr()), ctypes.c_void_p(ptr), nbytes, 3,
                              ctypes.c_void_p(compute.cuda_stream)) == 0
    cache.prefetch(0, s_fetch)  # after the reader: waits for it, then for the second store
    ptr2 = cache.acquire(0, compute)
    got2 = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda")
    assert hip.hipMemcpyAsync(ctypes.c_void_p(got2.data_ptr()), ctypes.c_void_p(ptr2), nbytes, 3,
                              ctypes.c_void_p(compute.cuda_stream)) == 0
    torch.cuda.synchronize()
    assert torch.equal(got, first)
    assert torch.equal(got2, second)
    cache.close()


def test_rcache_two_prefetches_into_one_slot_on_different_streams(lib):
    """Layers 0 and 2 share slot 0. Their prefetches are enqueued on two
    streams with no acquire between them: the second waits for the first, so
    the slot ends up holding layer 2 and acquire(2) reads it whole."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    nbytes = 32 << 20
    l0 = torch.randint(0, 2**15, (nbytes // 2,), dtype=torch.int16, device="cuda")
    l2 = torch.randint(0, 2**15, (nbytes // 2,), dtype=torch.int16, device="cuda")
    cache = mcs.RCache(3, nbytes)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    compute = torch.cuda.current_stream()
    cache.store(0, l0, s1)
    cache.store(2, l2, s1)
    torch.cuda.synchronize()
    cache.prefetch(0, s1)
    cache.prefetch(2, s2)
    ptr = cache.acquire(2, compute)
    got = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda")
    assert hip.hipMemcpyAsync(ctypes.c_void_p(got.data_ptr()), ctypes.c_void_p(ptr), nbytes, 3,
                              ctypes.c_void_p(compute.cuda_stream)) == 0
    torch.cuda.synchronize()
    assert torch.equal(got, l2)
    cache.close()
