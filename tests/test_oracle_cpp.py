"""The C++ oracle against the independent numpy transcription of the same
steps, and its own consistency: thread count never changes a result, and the
whole-head drivers equal the per-group functions they are made of."""
import math

import numpy as np
import pytest
import torch

import oracle.mcsparse_ref as R
from oracle import cpp
from sparse_attention_diffusion_pddp_amd import synth


@pytest.fixture(scope="module")
def C():
    return cpp.default()


def _head(w, seed, dtype=torch.bfloat16):
    return [t[0, :, 0, :].float().numpy().astype(np.float64) for t in synth.make_qkv(w, seed=seed, dtype=dtype)]


@pytest.mark.parametrize("N,d,T,pct,whiten", [(1024, 64, 64, 25, False), (1000, 128, 128, 15, False),
                                              (777, 64, 128, 20, True), (3000, 128, 64, 10, False),
                                              (5000, 32, 128, 5, True)])
def test_cpp_and_numpy_oracles_agree(C, N, d, T, pct, whiten):
    w = synth.small_workload(N, heads=1, head_dim=d, group_size=T, density_pct=pct)
    q, k, v = _head(w, seed=N + d)
    scale = 1.0 / math.sqrt(d)
    perm = C.pddp_group(q, T, whiten=whiten)
    assert np.array_equal(perm, R.pddp_group(q, T, whiten=whiten))
    o_c, L_c = C.dense_lse(q, k, v, scale)
    o_n, L_n = R.dense_lse(q, k, v, scale)
    np.testing.assert_allclose(o_c, o_n, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L_c, L_n, rtol=0, atol=1e-12)
    K = w.topk
    for g in (0, w.groups // 2, w.groups - 1):
        rows = perm[g * T:(g + 1) * T]
        A_c = C.group_mass(q[rows], k, L_c[rows], scale)
        A_n = R.group_mass(q[rows], k, L_c[rows], scale)
        np.testing.assert_allclose(A_c, A_n, rtol=1e-12, atol=1e-300)
        idx = R.topk_select(A_n, K)
        assert np.array_equal(C.topk_select(A_n, K), idx)
        osp_c = C.sparse_attention(q[rows], k, v, idx, scale)
        osp_n = R.sparse_attention(q[rows], k, v, idx, scale)
        np.testing.assert_allclose(osp_c, osp_n, rtol=0, atol=1e-12)
        od = R.round_bf16(o_n[rows])
        np.testing.assert_array_equal(C.residual(od, osp_n), R.residual(od, osp_n))
        r = R.residual(od, osp_n)
        # the reuse output is a bf16 rounding of sums equal to 1e-12: at most one bf16 step apart
        diff = np.abs(C.reuse_output(q[rows], k, v, idx, r, scale) - R.reuse_output(q[rows], k, v, idx, r, scale))
        assert np.all(diff <= np.abs(R.reuse_output(q[rows], k, v, idx, r, scale)) * 2**-7 + 1e-30)


def test_standardize_and_direction_agree(C):
    rng = np.random.default_rng(3)
    q = rng.standard_normal((500, 24)) * rng.uniform(0.1, 10, 24)
    q[:, 5] = 2.5  # a constant dimension
    z_c, var_c = C.standardize(q)
    z_n, var_n = R.standardize(q)
    np.testing.assert_allclose(var_c, var_n, rtol=1e-13, atol=0)
    np.testing.assert_allclose(z_c, z_n, rtol=0, atol=1e-12)
    cov = np.cov(q, rowvar=False)
    for it in (1, 3, 16):
        np.testing.assert_allclose(C.principal_direction(cov, it), R.principal_direction(cov, it), rtol=0, atol=1e-12)
    np.testing.assert_allclose(C.principal_direction(cov, 16, start=7), R.principal_direction(cov, 16, start=7),
                               rtol=0, atol=1e-12)


def test_round_bf16_agrees_bitwise(C):
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-40, 38, 100000),
                        [0.0, -0.0, np.inf, -np.inf, 3.3895313892515355e38, 3.39e38, 1e-45, -1e-41]])
    np.testing.assert_array_equal(C.round_bf16(x), R.round_bf16(x))


def test_thread_count_changes_nothing():
    one, many = cpp.CppOracle(threads=1), cpp.CppOracle(threads=7)
    w = synth.small_workload(2500, heads=1, head_dim=64, group_size=128, density_pct=12)
    q, k, v = _head(w, seed=9)
    scale = 1.0 / 8.0
    for whiten in (False, True):
        assert np.array_equal(one.pddp_group(q, 128, whiten=whiten), many.pddp_group(q, 128, whiten=whiten))
    perm = one.pddp_group(q, 128)
    a, b = one.anchor_head(q, k, v, perm, 128, w.topk, scale, with_mass=True), \
        many.anchor_head(q, k, v, perm, 128, w.topk, scale, with_mass=True)
    for key in a:
        assert np.array_equal(a[key], b[key]), key
    assert np.array_equal(one.reuse_head(q, k, v, perm, 128, a["idx"], a["r"], scale),
                          many.reuse_head(q, k, v, perm, 128, a["idx"], a["r"], scale))


def test_head_drivers_equal_their_parts(C):
    w = synth.small_workload(1100, heads=1, head_dim=64, group_size=128, density_pct=20)
    q, k, v = _head(w, seed=10)
    qt, kt, vt = [x + 0.03 * np.random.default_rng(11).standard_normal(x.shape) for x in (q, k, v)]
    scale = 1.0 / 8.0
    T, K = 128, w.topk
    perm = C.pddp_group(q, T)
    a = C.anchor_head(q, k, v, perm, T, K, scale, with_mass=True)
    od, L = C.dense_lse(q, k, v, scale)
    od = C.round_bf16(od)
    assert np.array_equal(a["o_dense"], od) and np.array_equal(a["lse"], L)
    out = C.reuse_head(qt, kt, vt, perm, T, a["idx"], a["r"], scale)
    for g in range(w.groups):
        rows = perm[g * T:(g + 1) * T]
        A = C.group_mass(q[rows], k, L[rows], scale)
        assert np.array_equal(a["mass"][g], A)
        idx = C.topk_select(A, K)
        assert np.array_equal(a["idx"][g], idx)
        r = C.residual(od[rows], C.sparse_attention(q[rows], k, v, idx, scale))
        assert np.array_equal(a["r"][rows], r)
        assert np.array_equal(out[rows], C.reuse_output(qt[rows], kt, vt, idx, r, scale))
