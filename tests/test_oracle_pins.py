"""Pins of the CPU oracle against facts fixed outside it.

Each test checks one oracle function against something other than itself:
exact decimal brute force, a library routine (torch SDPA, scipy logsumexp,
numpy eigh, torch's bf16 conversion, Python's sorted), a closed form, or an
invariant. A dropped term, a wrong sign, index or transposed operand in the
oracle fails at least one of them.

Every pin runs twice: on the C++ oracle (``oracle.cpp``, the default export
of ``oracle``) and on the independent numpy transcription of the same steps
(``oracle.mcsparse_ref``). A pin is a plain function of the oracle object
``O`` it checks, so the planted-mistake tests can hand it a mutated one.
"""
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest
import scipy.special
import torch

import oracle.mcsparse_ref as _numpy_oracle
from oracle import cpp as _cpp

getcontext().prec = 50


@pytest.fixture(params=["cpp", "numpy"])
def O(request):
    """The oracle implementation under test."""
    return _cpp.default() if request.param == "cpp" else _numpy_oracle


def bf16_values(rng, shape, scale=1.0):
    """Random float64 values that are exactly representable in bf16."""
    x = torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32))
    return x.to(torch.bfloat16).double().numpy()


# ---------------------------------------------------------------------------
# bf16 rounding
# ---------------------------------------------------------------------------

def test_round_bf16_matches_torch_rne(O):
    rng = np.random.default_rng(1)
    x = rng.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    # exact halfway cases between two bf16 neighbours, both parities
    base = torch.from_numpy(x[:1000]).to(torch.bfloat16).float().numpy()
    bits = base.view(np.uint32)
    halfway = (bits + np.uint32(0x8000)).view(np.float32)
    extra = np.array([0.0, -0.0, 1e-40, -3e-39, 1e-45, 3.3e38, 3.39e38, 3.4e38, 65504.0, 1.0 + 2**-8,
                      1.0 + 3 * 2**-8, 2**-126, 2**-130], dtype=np.float32)
    allx = np.concatenate([x, halfway, extra])
    want = torch.from_numpy(allx).to(torch.bfloat16).double().numpy()
    got = O.round_bf16(allx.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_round_bf16_direct_not_double_rounding(O):
    # 1 + 2^-8 + 2^-30 lies just above the halfway point between bf16 1.0 and 1+2^-7:
    # rounding straight from float64 gives 1+2^-7; via fp32 it would too, but
    # 1 + 2^-8 exactly is a tie and goes to even (1.0).
    assert O.round_bf16(np.array([1 + 2**-8]))[0] == 1.0
    assert O.round_bf16(np.array([1 + 2**-8 + 2**-40]))[0] == 1 + 2**-7
    assert O.round_bf16(np.array([1 + 3 * 2**-8]))[0] == 1 + 2**-6


# ---------------------------------------------------------------------------
# dense attention + LSE
# ---------------------------------------------------------------------------

def _decimal_dense(q, k, v, scale):
    """Exact-to-50-digits softmax attention, pure Python loops."""
    sc = Decimal(repr(scale))
    O_rows, L = [], []
    for qi in q:
        s = [sc * sum(Decimal(float(a)) * Decimal(float(b)) for a, b in zip(qi, kj)) for kj in k]
        z = sum(si.exp() for si in s)
        Li = z.ln()
        p = [(si - Li).exp() for si in s]
        O_rows.append([float(sum(pj * Decimal(float(vj[c])) for pj, vj in zip(p, v))) for c in range(v.shape[1])])
        L.append(float(Li))
    return np.array(O_rows), np.array(L)


def test_dense_lse_decimal_bruteforce(O):
    rng = np.random.default_rng(2)
    q, k, v = bf16_values(rng, (3, 4)), bf16_values(rng, (6, 4)), bf16_values(rng, (6, 4))
    scale = 1 / math.sqrt(4) * 3.0  # sharpen so the max term matters
    o, L = O.dense_lse(q, k, v, scale)
    o_ref, L_ref = _decimal_dense(q, k, v, scale)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L, L_ref, rtol=0, atol=1e-13)


def test_dense_lse_matches_torch_sdpa_and_scipy_logsumexp(O):
    rng = np.random.default_rng(3)
    q, k, v = bf16_values(rng, (70, 64)), bf16_values(rng, (301, 64)), bf16_values(rng, (301, 64))
    scale = 1 / 8.0
    o, L = O.dense_lse(q, k, v, scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None], scale=scale)[0].numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, scipy.special.logsumexp(scale * (q @ k.T), axis=1), rtol=0, atol=1e-12)


def test_dense_single_key_and_zero_keys(O):
    rng = np.random.default_rng(4)
    q, k, v = bf16_values(rng, (5, 8)), bf16_values(rng, (1, 8)), bf16_values(rng, (1, 8))
    o, L = O.dense_lse(q, k, v, 0.3)
    np.testing.assert_array_equal(o, np.repeat(v, 5, axis=0))
    np.testing.assert_allclose(L, 0.3 * (q @ k[0]), rtol=0, atol=1e-15)
    # all-zero keys: uniform attention, O = mean(V), L = ln N
    k0 = np.zeros((37, 8))
    v2 = bf16_values(rng, (37, 8))
    o, L = O.dense_lse(q, k0, v2, 0.3)
    np.testing.assert_allclose(o, np.repeat(v2.mean(axis=0, keepdims=True), 5, axis=0), rtol=0, atol=1e-15)
    np.testing.assert_allclose(L, np.full(5, math.log(37)), rtol=0, atol=1e-15)


# ---------------------------------------------------------------------------
# exact probabilities, group mass, top-K
# ---------------------------------------------------------------------------

def test_group_mass_decimal_bruteforce_and_row_sums(O):
    rng = np.random.default_rng(5)
    q, k = bf16_values(rng, (4, 4)), bf16_values(rng, (7, 4))
    scale = 0.9
    _, L = O.dense_lse(q, k, np.zeros((7, 4)), scale)
    A = O.group_mass(q, k, L, scale)
    # exact: P_ij = exp(s_ij) / sum_j' exp(s_ij'), summed over rows i
    sc = Decimal(repr(scale))
    want = [Decimal(0)] * 7
    for qi in q:
        s = [sc * sum(Decimal(float(a)) * Decimal(float(b)) for a, b in zip(qi, kj)) for kj in k]
        z = sum(x.exp() for x in s)
        for j in range(7):
            want[j] += s[j].exp() / z
    np.testing.assert_allclose(A, [float(w) for w in want], rtol=0, atol=1e-14)
    assert abs(A.sum() - 4.0) < 1e-13  # each row's probabilities sum to one


def test_selection_bruteforce_on_tiny_workload(O):
    """Tiny workload (1 head, N=1024, d=64, T=64, 25%): the oracle's top-K per
    group equals a brute force with per-row max normalisation (no LSE) and a
    full Python sort by (-A, j)."""
    from sparse_attention_diffusion_pddp_amd.synth import WORKLOADS, make_qkv
    w = WORKLOADS["tiny"]
    q, k, v = (t[0, :, 0, :].double().numpy() for t in make_qkv(w, seed=0, dtype=torch.float32))
    scale = 1 / math.sqrt(w.head_dim)
    perm = O.pddp_group(q, w.group_size)
    K = w.topk
    assert K == 256
    s_all = scale * (q @ k.T)
    e = np.exp(s_all - s_all.max(axis=1, keepdims=True))
    P_brute = e / e.sum(axis=1, keepdims=True)
    _, L = O.dense_lse(q, k, v, scale)
    for g in range(w.groups):
        rows = perm[g * 64:(g + 1) * 64]
        A = O.group_mass(q[rows], k, L[rows], scale)
        A_brute = P_brute[rows].sum(axis=0)
        np.testing.assert_allclose(A, A_brute, rtol=1e-12, atol=0)
        brute = sorted(range(len(A_brute)), key=lambda j: (-A_brute[j], j))[:K]
        got = O.topk_select(A, K)
        # equal sets unless two masses straddle the cut within rounding
        if set(got) != set(brute):
            diff = set(got) ^ set(brute)
            gap = max(A[j] for j in diff) - min(A[j] for j in diff)
            assert gap < 1e-12
        assert np.all(np.diff(got) > 0)


def test_topk_tie_rule_and_extremes(O):
    A = np.array([0.5, 0.7, 0.5, 0.7, 0.1, 0.5])
    assert O.topk_select(A, 3).tolist() == [0, 1, 3]  # 0.7, 0.7 then the lowest 0.5
    assert O.topk_select(A, 4).tolist() == [0, 1, 2, 3]
    assert O.topk_select(np.ones(10), 4).tolist() == [0, 1, 2, 3]
    assert O.topk_select(A, 6).tolist() == list(range(6))
    rng = np.random.default_rng(6)
    A = rng.integers(0, 5, 300).astype(float)  # many ties
    want = sorted(sorted(range(300), key=lambda j: (-A[j], j))[:77])
    assert O.topk_select(A, 77).tolist() == want


# ---------------------------------------------------------------------------
# sparse attention, residual, reuse
# ---------------------------------------------------------------------------

def test_sparse_decimal_bruteforce(O):
    rng = np.random.default_rng(7)
    q, k, v = bf16_values(rng, (2, 4)), bf16_values(rng, (9, 4)), bf16_values(rng, (9, 4))
    idx = np.array([1, 4, 5, 8])
    o = O.sparse_attention(q, k, v, idx, 1.3)
    o_ref, _ = _decimal_dense(q, k[idx], v[idx], 1.3)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)


def test_sparse_special_cases(O):
    rng = np.random.default_rng(8)
    q, k, v = bf16_values(rng, (16, 32)), bf16_values(rng, (50, 32)), bf16_values(rng, (50, 32))
    scale = 1 / math.sqrt(32)
    full = np.arange(50)
    od, _ = O.dense_lse(q, k, v, scale)
    np.testing.assert_allclose(O.sparse_attention(q, k, v, full, scale), od, rtol=0, atol=1e-14)
    # one key: output is that key's value row
    np.testing.assert_array_equal(O.sparse_attention(q, k, v, np.array([17]), scale), np.repeat(v[17:18], 16, 0))
    # equal scores (zero queries): mean of V over the selected set
    idx = np.array([2, 3, 10, 40])
    np.testing.assert_allclose(O.sparse_attention(np.zeros((3, 32)), k, v, idx, scale),
                               np.repeat(v[idx].mean(axis=0, keepdims=True), 3, 0), rtol=0, atol=1e-15)


def test_residual_closed_form_and_anchor_identity(O):
    """R_i = (1 - m_i) (Obar_i - O_sparse_i) with m_i the probability mass of the
    selected keys and Obar_i the probability-weighted mean of V over the
    discarded keys; and O_sparse + R reproduces the stored dense output."""
    rng = np.random.default_rng(9)
    q, k, v = bf16_values(rng, (20, 16)), bf16_values(rng, (80, 16)), bf16_values(rng, (80, 16))
    scale = 0.7
    idx = np.sort(rng.choice(80, 23, replace=False))
    rest = np.setdiff1d(np.arange(80), idx)
    od, L = O.dense_lse(q, k, v, scale)
    osp = O.sparse_attention(q, k, v, idx, scale)
    P = np.exp(scale * (q @ k.T) - L[:, None])
    m = P[:, idx].sum(axis=1, keepdims=True)
    obar = (P[:, rest] @ v[rest]) / P[:, rest].sum(axis=1, keepdims=True)
    closed = (1 - m) * (obar - osp)
    R = O.residual(od, osp)
    assert np.all(np.abs(R - closed) <= np.abs(closed) * 2**-8 + 1e-15)
    # anchor identity at storage level
    od_st = O.round_bf16(od)
    R_st = O.residual(od_st, osp)
    assert np.all(np.abs(osp + R_st - od_st) <= np.abs(R_st) * 2**-8 + 1e-300)


def test_full_density_residual_vanishes(O):
    rng = np.random.default_rng(10)
    q, k, v = bf16_values(rng, (12, 16)), bf16_values(rng, (40, 16)), bf16_values(rng, (40, 16))
    od, _ = O.dense_lse(q, k, v, 0.25)
    osp = O.sparse_attention(q, k, v, np.arange(40), 0.25)
    assert np.max(np.abs(O.residual(od, osp))) < 1e-14  # exact arithmetic: R = 0
    # from the stored bf16 output, R is that storage's rounding error
    od_st = O.round_bf16(od)
    assert np.all(np.abs(O.residual(od_st, osp)) <= np.abs(od) * 2**-8 + 1e-14)


def test_reuse_zero_drift_returns_dense(O):
    rng = np.random.default_rng(11)
    q, k, v = bf16_values(rng, (32, 16)), bf16_values(rng, (64, 16)), bf16_values(rng, (64, 16))
    idx = np.sort(rng.choice(64, 10, replace=False))
    od, _ = O.dense_lse(q, k, v, 0.25)
    od_st = O.round_bf16(od)
    R = O.residual(od_st, O.sparse_attention(q, k, v, idx, 0.25))
    out = O.reuse_output(q, k, v, idx, R, 0.25)
    # sparse + R = O_dense + (R's rounding), then one more bf16 rounding
    assert np.all(np.abs(out - od_st) <= (np.abs(R) + np.abs(od_st)) * 2**-8 * 1.0001)
    # and without R the output would be far off: R carries the discarded mass
    osp = O.sparse_attention(q, k, v, idx, 0.25)
    assert np.max(np.abs(osp - od_st)) > 20 * np.max(np.abs(out - od_st))


# ---------------------------------------------------------------------------
# PDDP
# ---------------------------------------------------------------------------

def _check_perm(perm, N, T):
    assert sorted(perm.tolist()) == list(range(N))
    G = -(-N // T)
    for g in range(G):
        grp = perm[g * T: min((g + 1) * T, N)]
        assert len(grp) == (T if g < G - 1 else N - (G - 1) * T)
        assert np.all(np.diff(grp) > 0)


@pytest.mark.parametrize("N,T", [(1000, 64), (3 * 64 + 5, 64), (64, 64), (1, 64), (5 * 128, 128), (777, 128)])
def test_pddp_is_a_tiled_bijection(O, N, T):
    rng = np.random.default_rng(N)
    q = bf16_values(rng, (N, 16))
    perm = O.pddp_group(q, T)
    _check_perm(perm, N, T)


def test_pddp_rank_one_reduces_to_argsort_chunks(O):
    """q_i = a_i w: every node's direction is +-w/|w| oriented by the largest
    |w_j| (here negative), so the groups are consecutive T-chunks of the
    tokens sorted by (sign * a_i, i)."""
    rng = np.random.default_rng(12)
    N, T, d = 7 * 32 + 11, 32, 6
    a = rng.integers(-20, 21, N) / 4.0  # many equal a_i -> index tie-break exercised
    w = np.array([0.5, -2.0, 1.0, 0.25, -1.0, 0.0])  # largest |w_j| is negative
    q = a[:, None] * w[None, :]
    perm = O.pddp_group(q, T)
    order = sorted(range(N), key=lambda i: (-a[i], i))
    G = -(-N // T)
    for g in range(G):
        want = sorted(order[g * T: (g + 1) * T])
        assert perm[g * T: (g + 1) * T].tolist() == want


def test_pddp_two_separated_clusters_split_exactly(O):
    rng = np.random.default_rng(13)
    T, d = 64, 8
    c = np.zeros(d)
    c[3] = 10.0
    lab = rng.permutation(np.r_[np.zeros(T, int), np.ones(T, int)])
    q = bf16_values(rng, (2 * T, d), 0.3) + np.where(lab[:, None] == 1, c, -c)
    perm = O.pddp_group(q, T)
    # the direction is ~ +e_3 (largest component positive): the -c cluster goes left
    assert sorted(perm[:T].tolist()) == sorted(np.nonzero(lab == 0)[0].tolist())
    assert sorted(perm[T:].tolist()) == sorted(np.nonzero(lab == 1)[0].tolist())


def test_pddp_odd_node_splits_at_floor_half(O):
    """A node of three tiles (G_S = 3) puts floor(3/2) = 1 tile left. Three
    tight clusters of T tokens: A far out on dim 0, B and C together on
    dim 0 but apart on dim 1. The root's direction is dim 0, so its lowest
    tile (A) goes left; the right child's direction is dim 1, which then
    separates B from C. Two tiles left instead would put A with half of B
    and C mixed, and the groups would no longer be the clusters."""
    rng = np.random.default_rng(16)
    T, d = 64, 4
    centres = np.array([[-20.0, 0.0, 0, 0], [10.0, -3.0, 0, 0], [10.0, 3.0, 0, 0]])
    lab = rng.permutation(np.repeat(np.arange(3), T))
    q = centres[lab] + bf16_values(rng, (3 * T, d), 0.05)
    perm = O.pddp_group(q, T)
    groups = [sorted(perm[g * T:(g + 1) * T].tolist()) for g in range(3)]
    want = [sorted(np.nonzero(lab == c)[0].tolist()) for c in range(3)]
    assert groups == want


def test_principal_direction_closed_form_iteration_count(O):
    """C = [[2,1],[1,2]] (+ zero block): diagonal tie -> start e_0, and
    C^k e_0 = ((3^k + 1)/2, (3^k - 1)/2): the result pins the start, the count
    of 16 iterations and the normalisation."""
    C = np.zeros((4, 4))
    C[:2, :2] = [[2.0, 1.0], [1.0, 2.0]]
    for iters in (1, 2, 5, 16):
        u = O.principal_direction(C, iters)
        x = np.array([(3**iters + 1) / 2, (3**iters - 1) / 2, 0, 0])
        np.testing.assert_allclose(u, x / np.linalg.norm(x), rtol=0, atol=1e-15)
    u15 = O.principal_direction(C, 15)
    u16 = O.principal_direction(C, 16)
    assert abs(u15[1] - u16[1]) > 1e-9


def test_principal_direction_matches_eigh_with_gap(O):
    rng = np.random.default_rng(14)
    d = 32
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    lam = np.r_[50.0, rng.uniform(0.5, 4.0, d - 1)]
    C = (Qm * lam) @ Qm.T
    u = O.principal_direction(C, 16)
    evals, evecs = np.linalg.eigh(C)
    top = evecs[:, -1]
    j = int(np.argmax(np.abs(top)))
    top = top if top[j] > 0 else -top
    np.testing.assert_allclose(u, top, rtol=0, atol=1e-9)
    assert u[np.argmax(np.abs(u))] > 0


def test_principal_direction_zero_covariance(O):
    assert np.all(O.principal_direction(np.zeros((5, 5)), 16) == 0)


def test_pddp_equal_queries_fall_back_to_index_order(O):
    q = np.ones((300, 8)) * 0.375
    perm = O.pddp_group(q, 64)
    assert perm.tolist() == list(range(300))


def test_pddp_first_split_is_median_of_projection(O):
    """Even G_S: the first split puts exactly the tokens below the projection
    median (on the top eigenvector of the centred covariance, via eigh) left."""
    rng = np.random.default_rng(15)
    N, T, d = 4 * 64, 64, 8
    q = bf16_values(rng, (N, d))
    q[:, 2] *= 6.0  # a dominant direction with a clear gap
    Xc = q - q.mean(axis=0)
    evals, evecs = np.linalg.eigh(Xc.T @ Xc / N)
    top = evecs[:, -1]
    top = top if top[np.argmax(np.abs(top))] > 0 else -top
    p = Xc @ top
    order = np.lexsort((np.arange(N), p))
    perm = O.pddp_group(q, T)
    assert sorted(perm[:2 * T].tolist()) == sorted(order[:2 * T].tolist())


def _three_factor_queries(rng, N):
    """Three independent factors: a on dim 0 at scale 100, b on dims 1-5 at
    scale 1, c on dims 6-7 at scale 0.01, each dim with 5% noise of its own
    scale. Raw variance is dominated by a. After per-dimension
    standardization the b block (five correlated dims) carries the largest
    correlation eigenvalue (~5, against ~2 for c and ~1 for a; 16 power
    iterations leave (2/5)^16 ~ 4e-7 of c). Scaling by 1/variance instead
    would favour c."""
    a, b, c = rng.standard_normal(N), rng.standard_normal(N), rng.standard_normal(N)
    cols = [100 * a] + [b] * 5 + [0.01 * c] * 2
    scales = [100, 1, 1, 1, 1, 1, 0.01, 0.01]
    q = np.stack([col + 0.05 * sc * rng.standard_normal(N) for col, sc in zip(cols, scales)], axis=1)
    return q, a, b, c


def test_whitened_pddp_root_split_follows_the_correlation_eigenvector(O):
    """Whitening (per-dimension standardization): the root split puts left the
    tokens below the median projection on the top eigenvector of the
    correlation matrix (numpy's eigh), the b factor here. The plain split
    follows the covariance's top eigenvector, the a factor. The two left sets
    differ."""
    rng = np.random.default_rng(21)
    N, T = 4 * 64, 64
    q, a, b, c = _three_factor_queries(rng, N)
    Z = (q - q.mean(axis=0)) / q.std(axis=0)
    evals, evecs = np.linalg.eigh(np.corrcoef(q, rowvar=False))
    assert evals[-1] > 4.5 and evals[-2] < 2.2  # a clear gap: b's block first
    top = evecs[:, -1]
    top = top if top[np.argmax(np.abs(top))] > 0 else -top
    p = Z @ top
    want = sorted(np.lexsort((np.arange(N), p))[:2 * T].tolist())
    got = sorted(O.pddp_group(q, T, whiten=True)[:2 * T].tolist())
    assert got == want
    # plain PDDP splits along dim 0 (the a factor), up to the few tokens the
    # other dims' small weight in its direction can move across the median
    plain = set(O.pddp_group(q, T)[:2 * T].tolist())
    low0, high0 = set(np.argsort(q[:, 0])[:2 * T].tolist()), set(np.argsort(-q[:, 0])[:2 * T].tolist())
    assert max(len(plain & low0), len(plain & high0)) >= 2 * T - 4
    assert len(plain & set(want)) < 1.6 * T  # a and b are independent


def test_whitened_pddp_is_exactly_invariant_to_power_of_two_dim_scaling(O):
    """Scaling one dimension by 4 (or 1/4) is exact in floating point, and
    standardization removes it exactly, so the whitened groups are bitwise
    the same. The plain groups are not invariant: the same scaling changes
    them."""
    from sparse_attention_diffusion_pddp_amd.synth import make_qkv, small_workload
    w = small_workload(640, heads=1, head_dim=16, group_size=64, density_pct=15)
    q = make_qkv(w, seed=22, dtype=torch.float32)[0][0, :, 0, :].double().numpy()
    q2 = q.copy()
    q2[:, 5] *= 4.0
    q2[:, 2] *= 0.25
    assert np.array_equal(O.pddp_group(q, 64, whiten=True), O.pddp_group(q2, 64, whiten=True))
    assert not np.array_equal(O.pddp_group(q, 64), O.pddp_group(q2, 64))


def test_standardize_closed_form_and_constant_dims(O):
    q = np.array([[1.0, 5.0, 2.0], [3.0, 5.0, 2.0], [5.0, 5.0, 8.0], [7.0, 5.0, 8.0]])
    z, var = O.standardize(q)
    # dim 0: mean 4, variance 5; dim 1 constant: variance 0, left unscaled (all 0);
    # dim 2: mean 5, variance 9
    np.testing.assert_array_equal(var, [5.0, 0.0, 9.0])
    np.testing.assert_allclose(z[:, 0], np.array([-3.0, -1.0, 1.0, 3.0]) / math.sqrt(5.0), rtol=0, atol=1e-15)
    np.testing.assert_array_equal(z[:, 1], 0.0)
    np.testing.assert_array_equal(z[:, 2], [-1.0, -1.0, 1.0, 1.0])
    # the whitened tree starts its root at the lowest dim of nonzero variance
    # and still yields a tiled bijection
    perm = O.pddp_group(np.repeat(q, 40, axis=0), 32, whiten=True)
    _check_perm(perm, 160, 32)


def test_topk_count_integer_ceil(O):
    assert O.topk_count(25, 1024) == 256
    assert O.topk_count(15, 32760) == 4914
    assert O.topk_count(25, 32760) == 8190
    assert O.topk_count(20, 75600) == 15120
    assert O.topk_count(15, 98304) == 14746
    assert O.topk_count(15, 64000) == 9600
    assert O.topk_count(100, 77) == 77
    assert O.topk_count(1, 1) == 1


# ---------------------------------------------------------------------------
# selection variants (block granularity, recall, output error)
# ---------------------------------------------------------------------------

def test_block_select_of_one_key_blocks_is_the_token_topk(O):
    rng = np.random.default_rng(30)
    A = rng.integers(0, 9, 500).astype(float) / 7.0  # many ties
    for K in (1, 37, 250, 500):
        assert O.block_select(A, K, 1).tolist() == O.topk_select(A, K).tolist()


def test_block_select_bruteforce_ties_and_partial_block(O):
    rng = np.random.default_rng(31)
    N, blk = 1000, 64  # 15 full blocks, keys 960..999 a partial block
    A = rng.random(N)
    A[960:] = 1e6  # the partial block never competes
    A[64:128] = A[192:256]  # blocks 1 and 3 tie exactly: the lower one ranks first
    sums = [math.fsum(A[b * blk:(b + 1) * blk]) for b in range(N // blk)]
    for nb in (1, 4, 9, 15):
        order = sorted(range(N // blk), key=lambda b: (-sums[b], b))[:nb]
        want = [b * blk + t for b in sorted(order) for t in range(blk)]
        assert O.block_select(A, nb, blk).tolist() == want
    # with the tie at the cut, exactly one of blocks 1 and 3 is kept: block 1
    rank = sorted(range(N // blk), key=lambda b: (-sums[b], b))
    cut = rank.index(1) + 1
    got = set(O.block_select(A, cut, blk).tolist())
    assert set(range(64, 128)) <= got and not set(range(192, 256)) & got


def test_group_recall_closed_forms(O):
    rng = np.random.default_rng(32)
    q, k = bf16_values(rng, (12, 8)), bf16_values(rng, (90, 8))
    _, L = O.dense_lse(q, k, np.zeros((90, 8)), 0.6)
    A = O.group_mass(q, k, L, 0.6)
    # every key: each row's probabilities sum to 1
    assert abs(O.group_recall(A, np.arange(90), 12) - 1.0) < 1e-13
    # a hand sum
    idx = np.array([3, 17, 40])
    assert O.group_recall(A, idx, 12) == pytest.approx(float(sum(A[[3, 17, 40]])) / 12, rel=1e-15, abs=0)
    # the top-K carry at least as much mass as any other K keys
    top = O.topk_select(A, 20)
    for _ in range(20):
        other = np.sort(rng.choice(90, 20, replace=False))
        assert O.group_recall(A, top, 12) >= O.group_recall(A, other, 12)


def test_rel_l1_closed_form(O):
    assert O.rel_l1(np.array([1.0, 2.0, 3.0]), np.array([1.0, 1.0, -1.0])) == pytest.approx((0 + 1 + 4) / 3)
    x = np.arange(12.0).reshape(3, 4) - 5
    assert O.rel_l1(x, x) == 0.0
    assert O.rel_l1(2 * x, x) == pytest.approx(1.0)
