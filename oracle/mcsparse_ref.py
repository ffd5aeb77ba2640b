"""CPU oracle for MC-Sparse's meta-cached token-level sparse attention.

TEST INFRASTRUCTURE ONLY. This module is imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``.
The library (``libmcsparse``) and its Python binding never import it, and it
imports nothing from them.

It is a plain, slow implementation in float64 (numpy; a library matmul, sort
or log-sum-exp serves as one step). It works on ONE (batch, head) slice at a
time: arrays are ``[N, d]`` with the values of the stored bf16 (or fp32) inputs
widened exactly to float64.

Sources (MC-Sparse, arXiv 2610.06801, as summarised on the pages):
  * paper landing page, Abstract: the cached metadata is query groups, KV
    indices chosen from exact attention probabilities, and dense-minus-sparse
    residuals, reused over the following denoising steps.
  * research walkthrough page (aiwillknow "mc-sparse"), method steps 1-5
    (Figure 6): step 1 Fast PDDP grouping (project on the principal
    direction, split at the median recursively, tile-sized groups); step 2
    dense attention with per-row log-sum-exp, a second QK pass recovering the
    probabilities, per-group accumulation and top-K of single KV tokens;
    step 3 residual R = dense output minus sparse output at the same anchor;
    step 4 reuse of query order, KV indices and R with fresh Q/K/V, adding R
    to the sparse result.

Readings where the pages are silent:
  * softmax scale s = 1/sqrt(d), no mask;
  * "principal direction" = leading eigenvector of the node's centred
    covariance, from a fixed number of power iterations started at the unit
    vector of the largest diagonal entry (lowest index on ties), oriented so
    its largest-magnitude component is positive (lowest index on ties);
  * "median" = a rank split at floor(G_S/2)*T tokens, ties in the projection
    broken by lower token index, lower-projection child first, rows inside a
    group ascending;
  * group accumulation = plain sum of the probabilities over the group's rows;
  * top-K order = (-A, j): equal mass goes to the lower key index; the chosen
    indices are stored ascending;
  * sparse attention = softmax renormalised over the selected keys;
  * R is rounded to bf16 (RNE) from the stored bf16 dense output; the reuse
    output is bf16(sparse + R);
  * whitening for PDDP (listed on the news page only as an open item, never
    defined) = per-dimension standardization of the head's queries before
    grouping. The root's power iteration starts at the lowest dimension of
    nonzero variance, since exact arithmetic ties every standardized variance
    at 1.

Parity status: every function here is pinned by tests in
``tests/test_oracle_*.py`` (closed forms, brute force in exact decimal
arithmetic, library routines, invariants). The only unpinned claim is that
this reading of "Fast PDDP" (and of its whitening) reproduces the authors'
groups: the pages print no groups to check against.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "round_bf16",
    "topk_count",
    "pddp_group",
    "principal_direction",
    "standardize",
    "dense_lse",
    "group_mass",
    "topk_select",
    "sparse_attention",
    "residual",
    "reuse_output",
    "block_select",
    "group_recall",
    "rel_l1",
]


# ---------------------------------------------------------------------------
# storage rounding
# ---------------------------------------------------------------------------

def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as
    float64. bf16 keeps 8 significant bits and fp32's exponent range; values
    are rounded straight from float64 (no double rounding through fp32).
    Values beyond the largest finite bf16 become +-inf; NaN stays NaN."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    finite = np.isfinite(x)
    xf = x[finite]
    # scale of one unit in the last place of an 8-significant-bit number,
    # clamped at bf16's subnormal spacing 2**-133
    mag = np.abs(xf)
    e = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    # guard against log2 rounding at exact powers of two
    e = np.where(2.0 ** e > mag, e - 1, e)
    e = np.where(2.0 ** (e + 1) <= mag, e + 1, e)
    ulp = 2.0 ** np.maximum(e - 7, -133)
    r = np.round(xf / ulp) * ulp  # np.round is round-half-to-even; xf/ulp is exact
    r = np.where(mag == 0, xf, r)
    big = np.abs(r) > 3.3895313892515355e38  # largest finite bf16
    r = np.where(big, np.copysign(np.inf, xf), r)
    out[finite] = r
    out[~finite] = x[~finite]
    return out


def topk_count(density_pct: int, seqlen: int) -> int:
    """K = ceil(pct * N / 100), integer arithmetic."""
    return (int(density_pct) * int(seqlen) + 99) // 100


# ---------------------------------------------------------------------------
# step 1: Fast PDDP query grouping
# ---------------------------------------------------------------------------

def principal_direction(C: np.ndarray, power_iters: int = 16, start: int | None = None) -> np.ndarray:
    """Leading eigenvector of the symmetric PSD matrix C by power iteration.

    u0 = e_j with j = argmax_j C_jj (lowest j on ties), or j = ``start`` when
    given; then exactly ``power_iters`` steps of u <- C u / ||C u||. If C u is
    the zero vector the direction is the zero vector (every projection is
    then 0). The result is oriented so that its largest-magnitude component
    is positive.
    """
    d = C.shape[0]
    u = np.zeros(d)
    u[int(np.argmax(np.diag(C))) if start is None else int(start)] = 1.0
    for _ in range(power_iters):
        w = C @ u
        nrm = math.sqrt(float(np.dot(w, w)))
        if nrm == 0.0:
            return np.zeros(d)
        u = w / nrm
    j = int(np.argmax(np.abs(u)))
    return -u if u[j] < 0 else u


def _split_node(q: np.ndarray, members: np.ndarray, n_left: int, power_iters: int, start: int | None = None):
    """One PDDP split: centre, covariance, principal direction, projection, rank split."""
    X = q[members]
    n = X.shape[0]
    mu = X.sum(axis=0) / n
    Xc = X - mu
    C = (Xc.T @ Xc) / n
    u = principal_direction(C, power_iters, start)
    p = (Xc * u[None, :]).sum(axis=1)  # row by row: identical rows give identical p
    order = np.lexsort((members, p))  # by projection, then by token index
    left = np.sort(members[order[:n_left]])
    right = np.sort(members[order[n_left:]])
    return left, right


def standardize(q: np.ndarray):
    """Whitening as this oracle reads it: every dimension of the head's
    queries centred and scaled to unit variance over the head's N tokens.

    The pages list whitening for PDDP only as an open item and never define
    it. Full whitening would make the root's covariance the identity, with
    no principal direction to split on. So the reading is the per-dimension
    one: x'_d = (x_d - mu_d) / sigma_d, with sigma_d the population standard
    deviation. A dimension of zero variance is left unscaled; it is all zero
    once centred. Returns (x', var).
    """
    N = q.shape[0]
    mu = q.sum(axis=0) / N
    Xc = q - mu
    var = (Xc * Xc).sum(axis=0) / N
    scale = np.where(var > 0, 1.0 / np.sqrt(np.where(var > 0, var, 1.0)), 1.0)
    return Xc * scale, var


def pddp_group(q: np.ndarray, group_size: int, power_iters: int = 16, whiten: bool = False) -> np.ndarray:
    """Fast PDDP grouping of one head's queries ``q [N, d]``.

    Returns ``perm [N]`` (int64): group g is ``perm[g*T : min((g+1)*T, N)]``,
    rows ascending. A node S of n tokens with G_S = ceil(n/T) groups is a leaf
    when G_S == 1; otherwise its first floor(G_S/2)*T tokens in (projection,
    index) order form the left child, the rest the right child, and the left
    child's groups come first.

    ``whiten``: the same recursion on ``standardize(q)``. Its root covariance
    has every nonzero variance equal to 1 in exact arithmetic, so the tie
    rule starts the root's power iteration at the lowest dimension of
    nonzero variance. That decision is taken exactly here, not from the
    rounded diagonal.
    """
    N = q.shape[0]
    T = int(group_size)
    root_start = None
    if whiten:
        q, var = standardize(q)
        nz = np.nonzero(var > 0)[0]
        root_start = int(nz[0]) if nz.size else 0
    out = []
    stack = [np.arange(N, dtype=np.int64)]
    root = True
    while stack:
        members = stack.pop()
        n = members.shape[0]
        G = -(-n // T)
        if G <= 1:
            out.append(np.sort(members))
            continue
        left, right = _split_node(q, members, (G // 2) * T, power_iters, root_start if root else None)
        root = False
        stack.append(right)  # popped after the whole left subtree
        stack.append(left)
    perm = np.concatenate(out) if out else np.zeros(0, dtype=np.int64)
    return perm


# ---------------------------------------------------------------------------
# step 2: dense attention with per-row log-sum-exp
# ---------------------------------------------------------------------------

def dense_lse(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Dense attention for the given query rows.

    s_ij = scale * q_i . k_j;  L_i = max_j s_ij + ln sum_j exp(s_ij - max_j s_ij);
    O_i = sum_j exp(s_ij - L_i) v_j.  Returns (O [M, d], L [M]) in float64.
    """
    s = scale * (q_rows @ k.T)
    m = s.max(axis=1, keepdims=True)
    L = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
    P = np.exp(s - L[:, None])
    return P @ v, L


# ---------------------------------------------------------------------------
# step 2 (cont.): exact probabilities, group accumulation, top-K
# ---------------------------------------------------------------------------

def group_mass(q_group: np.ndarray, k: np.ndarray, lse_group: np.ndarray, scale: float) -> np.ndarray:
    """A_j = sum over the group's rows i of P_ij = exp(scale * q_i . k_j - L_i)."""
    s = scale * (q_group @ k.T)
    return np.exp(s - lse_group[:, None]).sum(axis=0)


def topk_select(A: np.ndarray, K: int) -> np.ndarray:
    """The K keys with the largest mass; equal mass -> lower index; ascending."""
    j = np.arange(A.shape[0])
    order = np.lexsort((j, -A))
    return np.sort(order[:K]).astype(np.int64)


# ---------------------------------------------------------------------------
# steps 3-4: sparse attention, residual, reuse
# ---------------------------------------------------------------------------

def sparse_attention(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, idx: np.ndarray, scale: float) -> np.ndarray:
    """Softmax over the selected keys only (renormalised), taken in ascending index order."""
    ks, vs = k[idx], v[idx]
    s = scale * (q_rows @ ks.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return (e / e.sum(axis=1, keepdims=True)) @ vs


def residual(o_dense_stored: np.ndarray, o_sparse: np.ndarray) -> np.ndarray:
    """R = O_dense - O_sparse, with O_dense the stored (bf16) dense output; R stored as bf16."""
    return round_bf16(o_dense_stored - o_sparse)


def reuse_output(q_rows, k, v, idx, r_stored, scale) -> np.ndarray:
    """Reuse step: bf16(SparseAttn(fresh Q, K, V; cached idx) + cached R)."""
    return round_bf16(sparse_attention(q_rows, k, v, idx, scale) + r_stored)


# ---------------------------------------------------------------------------
# selection variants: block granularity, recall, output error
# ---------------------------------------------------------------------------

def block_select(A: np.ndarray, nblocks: int, block: int) -> np.ndarray:
    """Block granularity: block b is keys [b*block, (b+1)*block) and its mass
    the sum of theirs; among the N // block full blocks the ``nblocks`` of
    largest mass win (equal mass -> lower block); their keys, ascending."""
    nfull = A.shape[0] // block
    bm = A[: nfull * block].reshape(nfull, block).sum(axis=1)
    b = np.arange(nfull)
    chosen = np.sort(np.lexsort((b, -bm))[:nblocks])
    return (chosen[:, None] * block + np.arange(block)[None, :]).reshape(-1).astype(np.int64)


def group_recall(A: np.ndarray, idx: np.ndarray, n_rows: int) -> float:
    """Mean over the group's rows of the probability mass its selected keys carry."""
    return float(A[idx].sum() / n_rows)


def rel_l1(x: np.ndarray, ref: np.ndarray) -> float:
    """sum |x - ref| / sum |ref|."""
    return float(np.abs(x - ref).sum() / np.abs(ref).sum())
