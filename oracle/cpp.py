"""ctypes front of the C++ oracle (``mcsparse_oracle.cpp``), test
infrastructure only.

``CppOracle(path)`` exposes the same functions, with the same signatures and
float64 numpy arrays, as the numpy transcription in ``mcsparse_ref``:
``round_bf16``, ``topk_count``, ``pddp_group``, ``principal_direction``,
``standardize``, ``dense_lse``, ``group_mass``, ``topk_select``,
``sparse_attention``, ``residual``, ``reuse_output``; plus the whole-head
drivers ``reuse_head`` and ``anchor_head`` that spread a head's groups over
``threads`` std::thread workers. The default instance loads
``oracle/libmcsoracle.so`` (built by ``python -m oracle.build``).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libmcsoracle.so")

_d = ctypes.c_double
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_pd = ctypes.POINTER(ctypes.c_double)
_pl = ctypes.POINTER(ctypes.c_int64)

_SIGS = {
    "orc_version": (_i32, []),
    "orc_mutant": (_i32, []),
    "orc_round_bf16": (None, [_pd, _i64, _pd]),
    "orc_principal_direction": (None, [_pd, _i32, _i32, _i32, _pd]),
    "orc_standardize": (None, [_pd, _i32, _i32, _pd, _pd]),
    "orc_pddp_group": (None, [_pd, _i32, _i32, _i32, _i32, _i32, _i32, _pl]),
    "orc_dense_lse": (None, [_pd, _i32, _pd, _pd, _i32, _i32, _d, _i32, _pd, _pd]),
    "orc_group_mass": (None, [_pd, _i32, _pd, _i32, _i32, _pd, _d, _i32, _pd]),
    "orc_topk_select": (None, [_pd, _i32, _i32, _pl]),
    "orc_sparse_attention": (None, [_pd, _i32, _pd, _pd, _i32, _pl, _i32, _d, _pd]),
    "orc_residual": (None, [_pd, _pd, _i64, _pd]),
    "orc_reuse_output": (None, [_pd, _i32, _pd, _pd, _i32, _pl, _i32, _pd, _d, _pd]),
    "orc_block_select": (None, [_pd, _i32, _i32, _i32, _pl]),
    "orc_group_recall": (_d, [_pd, _pl, _i32, _i32]),
    "orc_rel_l1": (_d, [_pd, _pd, _i64]),
    "orc_reuse_head": (None, [_pd, _pd, _pd, _i32, _i32, _pl, _i32, _pl, _i64, _pl, _i32, _pd, _d, _i32, _pd]),
    "orc_anchor_head": (None, [_pd, _pd, _pd, _i32, _i32, _pl, _i32, _i32, _d, _i32, _pd, _pd, _pl, _pd, _pd]),
}


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _i64a(x):
    return np.ascontiguousarray(x, dtype=np.int64)


def _p(a):
    return a.ctypes.data_as(_pd)


def _pi(a):
    return a.ctypes.data_as(_pl)


class CppOracle:
    """The C++ oracle loaded from one shared object."""

    def __init__(self, path: str = LIB, threads: int | None = None):
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m oracle.build`")
        self.lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(self.lib, name)
            fn.restype = res
            fn.argtypes = args
        self.threads = threads or default_threads()
        self.mutant = self.lib.orc_mutant()

    # ---- storage rounding -------------------------------------------------
    def round_bf16(self, x):
        a = _f64(x)
        out = np.empty_like(a)
        self.lib.orc_round_bf16(_p(a), a.size, _p(out))
        return out

    @staticmethod
    def topk_count(density_pct: int, seqlen: int) -> int:
        """K = ceil(pct * N / 100), integer arithmetic."""
        return (int(density_pct) * int(seqlen) + 99) // 100

    # ---- step 1 -------------------------------------------------------------
    def principal_direction(self, C, power_iters: int = 16, start: int | None = None):
        C = _f64(C)
        u = np.empty(C.shape[0])
        self.lib.orc_principal_direction(_p(C), C.shape[0], power_iters, -1 if start is None else int(start), _p(u))
        return u

    def standardize(self, q):
        q = _f64(q)
        z = np.empty_like(q)
        var = np.empty(q.shape[1])
        self.lib.orc_standardize(_p(q), q.shape[0], q.shape[1], _p(z), _p(var))
        return z, var

    def pddp_group(self, q, group_size: int, power_iters: int = 16, whiten: bool = False):
        q = _f64(q)
        perm = np.empty(q.shape[0], dtype=np.int64)
        self.lib.orc_pddp_group(_p(q), q.shape[0], q.shape[1], int(group_size), int(power_iters), int(bool(whiten)),
                                self.threads, _pi(perm))
        return perm

    # ---- step 2 -------------------------------------------------------------
    def dense_lse(self, q_rows, k, v, scale: float):
        q, k, v = _f64(q_rows), _f64(k), _f64(v)
        o = np.empty((q.shape[0], v.shape[1]))
        L = np.empty(q.shape[0])
        self.lib.orc_dense_lse(_p(q), q.shape[0], _p(k), _p(v), k.shape[0], q.shape[1], float(scale), self.threads,
                               _p(o), _p(L))
        return o, L

    def group_mass(self, q_group, k, lse_group, scale: float):
        q, k, L = _f64(q_group), _f64(k), _f64(lse_group)
        A = np.empty(k.shape[0])
        self.lib.orc_group_mass(_p(q), q.shape[0], _p(k), k.shape[0], q.shape[1], _p(L), float(scale), self.threads,
                                _p(A))
        return A

    def topk_select(self, A, K: int):
        A = _f64(A)
        idx = np.empty(int(K), dtype=np.int64)
        self.lib.orc_topk_select(_p(A), A.shape[0], int(K), _pi(idx))
        return idx

    # ---- steps 3-4 ----------------------------------------------------------
    def sparse_attention(self, q_rows, k, v, idx, scale: float):
        q, k, v, idx = _f64(q_rows), _f64(k), _f64(v), _i64a(idx)
        o = np.empty((q.shape[0], v.shape[1]))
        self.lib.orc_sparse_attention(_p(q), q.shape[0], _p(k), _p(v), q.shape[1], _pi(idx), idx.shape[0],
                                      float(scale), _p(o))
        return o

    def residual(self, o_dense_stored, o_sparse):
        a, b = _f64(o_dense_stored), _f64(o_sparse)
        a, b = np.broadcast_arrays(a, b)
        a, b = _f64(a), _f64(b)
        r = np.empty_like(a)
        self.lib.orc_residual(_p(a), _p(b), a.size, _p(r))
        return r

    def reuse_output(self, q_rows, k, v, idx, r_stored, scale: float):
        q, k, v, idx, r = _f64(q_rows), _f64(k), _f64(v), _i64a(idx), _f64(r_stored)
        o = np.empty((q.shape[0], v.shape[1]))
        self.lib.orc_reuse_output(_p(q), q.shape[0], _p(k), _p(v), q.shape[1], _pi(idx), idx.shape[0], _p(r),
                                  float(scale), _p(o))
        return o

    # ---- selection variants (granularity ablation) ----------------------------
    def block_select(self, A, nblocks: int, block: int):
        """Keys of the `nblocks` full `block`-key blocks of largest summed
        mass (equal mass -> lower block), block by block, ascending."""
        A = _f64(A)
        N = A.shape[0]
        if not 1 <= int(block) <= N or not 1 <= int(nblocks) <= N // int(block):
            raise ValueError("need 1 <= block <= N and 1 <= nblocks <= N // block")
        idx = np.empty(int(nblocks) * int(block), dtype=np.int64)
        self.lib.orc_block_select(_p(A), N, int(block), int(nblocks), _pi(idx))
        return idx

    def group_recall(self, A, idx, n_rows: int) -> float:
        """Mean over the group's rows of the probability mass of the selected keys."""
        A, idx = _f64(A), _i64a(idx)
        if idx.size and (idx.min() < 0 or idx.max() >= A.shape[0]):
            raise ValueError("key index out of range")
        return float(self.lib.orc_group_recall(_p(A), _pi(idx), idx.shape[0], int(n_rows)))

    def rel_l1(self, x, ref) -> float:
        """sum |x - ref| / sum |ref|."""
        x, ref = _f64(x), _f64(ref)
        if x.shape != ref.shape:
            raise ValueError("x and ref must have one shape")
        return float(self.lib.orc_rel_l1(_p(x), _p(ref), x.size))

    # ---- whole-head drivers (std::thread over the head's groups) -------------
    def reuse_head(self, q, k, v, perm, group_size: int, idx, r, scale: float, groups=None):
        """Reuse output of one head: q, k, v, r [N, d] by token, perm [N].
        ``groups`` lists the group ids to compute (all by default) and idx
        holds one index row per listed group; rows of other groups stay 0."""
        q, k, v, r, perm, idx = _f64(q), _f64(k), _f64(v), _f64(r), _i64a(perm), _i64a(idx)
        N, d = q.shape
        T = int(group_size)
        G = -(-N // T)
        gids = np.arange(G, dtype=np.int64) if groups is None else _i64a(groups)
        if k.shape != (N, d) or v.shape != (N, d) or r.shape != (N, d) or perm.shape != (N,):
            raise ValueError("q, k, v, r must be [N, d] and perm [N]")
        if idx.ndim != 2 or idx.shape[0] != gids.shape[0] or not 1 <= idx.shape[1] <= N:
            raise ValueError("idx needs one row of 1..N indices per listed group")
        if gids.size and (gids.min() < 0 or gids.max() >= G) or idx.size and (idx.min() < 0 or idx.max() >= N):
            raise ValueError("group id or key index out of range")
        out = np.zeros((N, d))
        self.lib.orc_reuse_head(_p(q), _p(k), _p(v), N, d, _pi(perm), T, _pi(gids), gids.shape[0], _pi(idx),
                                idx.shape[1], _p(r), float(scale), self.threads, _p(out))
        return out

    def anchor_head(self, q, k, v, perm, group_size: int, topk: int, scale: float, with_mass: bool = False):
        """Anchor step of one head on the given groups: O_dense (bf16-stored),
        LSE, per-group top-K indices (and mass rows) and R, all by token."""
        q, k, v, perm = _f64(q), _f64(k), _f64(v), _i64a(perm)
        N, d = q.shape
        G = -(-N // group_size)
        if k.shape != (N, d) or v.shape != (N, d) or perm.shape != (N,) or not 1 <= int(topk) <= N:
            raise ValueError("q, k, v must be [N, d], perm [N] and topk in [1, N]")
        od, L, r = np.empty((N, d)), np.empty(N), np.empty((N, d))
        idx = np.empty((G, int(topk)), dtype=np.int64)
        mass = np.empty((G, N)) if with_mass else None
        self.lib.orc_anchor_head(_p(q), _p(k), _p(v), N, d, _pi(perm), int(group_size), int(topk), float(scale),
                                 self.threads, _p(od), _p(L), _pi(idx), _p(mass) if with_mass else None, _p(r))
        out = {"o_dense": od, "lse": L, "idx": idx, "r": r}
        if with_mass:
            out["mass"] = mass
        return out


_default = None


def default() -> CppOracle:
    global _default
    if _default is None:
        _default = CppOracle()
    return _default
