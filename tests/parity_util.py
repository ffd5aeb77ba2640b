"""Comparison helpers shared by the GPU parity tests (no method arithmetic)."""
import numpy as np
import torch

# float tolerance on bf16 outputs with fp32 accumulation
MAX_ABS = 2e-2
REL_L2 = 5e-3
LSE_ABS = 1e-3
# selected sets may differ only by swapping keys whose exact masses differ by less than this
MASS_GAP = 1e-6


def head_np(t: torch.Tensor, b: int, h: int) -> np.ndarray:
    """One head of a CPU [B, N, H, d] tensor as float64 (exact widening)."""
    return t[b, :, h, :].float().numpy().astype(np.float64)


def bf16_tensor(x: np.ndarray) -> torch.Tensor:
    """float64 values already on the bf16 grid -> bf16 tensor (exact)."""
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)


def float_report(got, want, denom=None):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = got - want
    d = want if denom is None else np.asarray(denom, dtype=np.float64)
    return float(np.abs(err).max()), float(np.linalg.norm(err) / max(np.linalg.norm(d), 1e-300))


def assert_close(got, want, name, denom=None, max_abs=MAX_ABS, rel_l2=REL_L2):
    ma, rl = float_report(got, want, denom)
    assert ma <= max_abs and rl <= rel_l2, f"{name}: max-abs {ma:.3e} (<= {max_abs}), rel-L2 {rl:.3e} (<= {rel_l2})"
    return ma, rl


def assert_close_residual(got, want_r, o_dense, name):
    """R is a difference: near zero at high density, larger than O at very low
    density. Its rel-L2 denominator is the larger of ||R|| and ||O_dense||."""
    want_r = np.asarray(want_r, dtype=np.float64)
    o_dense = np.asarray(o_dense, dtype=np.float64)
    denom = want_r if np.linalg.norm(want_r) >= np.linalg.norm(o_dense) else o_dense
    return assert_close(got, want_r, name, denom=denom)


def assert_close_chained_reuse(got, want, r, name):
    """Reuse output of a chained pipeline (each side fed its own R): R is
    stored in bf16, so when |R| exceeds |O_t| (very low density) one bf16
    step of R -- which the two sides may round differently, since their
    O_dense differ by rounding -- lands in O_t. The rel-L2 denominator is the
    larger of ||O_t|| and ||R||; max-abs stays absolute."""
    want = np.asarray(want, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    denom = want if np.linalg.norm(want) >= np.linalg.norm(r) else r
    return assert_close(got, want, name, denom=denom)


def audit_topk(got, want, mass, K, N, name=""):
    """GPU index row vs the oracle's: valid (ascending, unique, in range, K of
    them) and equal as a set except for swaps across the cut whose oracle
    masses differ by less than MASS_GAP. Returns the number of swaps."""
    got = np.asarray(got, dtype=np.int64)
    want = np.asarray(want, dtype=np.int64)
    assert got.shape == (K,), name
    assert np.all(np.diff(got) > 0), f"{name}: not strictly ascending"
    assert got[0] >= 0 and got[-1] < N, f"{name}: out of range"
    extra = np.setdiff1d(got, want)
    missing = np.setdiff1d(want, got)
    assert len(extra) == len(missing)
    if len(extra):
        gap = mass[missing].max() - mass[extra].min()
        assert gap < MASS_GAP, f"{name}: {len(extra)} swaps, mass gap {gap:.3e} >= {MASS_GAP}"
    return len(extra)
