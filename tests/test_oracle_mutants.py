"""Planted mistakes in the oracle must fail its pins.

Each case swaps one oracle function for a copy with a plausible slip (a
dropped term, a wrong sign, a transposed operand, an off-by-one count, the
wrong tie rule) and runs the pin that should catch it. Everything runs on the
CPU and touches only the oracle.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.mcsparse_ref as ref
from tests import test_oracle_pins as pins


def _dense_no_scale(q_rows, k, v, scale):
    return ref.__dict__["_orig_dense_lse"](q_rows, k, v, 1.0)


def _dense_transposed(q_rows, k, v, scale):
    s = scale * (q_rows @ k.T)
    m = s.max(axis=1, keepdims=True)
    L = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
    P = np.exp(s - L[:, None])
    return P @ v[::-1], L  # values paired with the wrong keys


def _dense_lse_without_max(q_rows, k, v, scale):
    o, L = ref.__dict__["_orig_dense_lse"](q_rows, k, v, scale)
    return o, L - (scale * (q_rows @ k.T)).max(axis=1)  # dropped m_i term


def _mass_wrong_sign(q_group, k, lse_group, scale):
    s = scale * (q_group @ k.T)
    return np.exp(s + lse_group[:, None]).sum(axis=0)


def _topk_high_index_ties(A, K):
    j = np.arange(A.shape[0])
    order = np.lexsort((-j, -A))
    return np.sort(order[:K])


def _residual_flipped(o_dense_stored, o_sparse):
    return ref.round_bf16(o_sparse - o_dense_stored)


def _pd_15(C, power_iters=16, start=None):
    return ref.__dict__["_orig_principal_direction"](C, 15, start)


def _pd_no_orientation(C, power_iters=16, start=None):
    u = ref.__dict__["_orig_principal_direction"](C, power_iters, start)
    return -u


def _sparse_unnormalised(q_rows, k, v, idx, scale):
    ks, vs = k[idx], v[idx]
    s = scale * (q_rows @ ks.T)
    return np.exp(s - s.max(axis=1, keepdims=True)) @ vs


def _std_unscaled(q):
    Xc, var = ref.__dict__["_orig_standardize"](q)
    return q - q.sum(axis=0) / q.shape[0], var  # centred, never scaled


def _std_by_variance(q):
    N = q.shape[0]
    Xc = q - q.sum(axis=0) / N
    var = (Xc * Xc).sum(axis=0) / N
    return Xc / np.where(var > 0, var, 1.0), var  # 1/var instead of 1/sd


def _std_times_sd(q):
    N = q.shape[0]
    Xc = q - q.sum(axis=0) / N
    var = (Xc * Xc).sum(axis=0) / N
    return Xc * np.sqrt(var), var  # inverted scale


MUTANTS = [
    ("dense_lse", _dense_no_scale, pins.test_dense_lse_matches_torch_sdpa_and_scipy_logsumexp),
    ("dense_lse", _dense_transposed, pins.test_dense_lse_decimal_bruteforce),
    ("dense_lse", _dense_lse_without_max, pins.test_dense_single_key_and_zero_keys),
    ("group_mass", _mass_wrong_sign, pins.test_group_mass_decimal_bruteforce_and_row_sums),
    ("topk_select", _topk_high_index_ties, pins.test_topk_tie_rule_and_extremes),
    ("residual", _residual_flipped, pins.test_residual_closed_form_and_anchor_identity),
    ("principal_direction", _pd_15, pins.test_principal_direction_closed_form_iteration_count),
    ("principal_direction", _pd_no_orientation, pins.test_pddp_rank_one_reduces_to_argsort_chunks),
    ("sparse_attention", _sparse_unnormalised, pins.test_sparse_decimal_bruteforce),
    ("standardize", _std_unscaled, pins.test_whitened_pddp_root_split_follows_the_correlation_eigenvector),
    ("standardize", _std_by_variance, pins.test_whitened_pddp_root_split_follows_the_correlation_eigenvector),
    ("standardize", _std_times_sd, pins.test_standardize_closed_form_and_constant_dims),
]


@pytest.mark.parametrize("name,mutant,pin", MUTANTS, ids=[f"{m[0]}-{m[1].__name__}" for m in MUTANTS])
def test_pin_catches_planted_mistake(monkeypatch, name, mutant, pin):
    monkeypatch.setitem(ref.__dict__, f"_orig_{name}", getattr(ref, name))
    monkeypatch.setattr(ref, name, mutant)
    monkeypatch.setattr(oracle, name, mutant)
    with pytest.raises(AssertionError):
        pin()


def test_pins_pass_unmutated():
    for _, _, pin in MUTANTS:
        pin()
    assert math.isfinite(1.0)
