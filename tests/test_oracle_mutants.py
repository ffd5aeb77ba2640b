"""Planted mistakes in the oracle must fail its pins.

numpy oracle: each case swaps one function for a copy with a plausible slip
(a dropped term, a wrong sign, a transposed operand, an off-by-one count, the
wrong tie rule) and runs the pin that should catch it.

C++ oracle: the same kinds of slip are compiled into copies of the library
(ORC_MUTANT = 1..14 in mcsparse_oracle.cpp, one slip each), and each copy
must fail its pin. Everything runs on the CPU and touches only the oracle.
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


def _pddp_larger_half_left(q, group_size, power_iters=16, whiten=False):
    T = int(group_size)
    out, stack = [], [np.arange(q.shape[0], dtype=np.int64)]
    while stack:
        members = stack.pop()
        G = -(-members.shape[0] // T)
        if G <= 1:
            out.append(np.sort(members))
            continue
        left, right = ref._split_node(q, members, ((G + 1) // 2) * T, power_iters)  # ceil instead of floor
        stack.append(right)
        stack.append(left)
    return np.concatenate(out)


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


def _blocks_with_partial(A, nblocks, block):
    N = A.shape[0]
    nb_all = -(-N // block)
    pad = np.concatenate([A, np.zeros(nb_all * block - N)])
    bm = pad.reshape(nb_all, block).sum(axis=1)  # the short last block competes
    chosen = np.sort(np.lexsort((np.arange(nb_all), -bm))[:nblocks])
    return np.minimum((chosen[:, None] * block + np.arange(block)).reshape(-1), N - 1)


def _recall_over_keys(A, idx, n_rows):
    return float(A[idx].sum() / len(idx))


MUTANTS = [
    ("dense_lse", _dense_no_scale, pins.test_dense_lse_matches_torch_sdpa_and_scipy_logsumexp),
    ("dense_lse", _dense_transposed, pins.test_dense_lse_decimal_bruteforce),
    ("dense_lse", _dense_lse_without_max, pins.test_dense_single_key_and_zero_keys),
    ("group_mass", _mass_wrong_sign, pins.test_group_mass_decimal_bruteforce_and_row_sums),
    ("topk_select", _topk_high_index_ties, pins.test_topk_tie_rule_and_extremes),
    ("residual", _residual_flipped, pins.test_residual_closed_form_and_anchor_identity),
    ("principal_direction", _pd_15, pins.test_principal_direction_closed_form_iteration_count),
    ("principal_direction", _pd_no_orientation, pins.test_pddp_rank_one_reduces_to_argsort_chunks),
    ("pddp_group", _pddp_larger_half_left, pins.test_pddp_odd_node_splits_at_floor_half),
    ("sparse_attention", _sparse_unnormalised, pins.test_sparse_decimal_bruteforce),
    ("standardize", _std_unscaled, pins.test_whitened_pddp_root_split_follows_the_correlation_eigenvector),
    ("standardize", _std_by_variance, pins.test_whitened_pddp_root_split_follows_the_correlation_eigenvector),
    ("standardize", _std_times_sd, pins.test_standardize_closed_form_and_constant_dims),
    ("block_select", _blocks_with_partial, pins.test_block_select_bruteforce_ties_and_partial_block),
    ("group_recall", _recall_over_keys, pins.test_group_recall_closed_forms),
]


@pytest.mark.parametrize("name,mutant,pin", MUTANTS, ids=[f"{m[0]}-{m[1].__name__}" for m in MUTANTS])
def test_pin_catches_planted_mistake(monkeypatch, name, mutant, pin):
    monkeypatch.setitem(ref.__dict__, f"_orig_{name}", getattr(ref, name))
    monkeypatch.setattr(ref, name, mutant)
    monkeypatch.setattr(oracle, name, mutant)
    with pytest.raises(AssertionError):
        pin(ref)


def test_pins_pass_unmutated():
    for _, _, pin in MUTANTS:
        pin(ref)
    assert math.isfinite(1.0)


# ORC_MUTANT id -> the pin that must catch it
CPP_MUTANTS = {
    1: pins.test_dense_lse_matches_torch_sdpa_and_scipy_logsumexp,   # scale dropped
    2: pins.test_dense_single_key_and_zero_keys,                     # LSE without its max term
    3: pins.test_dense_lse_decimal_bruteforce,                       # values paired with the wrong keys
    4: pins.test_group_mass_decimal_bruteforce_and_row_sums,         # +L instead of -L
    5: pins.test_topk_tie_rule_and_extremes,                         # ties to the higher index
    6: pins.test_sparse_decimal_bruteforce,                          # softmax not renormalised
    7: pins.test_principal_direction_closed_form_iteration_count,    # one power iteration short
    8: pins.test_pddp_rank_one_reduces_to_argsort_chunks,            # orientation reversed
    9: pins.test_pddp_odd_node_splits_at_floor_half,                 # ceil(G/2) tiles left
    10: pins.test_whitened_pddp_root_split_follows_the_correlation_eigenvector,  # never scaled
    11: pins.test_residual_closed_form_and_anchor_identity,          # sparse - dense
    12: pins.test_round_bf16_matches_torch_rne,                      # truncation
    13: pins.test_block_select_bruteforce_ties_and_partial_block,    # the short last block competes
    14: pins.test_group_recall_closed_forms,                         # divided by the key count
}


@pytest.fixture(scope="module")
def cpp_mutants(tmp_path_factory):
    from oracle import build
    from oracle.cpp import CppOracle
    d = tmp_path_factory.mktemp("oracle_mutants")
    return {m: CppOracle(build.build(mutant=m, out=str(d / f"mutant{m}.so"), verbose=False)) for m in CPP_MUTANTS}


@pytest.mark.parametrize("m", sorted(CPP_MUTANTS))
def test_cpp_pin_catches_planted_mistake(cpp_mutants, m):
    o = cpp_mutants[m]
    assert o.mutant == m
    with pytest.raises(AssertionError):
        CPP_MUTANTS[m](o)


def test_cpp_pins_pass_unmutated():
    from oracle import cpp
    o = cpp.default()
    assert o.mutant == 0
    for pin in set(CPP_MUTANTS.values()):
        pin(o)
