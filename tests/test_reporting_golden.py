"""The reporting formulas reproduce the relations printed in the pages' tables."""
import json
import os

import pytest

from sparse_attention_diffusion_pddp_amd import metrics

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_table6_eta_is_rho_times_density():
    t = load("table6_kernel_speedup.json")
    n = 0
    for row in t["rows"].values():
        for s, rho, eta in zip(t["densities"], row["rho"], row["eta"]):
            # rho = t_dense / t_sparse; feed a time pair with that ratio
            r, e = metrics.kernel_speedup(rho * 10.0, 10.0, s)
            assert r == pytest.approx(rho)
            assert round(e + 1e-9, 2) == eta
            n += 1
    assert n == 12


def test_table7_amortisation():
    t = load("table7_grouping_latency.json")
    for row in t["fast_pddp"].values():
        assert round(metrics.amortized_grouping_ms(row["single"], 2, t["steps"]) + 1e-9, 2) == row["amortized"]
    for row in t["flash_kmeans"].values():
        a = metrics.amortized_kmeans_ms(row["init"], row["update"], t["steps"])
        assert abs(a - row["amortized"]) <= 0.01


def test_table8_c_over_v_needs_mib():
    t = load("table8_offload.json")
    for row in t["rows"].values():
        cv = metrics.offload_ratio(row["C_tflop"], row["V"])
        # printed C/V within the rounding of C (3 significant digits)
        assert abs(cv - row["C_over_V"]) / row["C_over_V"] < 0.002
        # decimal megabytes would be ~4.9% off
        assert abs(row["C_tflop"] * 1e12 / (row["V"] * 1e6) - row["C_over_V"]) / row["C_over_V"] > 0.04
        assert row["hidden"] == (row["transfer_ms"] < row["compute_ms"])


def test_work_counts():
    assert metrics.sparse_flops(1, 12, 32760, 4914, 128) == 989_077_340_160
    assert metrics.dense_flops(1, 40, 75600, 128) == 117_050_572_800_000
    assert abs(metrics.align_ratio(32760, 128, 4914, 64) - 1.0032) < 1e-3
    assert metrics.align_ratio(1024, 64, 256, 64) == 1.0


def test_recall_and_rel_l1_formulas_match_the_oracle():
    """metrics.group_recall / rel_l1 (torch reductions used by the variant
    diagnostics) against the oracle's definitions, on the CPU."""
    import numpy as np
    import torch

    import oracle as O
    from sparse_attention_diffusion_pddp_amd import metrics
    rng = np.random.default_rng(40)
    A = rng.random((3, 7, 300))
    idx = np.sort(np.stack([np.stack([rng.choice(300, 45, replace=False) for _ in range(7)]) for _ in range(3)]), -1)
    rows = torch.tensor([128.0] * 6 + [44.0])
    got = metrics.group_recall(torch.from_numpy(A), torch.from_numpy(idx), rows).numpy()
    for h in range(3):
        for g in range(7):
            assert abs(got[h, g] - O.group_recall(A[h, g], idx[h, g], int(rows[g]))) < 1e-14
    x, ref = rng.standard_normal((50, 9)), rng.standard_normal((50, 9))
    assert abs(metrics.rel_l1(torch.from_numpy(x), torch.from_numpy(ref)) - O.rel_l1(x, ref)) < 1e-14
    assert metrics.matched_blocks(4914, 64) == 77 and metrics.matched_blocks(8190, 64) == 128
    assert metrics.matched_blocks(10, 64) == 1 and metrics.matched_blocks(96, 64) == 2


def test_pddp_work_counts():
    """Tree depth and the grouping's algorithmic bytes and float64 FLOPs,
    against hand counts."""
    from sparse_attention_diffusion_pddp_amd import metrics
    assert metrics.pddp_levels(32760, 128) == 8      # 256 groups
    assert metrics.pddp_levels(98304, 128) == 10     # 768 groups: 3 x 2^8
    assert metrics.pddp_levels(64000, 128) == 9      # 500 groups
    assert metrics.pddp_levels(128, 128) == 0 and metrics.pddp_levels(129, 128) == 1
    assert metrics.pddp_algorithmic_bytes(1, 1, 300, 64, 128) == 2 * 300 * 64 * 2 + 300 * 4  # 3 groups: 2 levels
    # N = 300, d = 32, T = 128: levels 2, groups 3 (2 split nodes); 3 tiles of 16 x 16 per token;
    # accumulated tokens 300 + 150 = 450
    want = 2 * (450 * 3 * 256 + 2 * 16 * 32 * 32 + 2 * 300 * 32)
    assert metrics.pddp_fp64_flops(1, 1, 300, 32, 128) == want
