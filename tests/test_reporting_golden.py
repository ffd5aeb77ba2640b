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
