"""bench.py's host-side logic, on the CPU: the one-GPU refusal, the traffic
summary arithmetic from rocprofv3 counter CSVs, and the activation sets of
the layer-stack schedules."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_write_traffic_scales_by_the_copy(tmp_path, monkeypatch):
    k = "void mcs::attention_kernel<128, 4, 1>(mcs::AttnArgs)"
    other = "void mcs::attention_kernel<128, 4, 0>(mcs::AttnArgs)"
    copy = "__amd_rocclr_copyBuffer"
    _counters(tmp_path / "f", [{"Kernel_Name": k, "Counter_Name": "FETCH_SIZE", "Counter_Value": 1000.0},
                               {"Kernel_Name": k, "Counter_Name": "FETCH_SIZE", "Counter_Value": 3000.0},
                               {"Kernel_Name": other, "Counter_Name": "FETCH_SIZE", "Counter_Value": 9e9}])
    _counters(tmp_path / "w", [{"Kernel_Name": k, "Counter_Name": "WRITE_SIZE", "Counter_Value": 500.0}])
    # a 1 GiB copy read back as half its size and written in full
    _counters(tmp_path / "fc", [{"Kernel_Name": copy, "Counter_Name": "FETCH_SIZE", "Counter_Value": 524288.0}])
    _counters(tmp_path / "wc", [{"Kernel_Name": copy, "Counter_Name": "WRITE_SIZE", "Counter_Value": 1048576.0}])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    bench.write_traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "fc"), str(tmp_path / "wc"))
    t = json.loads(out.read_text())
    assert t["fetch_kib_per_launch"] == 2000.0 and t["write_kib_per_launch"] == 500.0
    assert t["fetch_scale"] == 2.0 and t["write_scale"] == 1.0
    assert t["bytes_per_launch"] == (2000 * 2 + 500) * 1024
    assert t["kernel_hash"] == bench.kernel_hash()
    # reported only for a launch of the counted work (wan480p at 15%)
    assert t["workload"] == "wan480p" and t["per_launch_flop"] == 989077340160
    assert t["head_dim"] == 128 and t["group_size"] == 128
    assert bench.load_traffic(989077340160, 128, 128) == (2000 * 2 + 500) * 1024
    assert bench.load_traffic(17812571553792, 128, 128) is None  # longvideo's reuse call
    # the same work in 64-row groups runs another kernel instance
    assert bench.load_traffic(989077340160, 128, 64) is None


def test_committed_traffic_is_ignored_once_the_kernel_changes(monkeypatch):
    assert bench.load_traffic(989077340160, 128, 128) is not None
    monkeypatch.setattr(bench, "kernel_hash", lambda: "not-the-hash")
    assert bench.load_traffic(989077340160, 128, 128) is None


def test_kernel_hash_ignores_comments_only():
    """Comments and layout do not count as a kernel change; code, strings
    holding comment markers, and character literals do."""
    a = "int f(int x) {\n  return x + 1;  // one more\n}\n"
    b = "/* header */\nint f(int x) {\n    return x + 1;\n}  // end\n"
    c = "int f(int x) {\n  return x + 2;\n}\n"
    assert bench.strip_comments(a) == bench.strip_comments(b) == "int f(int x) { return x + 1; }"
    assert bench.strip_comments(a) != bench.strip_comments(c)
    s = 'const char *p = "a // b /* c */"; char q = \'"\'; // x'
    assert bench.strip_comments(s) == 'const char *p = "a // b /* c */"; char q = \'"\';'


@pytest.mark.parametrize("anchors,expect", [
    ((1,), {1: 0, 2: 1, 12: 1}),
    ((10, 26), {1: 0, 10: 0, 11: 1, 25: 1, 26: 2, 27: 3, 50: 3}),
])
def test_schedule_input_sets(anchors, expect):
    for step, k in expect.items():
        assert bench.input_set(step, anchors) == k, step


def test_cpu_baseline_times_the_cpp_oracle():
    """The baseline leg runs the C++ oracle's reuse driver on a bounded
    sample and reports its worker count as cores."""
    from oracle import cpp
    from sparse_attention_diffusion_pddp_amd import synth
    w = synth.small_workload(1200, heads=2, head_dim=64, group_size=128, density_pct=10)
    out = bench.cpu_baseline(w, 0.2, seed=3, n_groups=4)
    assert out["kind"] == "oracle" and out["unit"] == "TFLOP/s"
    assert out["cores"] == cpp.default().threads >= 1
    assert out["value"] > 0 and "first 4 query groups of head 0" in out["sample"]
    assert "C++ float64 oracle" in out["sample"]
