#!/usr/bin/env python
"""Benchmark of the MC-Sparse hot path on one MI355X.

One step = one anchor step (PDDP grouping, dense attention + LSE, exact
top-K selection, residual) followed by the workload's reuse steps (sparse
attention over the cached indices with freshly drifted Q/K/V, plus R), for
one attention layer with all heads, on synthetic inputs already resident in
HBM. Default workload: the Wan2.1-1.3B 480p shape (12 heads, N = 32760,
d = 128, groups of 128, 15% density, 4 reuse steps).

value: effective TFLOP/s of the reuse step, 4*B*H*N*K*d FLOPs per call
(only selected keys, nominal rows) over the measured call time. The anchor
step's milliseconds (per stage and total) are reported beside it.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "reuse-step sparse attn eff. TFLOP/s @15% density + anchor-step ms (1 GPU)"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
PEAK_FP64_TFLOPS = 78.6  # MI355X float64 (matrix and vector)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sparse_apply_wan480p_traffic.json")
KERNEL_SOURCES = ["mcs_attention.hip", "mcs_common.hpp", "mcs_lds.hpp"]


def strip_comments(src: str) -> str:
    """C++ source without its comments and with runs of whitespace made one
    space, so that edits to comments alone keep the hash; string and
    character literals are kept as they are."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_hash() -> str:
    """Hash of the sparse-apply kernel's code (comments left out)."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "sparse_attention_diffusion_pddp_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(strip_comments(fh.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(per_launch_flops, head_dim, group_size):
    """HBM bytes per sparse_apply launch from committed rocprofv3 counters,
    if they were taken on the current kernel source, on the same kernel
    instance (head dim and group size) and on a launch of the same work (the
    counted workload's effective FLOPs)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_hash() or t.get("per_launch_flop") != per_launch_flops:
        return None
    if t.get("head_dim") != head_dim or t.get("group_size") != group_size:
        return None
    return t.get("bytes_per_launch")


def write_traffic(fetch_dir, write_dir, fetch_copy_dir, write_copy_dir, kernel="attention_kernel<128, 4, 1>"):
    """Turns four rocprofv3 --pmc runs (FETCH_SIZE / WRITE_SIZE of this bench
    with --steps 1 --warmup 0, and of --copy-calibration) into the traffic
    file read above: KiB per dispatch of `kernel`, each counter scaled by
    what it reads for a plain 1 GiB device copy. Needs no GPU."""
    import collections
    import csv
    import glob

    def per_dispatch(d, counter, match):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        vals = collections.defaultdict(list)
        for f in files:
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if r["Counter_Name"] == counter and match in r["Kernel_Name"]:
                        vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        if len(vals) != 1:
            raise SystemExit(f"{counter} in {d}: expected one kernel matching {match!r}, found {sorted(vals)}")
        v = next(iter(vals.values()))
        return sum(v) / len(v), len(v)

    copy_kib = (1 << 30) / 1024
    fetch, n_f = per_dispatch(fetch_dir, "FETCH_SIZE", kernel)
    write, n_w = per_dispatch(write_dir, "WRITE_SIZE", kernel)
    fetch_c, _ = per_dispatch(fetch_copy_dir, "FETCH_SIZE", "copyBuffer")
    write_c, _ = per_dispatch(write_copy_dir, "WRITE_SIZE", "copyBuffer")
    fs, ws = copy_kib / fetch_c, copy_kib / write_c
    from sparse_attention_diffusion_pddp_amd import metrics, synth
    w = synth.WORKLOADS["wan480p"]  # the workload of the counted bench runs
    m = re.match(r"attention_kernel<(\d+), (\d+), 1>", kernel)
    if not m:
        raise SystemExit(f"not a sparse-apply kernel instance: {kernel!r}")
    out = {"kernel": f"{kernel} (mcs_sparse_apply), wan480p 15%", "kernel_hash": kernel_hash(),
           "head_dim": int(m.group(1)), "group_size": 32 * int(m.group(2)),
           "workload": "wan480p", "per_launch_flop": metrics.sparse_flops(w.batch, w.heads, w.seqlen, w.topk, w.head_dim),
           "dispatches": {"fetch": n_f, "write": n_w},
           "fetch_kib_per_launch": round(fetch, 1), "write_kib_per_launch": round(write, 1),
           "copy_calibration_kib": {"bytes_copied_kib": copy_kib, "fetch_kib": round(fetch_c, 1),
                                    "write_kib": round(write_c, 1)},
           "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
           "bytes_per_launch": int(round((fetch * fs + write * ws) * 1024))}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def gemm_reference(n: int = 16384, reps: int = 4) -> dict:
    """What a large dense bf16 GEMM from the platform library (torch.matmul,
    hipBLASLt) sustains on this GPU, warm: a practical MFMA ceiling beside the
    datasheet peak. Both operands are plain contiguous 2-D tensors."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    a = torch.randn(n, n, device="cuda", generator=g).to(torch.bfloat16).contiguous()
    b = torch.randn(n, n, device="cuda", generator=g).to(torch.bfloat16).contiguous()
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b, c
    return {"tflops": round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1), "ms": round(ms, 4), "shape": [n, n, n],
            "lib": "torch.matmul bf16 (hipBLASLt), warm"}


def cpu_baseline(w, seconds: float, seed: int, n_groups: int = 64):
    """The oracle, untuned, timed on the host on a bounded sample of the reuse
    step: the first ``n_groups`` query groups of head 0, through the C++
    oracle's head driver (std::thread over the groups; its thread count is
    ``cores``). The anchor metadata of those groups (PDDP groups, top-K
    indices, R) is prepared first, untimed."""
    import numpy as np

    import oracle as O
    import oracle.mcsparse_ref as ref
    from oracle import cpp
    from sparse_attention_diffusion_pddp_amd import synth

    T, K, d = w.group_size, w.topk, w.head_dim
    scale = 1.0 / math.sqrt(d)
    q, k, v = synth.make_qkv(w, seed=seed, heads=[0])
    qt, kt, vt = synth.drift_qkv(w, (q, k, v), step=1, seed=seed, heads=[0])
    hq, hk, hv, hqt, hkt, hvt = (t[0, :, 0].float().numpy().astype(np.float64) for t in (q, k, v, qt, kt, vt))
    perm = O.pddp_group(hq, T)
    groups = np.arange(min(n_groups, w.groups))
    idx = np.zeros((len(groups), K), dtype=np.int64)
    r = np.zeros_like(hq)
    # untimed preparation; the numpy transcription's library matmul keeps it short
    for e, g in enumerate(groups):
        rows = perm[g * T:(g + 1) * T]
        od, L = ref.dense_lse(hq[rows], hk, hv, scale)
        idx[e] = O.topk_select(O.group_mass(hq[rows], hk, L, scale), K)
        r[rows] = O.residual(O.round_bf16(od), O.sparse_attention(hq[rows], hk, hv, idx[e], scale))
    oracle = cpp.default()
    rows_done = sum(min(T, w.seqlen - g * T) for g in groups)
    elapsed, flops, passes = 0.0, 0, 0
    while elapsed < seconds:
        t0 = time.perf_counter()
        oracle.reuse_head(hqt, hkt, hvt, perm, T, idx, r, scale, groups=groups)
        elapsed += time.perf_counter() - t0
        flops += 4 * rows_done * K * d
        passes += 1
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": oracle.threads, "kind": "oracle",
            "sample": f"reuse step of {w.name}: the first {len(groups)} query groups of head 0 "
                      f"(of {w.groups * w.heads} groups in the layer), {passes} passes, {elapsed:.1f} s of "
                      f"oracle time; C++ float64 oracle on {oracle.threads} std::thread workers"}


def input_set(step, anchors):
    """Which activation set a denoising step uses (see schedule_inputs):
    0 up to the first anchor, then one drifted set between anchors and one at
    each later anchor."""
    anchors = sorted(anchors)
    if step <= anchors[0]:
        return 0
    n = sum(1 for a in anchors if a <= step)
    return 2 * n - 2 if step in anchors else 2 * n - 1


def schedule_inputs(w, sched, seed):
    """Activations for a layer-stack run: the first anchor's Q/K/V (also used
    by the dense warm-up steps before it), then one drifted set between
    anchors and one at each later anchor. The cost of a call does not depend
    on the values; the drift keeps each anchor's metadata its own."""
    from sparse_attention_diffusion_pddp_amd import synth

    anchors = sorted(sched.anchor_steps)
    sets = [synth.make_qkv(w, seed=seed)]
    for i in range(1, 2 * len(anchors)):
        sets.append(synth.drift_qkv(w, sets[-1], step=i, seed=seed))
    dev = [tuple(t.cuda() for t in x) for x in sets]
    return (lambda step, layer: dev[input_set(step, anchors)]), dev


def run_schedule(args, w, sched, offload=True, offload_idx=False):
    """A whole layer stack over all denoising steps through StackRunner
    (appendix Table 9 schedules): dense warm-up steps and always-dense
    layers, anchors that (re)build groups, indices and R, reuse layers in
    between; R offloaded to pinned host memory and prefetched one layer
    ahead on a side stream (Table 8's per-layer accounting)."""
    import torch

    from sparse_attention_diffusion_pddp_amd import binding as mcs
    from sparse_attention_diffusion_pddp_amd import metrics, schedule

    mcs.load()
    torch.cuda.set_device(0)
    B, H, N, d, T, K = w.batch, w.heads, w.seqlen, w.head_dim, w.group_size, w.topk
    inputs, dev = schedule_inputs(w, sched, args.seed)
    runner = schedule.StackRunner(sched, dev[0][0].shape, T, K, offload=offload, offload_idx=offload_idx)
    runner.run(inputs)  # warm-up pass of the whole schedule
    torch.cuda.synchronize()
    ev = {}
    t0 = time.perf_counter()
    runner.run(inputs, events=ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the bare H2D copy of one layer's offloaded bytes from pinned memory,
    # nothing else running
    bm_bytes = runner.bm_bytes if offload_idx else 0
    moved = runner.r_bytes + bm_bytes
    host = torch.empty(moved, dtype=torch.uint8, pin_memory=True)
    devbuf = torch.empty(moved, dtype=torch.uint8, device="cuda")
    e = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    devbuf.copy_(host, non_blocking=True)
    e[0].record()
    for i in range(5):
        devbuf.copy_(host, non_blocking=True)
        e[i + 1].record()
    torch.cuda.synchronize()
    h2d_ms = e[0].elapsed_time(e[5]) / 5
    runner.close()

    def avg(kind):
        xs = [a.elapsed_time(b) for a, b in ev.get(kind, [])]
        return (sum(xs) / len(xs) if xs else 0.0), len(xs)

    reuse_ms, n_reuse = avg("reuse")
    decode_ms, _ = avg("decode")
    pf_ms, n_pf = avg("prefetch")
    anchor_ms, n_anchor = avg("anchor")
    pddp_ms, _ = avg("pddp")
    dense_ms, n_dense = avg("dense")
    step_ms = [a.elapsed_time(b) for a, b in ev["step"]]
    plan = schedule.plan(sched)
    kinds = {st: {a for s2, _, a in plan if s2 == st} for st in range(1, sched.steps + 1)}
    anchor_steps = sorted(sched.anchor_steps)
    reuse_steps = [st for st in range(1, sched.steps + 1) if kinds[st] == {schedule.DENSE, schedule.REUSE}]
    warm_steps = [st for st in range(1, sched.steps + 1) if kinds[st] == {schedule.DENSE}]
    step_avg = lambda sts: (sum(step_ms[st - 1] for st in sts) / len(sts)) if sts else 0.0
    flops = metrics.sparse_flops(B, H, N, K, d)
    value = flops / (reuse_ms * 1e-3) / 1e12
    # a reuse step is the dense layers plus the sparse layers' reuse calls;
    # what is left over is time the compute stream spent waiting for prefetches
    n_sparse = len(runner.sparse_layers)
    n_dl = len(sched.dense_layers)
    exposed = (sum(step_ms[st - 1] - n_dl * dense_ms - n_sparse * reuse_ms for st in reuse_steps) / len(reuse_steps)
               if reuse_steps else 0.0)
    all_dense_ms = sched.steps * sched.layers * dense_ms
    r_bytes = runner.r_bytes
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": sched.steps,
        "warmup": 1,
        "ms_per_step": round(wall * 1e3 / sched.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "heads": H, "seqlen": N, "grid": list(w.grid), "head_dim": d,
                   "group_size": T, "density_pct": w.density_pct, "topk": K, "layers": sched.layers,
                   "denoise_steps": sched.steps, "warmup_steps": sched.warmup_steps,
                   "anchor_steps": anchor_steps, "dense_layers": list(sched.dense_layers),
                   "offload": offload, "offload_idx": offload_idx, "seed": args.seed},
        "schedule_counts": {"dense": n_dense, "anchor": n_anchor, "reuse": n_reuse, "prefetch": n_pf,
                            "store": len(ev.get("store", []))},
        "anchor_step_ms": [round(step_ms[st - 1], 3) for st in anchor_steps],
        "anchor_layer_ms": round(anchor_ms, 3),
        "pddp_layer_ms": round(pddp_ms, 3),
        "pddp_ms_amortized_per_step": round(pddp_ms * len(anchor_steps) / max(1, sched.steps - sched.warmup_steps), 4),
        "warmup_step_ms_avg": round(step_avg(warm_steps), 3),
        "reuse_step_ms_avg": round(step_avg(reuse_steps), 3),
        "reuse_layer_ms": round(reuse_ms, 4),
        "dense_layer_ms": round(dense_ms, 3),
        "denoise_ms": round(sum(step_ms), 1),
        "all_dense_denoise_ms": round(all_dense_ms, 1),
        "attention_speedup_vs_all_dense": round(all_dense_ms / sum(step_ms), 3),
        "table8_row": {"V_MB": round(moved / 1e6, 1), "V_MiB": round(moved / 2**20, 1),
                       "R_MB": round(r_bytes / 1e6, 1),
                       "idx_bitmap_MB": round(bm_bytes / 1e6, 1),
                       "idx_int32_MB": round(B * H * runner.G * K * 4 / 1e6, 1),
                       "C_TFLOP": round(flops / 1e12, 3),
                       "C_over_V": round(metrics.offload_ratio(flops / 1e12, moved / 2**20)),
                       "transfer_ms": round(h2d_ms, 3), "transfer_GBps": round(moved / (h2d_ms * 1e-3) / 1e9, 1),
                       "prefetch_span_ms": round(pf_ms, 3),
                       "decode_ms": round(decode_ms, 3),
                       "compute_ms": round(reuse_ms, 3),
                       "exposed_wait_ms_per_reuse_step": round(exposed, 3),
                       "hidden_per_layer": bool(h2d_ms <= reuse_ms),
                       "hidden": bool(exposed <= 0.01 * step_avg(reuse_steps))},
        "roofline": {"bound": "mfma", "achieved": round(value, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(value / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "attention_kernel<128,4,sparse> (mcs_sparse_apply)", "per_launch_flop": flops,
                     "avg_launch_ms": round(reuse_ms, 4)},
    }
    print(json.dumps(out), flush=True)


def run_kernel_only(args, w):
    """Wan14B-720p-shaped layer: the sparse_apply kernel alone on groups and
    indices prepared by the library's own anchor calls (untimed), next to the
    same library's dense attention (paper landing page, Table 6: kernel
    speedup with selection and grouping excluded). Timed with and without
    the +R epilogue; rho / eta use the plain sparse kernel."""
    import torch

    from sparse_attention_diffusion_pddp_amd import binding as mcs
    from sparse_attention_diffusion_pddp_amd import metrics, synth

    mcs.load()
    torch.cuda.set_device(0)
    B, H, N, d, T, K, G = w.batch, w.heads, w.seqlen, w.head_dim, w.group_size, w.topk, w.groups
    q, k, v = (t.cuda() for t in synth.make_qkv(w, seed=args.seed))
    desc = mcs.desc_for(q)
    perm = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    idx = torch.empty((B, H, G, K), dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    r = torch.empty_like(q)
    out = torch.empty_like(q)
    ws = torch.empty(mcs.pddp_workspace_size(desc, T), dtype=torch.uint8, device="cuda")
    mcs.pddp_group(q, T, perm, ws)
    del ws
    mcs.anchor_dense_lse(q, k, v, o, lse)
    ws = torch.empty(mcs.select_workspace_size(desc, T, K), dtype=torch.uint8, device="cuda")
    mcs.anchor_select_topk(q, k, lse, perm, T, K, idx, ws=ws)
    del ws
    mcs.residual(q, k, v, o, perm, T, idx, K, r)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    def timed(fn, n, warm):
        for _ in range(warm):
            fn()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        e[0].record()
        for i in range(n):
            fn()
            e[i + 1].record()
        torch.cuda.synchronize()
        return sum(e[i].elapsed_time(e[i + 1]) for i in range(n)) / n

    t0 = time.perf_counter()
    sparse_r_ms = timed(lambda: mcs.sparse_apply(q, k, v, perm, T, idx, K, r, out), args.steps, args.warmup)
    wall = time.perf_counter() - t0
    sparse_ms = timed(lambda: mcs.sparse_apply(q, k, v, perm, T, idx, K, None, out), args.steps, args.warmup)
    dense_ms = timed(lambda: mcs.anchor_dense_lse(q, k, v, o, None), 3, 1)
    flops = metrics.sparse_flops(B, H, N, K, d)
    value = flops / (sparse_r_ms * 1e-3) / 1e12
    rho, eta = metrics.kernel_speedup(dense_ms, sparse_ms, K / N)
    out_line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "heads": H, "seqlen": N, "grid": list(w.grid), "head_dim": d,
                   "group_size": T, "density_pct": w.density_pct, "topk": K, "kernel_only": True, "seed": args.seed},
        "sparse_apply_ms": round(sparse_r_ms, 4),
        "sparse_kernel_ms": round(sparse_ms, 4),
        "sparse_kernel_tflops": round(flops / (sparse_ms * 1e-3) / 1e12, 2),
        "dense_ms": round(dense_ms, 3),
        "dense_tflops": round(metrics.dense_flops(B, H, N, d) / (dense_ms * 1e-3) / 1e12, 2),
        "speedup_vs_dense": round(rho, 3),
        "eta": round(eta, 3),
        "align": round(metrics.align_ratio(N, T, K, 64), 4),
        "roofline": {"bound": "mfma", "achieved": round(value, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(value / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "attention_kernel<128,4,sparse> (mcs_sparse_apply)", "per_launch_flop": flops,
                     "avg_launch_ms": round(sparse_r_ms, 4)},
    }
    print(json.dumps(out_line), flush=True)


def run_variants(args, w):
    """Selection variants on synthetic data (paper landing page, Tables 3-4):
    query order (PDDP groups, whitened PDDP groups, or consecutive tokens) x
    granularity (single keys vs 64-key blocks) at a matched realised density;
    recall, anchor and reuse errors per variant. The pipeline lives in the
    package (variants.run); this prints its result as one JSON line."""
    import torch

    from sparse_attention_diffusion_pddp_amd import binding as mcs
    from sparse_attention_diffusion_pddp_amd import variants

    mcs.load()
    torch.cuda.set_device(0)
    print(json.dumps(variants.run(w, seed=args.seed)), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="wan480p")
    ap.add_argument("--density", type=int, default=None, help="override the density in percent")
    ap.add_argument("--group-size", type=int, default=None, choices=[64, 128],
                    help="override the query group (tile) size of the default bench")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--offload", choices=["auto", "on", "off"], default="auto",
                    help="layer-stack workloads: R in pinned host memory with one-layer-ahead prefetch "
                         "(auto: on for voxel3d, whose offload the schedule is taken from; off for wanvideo, "
                         "whose 30 layers of R fit in HBM many times over)")
    ap.add_argument("--offload-idx", action="store_true",
                    help="layer-stack workloads with offload: also offload the KV indices, as bitmaps")
    ap.add_argument("--variants", action="store_true",
                    help="selection-variant diagnostics (query order x granularity) instead of the bench line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (scales the rocprofv3 byte counters)")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH", "WRITE", "FETCH_COPY", "WRITE_COPY"),
                    help="summarise four rocprofv3 --pmc output folders into the committed traffic file")
    args = ap.parse_args()

    if args.write_traffic:
        return write_traffic(*args.write_traffic)

    if args.copy_calibration:
        import torch
        torch.cuda.set_device(0)
        x = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        y = torch.empty_like(x)
        for _ in range(5):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": x.numel() * 4, "copies": 5}))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the hot path shards by heads with no exchange, so the bench measures one GPU's share.",
              file=sys.stderr)
        sys.exit(2)

    if args.variants:
        from sparse_attention_diffusion_pddp_amd import synth
        w = synth.WORKLOADS[args.workload]
        if args.density is not None:
            w = w.with_density(args.density)
        return run_variants(args, w)
    if args.workload in ("voxel3d", "wanvideo"):
        from sparse_attention_diffusion_pddp_amd import schedule, synth
        name, sched = (("voxel3d", schedule.HY3D) if args.workload == "voxel3d"
                       else ("wan480p", schedule.WAN_1_3B_VIDEO))
        w = synth.WORKLOADS[name]
        if args.density is not None:
            w = w.with_density(args.density)
        offload = args.offload == "on" or (args.offload == "auto" and args.workload == "voxel3d")
        return run_schedule(args, w, sched, offload=offload, offload_idx=offload and args.offload_idx)
    if args.workload == "wan720p":
        from sparse_attention_diffusion_pddp_amd import synth
        w = synth.WORKLOADS["wan720p"]
        if args.density is not None:
            w = w.with_density(args.density)
        return run_kernel_only(args, w)

    import torch

    from sparse_attention_diffusion_pddp_amd import binding as mcs
    from sparse_attention_diffusion_pddp_amd import metrics, synth

    mcs.load()
    torch.cuda.set_device(0)
    w = synth.WORKLOADS[args.workload]
    if args.density is not None:
        w = w.with_density(args.density)
    if args.group_size is not None:
        import dataclasses
        w = dataclasses.replace(w, group_size=args.group_size)
    B, H, N, d, T, K, G = w.batch, w.heads, w.seqlen, w.head_dim, w.group_size, w.topk, w.groups
    R_STEPS = max(1, w.reuse_steps)

    # ---- inputs, resident in HBM ------------------------------------------------
    q, k, v = synth.make_qkv(w, seed=args.seed)
    steps_in = [(q, k, v)]
    for s in range(1, R_STEPS + 1):
        steps_in.append(synth.drift_qkv(w, steps_in[-1], step=s, seed=args.seed))
    dev = [tuple(t.cuda() for t in x) for x in steps_in]
    del steps_in
    dq, dk, dv = dev[0]
    desc = mcs.desc_for(dq)
    ws_pddp = torch.empty(mcs.pddp_workspace_size(desc, T), dtype=torch.uint8, device="cuda")
    ws_sel = torch.empty(mcs.select_workspace_size(desc, T, K), dtype=torch.uint8, device="cuda")
    perm = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    o = torch.empty_like(dq)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, H, G, K), dtype=torch.int32, device="cuda")
    r = torch.empty_like(dq)
    ot = [torch.empty_like(dq) for _ in range(R_STEPS)]

    stages = ["pddp", "dense_lse", "select_topk", "residual"] + [f"reuse{s}" for s in range(1, R_STEPS + 1)]

    # cold caches: before every timed stage a 1 GiB write evicts the L2s and
    # the 256 MB MALL, so each stage starts from HBM; the events bracket the
    # stage alone
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

    def step(ev):
        calls = [lambda: mcs.pddp_group(dq, T, perm, ws_pddp),
                 lambda: mcs.anchor_dense_lse(dq, dk, dv, o, lse),
                 lambda: mcs.anchor_select_topk(dq, dk, lse, perm, T, K, idx, ws=ws_sel),
                 lambda: mcs.residual(dq, dk, dv, o, perm, T, idx, K, r)]
        calls += [(lambda s_: lambda: mcs.sparse_apply(*dev[s_], perm, T, idx, K, r, ot[s_ - 1]))(s)
                  for s in range(1, R_STEPS + 1)]
        for j, call in enumerate(calls):
            flush.fill_(j)
            ev[2 * j].record()
            call()
            ev[2 * j + 1].record()

    def new_events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(stages))]

    for _ in range(args.warmup):
        step(new_events())
    torch.cuda.synchronize()

    evs = [new_events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    stage_ms = {name: sum(e[2 * j].elapsed_time(e[2 * j + 1]) for e in evs) / args.steps
                for j, name in enumerate(stages)}
    anchor_ms = sum(stage_ms[s] for s in stages[:4])
    reuse_ms = sum(stage_ms[f"reuse{s}"] for s in range(1, R_STEPS + 1)) / R_STEPS
    flops = metrics.sparse_flops(B, H, N, K, d)
    value = flops / (reuse_ms * 1e-3) / 1e12

    # warm caches (secondary): the reuse calls back to back, inputs left in L2/MALL
    we = [torch.cuda.Event(enable_timing=True) for _ in range(2 * R_STEPS + 1)]
    for s in range(1, R_STEPS + 1):
        mcs.sparse_apply(*dev[s], perm, T, idx, K, r, ot[s - 1])
    we[0].record()
    for i in range(2 * R_STEPS):
        s = 1 + i % R_STEPS
        mcs.sparse_apply(*dev[s], perm, T, idx, K, r, ot[s - 1])
        we[i + 1].record()
    torch.cuda.synchronize()
    reuse_warm_ms = we[0].elapsed_time(we[-1]) / (2 * R_STEPS)
    pddp_bytes = metrics.pddp_algorithmic_bytes(B, H, N, d, T)
    pddp_flop = metrics.pddp_fp64_flops(B, H, N, d, T)

    # the same library's dense path (lse = NULL), the speedup denominator
    o2 = torch.empty_like(dq)
    de = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for _ in range(2):
        mcs.anchor_dense_lse(dq, dk, dv, o2, None)
    de[0].record()
    for i in range(5):
        mcs.anchor_dense_lse(dq, dk, dv, o2, None)
        de[i + 1].record()
    torch.cuda.synchronize()
    dense_ms = de[0].elapsed_time(de[5]) / 5
    density = K / N
    rho, eta = metrics.kernel_speedup(dense_ms, reuse_ms, density)
    anchor_only = stage_ms["select_topk"] + stage_ms["residual"] + stage_ms["pddp"]

    traffic = load_traffic(flops, d, T)
    achieved = value
    gemm = gemm_reference()
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic, "kernel": f"attention_kernel<{d},{T // 32},sparse> (mcs_sparse_apply)",
                "per_launch_flop": flops, "avg_launch_ms": round(reuse_ms, 4),
                "frac_of_gemm_ref": round(achieved / gemm["tflops"], 4)}

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "heads": H, "seqlen": N, "grid": list(w.grid), "head_dim": d,
                   "group_size": T, "density_pct": w.density_pct, "topk": K, "reuse_steps": R_STEPS,
                   "caches": "cold (1 GiB write before each timed stage)", "seed": args.seed},
        "reuse_step_ms_warm": round(reuse_warm_ms, 4),
        "value_warm": round(flops / (reuse_warm_ms * 1e-3) / 1e12, 2),
        "pddp": {"ms": round(stage_ms["pddp"], 4), "algorithmic_bytes": pddp_bytes,
                 "GBps": round(pddp_bytes / (stage_ms["pddp"] * 1e-3) / 1e9, 1),
                 "frac_hbm": round(pddp_bytes / (stage_ms["pddp"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                 "fp64_flop": pddp_flop,
                 "fp64_TFLOPs": round(pddp_flop / (stage_ms["pddp"] * 1e-3) / 1e12, 2),
                 "frac_fp64": round(pddp_flop / (stage_ms["pddp"] * 1e-3) / 1e12 / PEAK_FP64_TFLOPS, 4)},
        "anchor_step_ms": round(anchor_ms, 3),
        "anchor_stages_ms": {s: round(stage_ms[s], 3) for s in stages[:4]},
        "reuse_step_ms": round(reuse_ms, 4),
        "dense_ms": round(dense_ms, 3),
        "dense_tflops": round(metrics.dense_flops(B, H, N, d) / (dense_ms * 1e-3) / 1e12, 2),
        "speedup_vs_dense": round(rho, 3),
        "eta": round(eta, 3),
        "align": round(metrics.align_ratio(N, T, K, 64), 4),
        "anchor_overhead_density_points": round(metrics.anchor_overhead_points(anchor_only, dense_ms), 3),
        "pddp_ms_amortized_2_per_40": round(metrics.amortized_grouping_ms(stage_ms["pddp"]), 4),
        "roofline": roofline,
        "gemm_ref": gemm,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, args.seed)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
