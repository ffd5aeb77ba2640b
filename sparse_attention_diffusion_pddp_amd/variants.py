"""Selection variants on synthetic data: the ablation axes of the paper
landing page, Tables 3-4, at a matched realised density.

* query order: PDDP groups, whitened PDDP groups, or consecutive tokens (no
  reordering);
* granularity: single keys (the library's exact top-K) or blocks of 64
  consecutive keys ranked by their summed exact group mass
  (mcs_select_blocks; only full blocks compete, so every block variant keeps
  exactly matched_blocks(K, 64) * 64 keys).

Per variant: recall (the mean over groups of the selected keys' share of the
group's probability mass), the sparse output's relative L1 error against
dense at the anchor (no R), and the error of sparse + R against dense on each
drifted reuse step. Every selection and attention step runs in the library's
kernels; recall and the L1 errors are reductions over their outputs.
"""
from __future__ import annotations

import torch

from . import binding as mcs
from . import metrics, synth

BLOCK = 64


def group_sizes(N: int, T: int, device="cuda") -> torch.Tensor:
    G = -(-N // T)
    sizes = torch.full((G,), float(T), device=device)
    sizes[-1] = N - (G - 1) * T
    return sizes


def run(w: synth.Workload, seed: int = 0, block: int = BLOCK, keep_tensors: bool = False) -> dict:
    """All variants of one workload; with ``keep_tensors`` the GPU's groups,
    masses and index lists come back too (for checks against the oracle)."""
    B, H, N, d, T, K, G = w.batch, w.heads, w.seqlen, w.head_dim, w.group_size, w.topk, w.groups
    nb = metrics.matched_blocks(K, block)
    Kb = nb * block
    steps = [synth.make_qkv(w, seed=seed)]
    for s_ in range(1, max(1, w.reuse_steps) + 1):
        steps.append(synth.drift_qkv(w, steps[-1], step=s_, seed=seed))
    dev = [tuple(t.cuda() for t in x) for x in steps]
    q, k, v = dev[0]
    desc = mcs.desc_for(q)
    dense = []
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    for i, (qs, ks, vs) in enumerate(dev):
        o = torch.empty_like(qs)
        mcs.anchor_dense_lse(qs, ks, vs, o, lse if i == 0 else None)
        dense.append(o)

    ws = torch.empty(mcs.pddp_workspace_size(desc, T), dtype=torch.uint8, device="cuda")
    perms = {"pddp": torch.empty((B, H, N), dtype=torch.int32, device="cuda"),
             "pddp_whitened": torch.empty((B, H, N), dtype=torch.int32, device="cuda")}
    grouping_ms = {}
    for name, white in (("pddp", False), ("pddp_whitened", True)):
        mcs.pddp_group(q, T, perms[name], ws, whiten=white)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            mcs.pddp_group(q, T, perms[name], ws, whiten=white)
        e1.record()
        torch.cuda.synchronize()
        grouping_ms[name] = round(e0.elapsed_time(e1) / 5, 3)
    del ws
    perms["none"] = torch.arange(N, dtype=torch.int32, device="cuda").expand(B, H, N).contiguous()
    sizes = group_sizes(N, T)
    mass = torch.empty((B, H, G, N), dtype=torch.float32, device="cuda")
    bws = torch.empty(mcs.select_blocks_workspace_size(desc, T, block, nb), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    rows, kept = [], {}
    for order in ("pddp", "pddp_whitened", "none"):
        perm = perms[order]
        idx_tok = torch.empty((B, H, G, K), dtype=torch.int32, device="cuda")
        mcs.anchor_select_topk(q, k, lse, perm, T, K, idx_tok, group_mass=mass)
        idx_blk = torch.empty((B, H, G, Kb), dtype=torch.int32, device="cuda")
        mcs.select_blocks(desc, mass, T, block, nb, idx_blk, ws=bws)
        if keep_tensors:
            kept[order] = {"perm": perm.clone(), "mass": mass.clone(), "token": idx_tok, f"block{block}": idx_blk}
        for gran, idx, kk in (("token", idx_tok, K), (f"block{block}", idx_blk, Kb)):
            recall = metrics.group_recall(mass, idx, sizes)
            mcs.sparse_apply(q, k, v, perm, T, idx, kk, None, out)
            err_anchor = metrics.rel_l1(out, dense[0])
            if keep_tensors:
                kept[order][f"{gran}_anchor_out"] = out.clone()
            r = torch.empty_like(q)
            mcs.residual(q, k, v, dense[0], perm, T, idx, kk, r)
            errs = []
            for (qs, ks, vs), od in zip(dev[1:], dense[1:]):
                mcs.sparse_apply(qs, ks, vs, perm, T, idx, kk, r, out)
                errs.append(metrics.rel_l1(out, od))
            rows.append({"order": order, "granularity": gran, "keys": kk,
                         "density_pct": round(100.0 * kk / N, 2), "recall": round(float(recall.mean()), 4),
                         "rel_l1_sparse_anchor": round(err_anchor, 4),
                         "rel_l1_reuse_with_R": [round(e, 4) for e in errs],
                         **({"recall_per_group": recall} if keep_tensors else {})})
    torch.cuda.synchronize()
    res = {"workload": w.name, "config": {"heads": H, "seqlen": N, "head_dim": d, "group_size": T,
                                          "density_pct": w.density_pct, "block": block, "blocks": nb,
                                          "reuse_steps": len(dev) - 1, "drift": w.drift, "seed": seed},
           "grouping_ms": grouping_ms, "variants": rows}
    if keep_tensors:
        res["tensors"] = kept
        res["inputs"] = steps
        res["dense"] = [o.cpu() for o in dense]
        res["lse"] = lse.cpu()
    return res
