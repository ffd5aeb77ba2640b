"""Work counts and the reporting formulas the pages use for this path.

Nominal counts follow the method, not the tiling: FLOPs count 2 per
multiply-add and only the selected keys of a sparse call.
"""
from __future__ import annotations

MIB = 1 << 20


def sparse_flops(batch, heads, seqlen, topk, head_dim) -> int:
    """QK^T and PV over the selected keys of every query row: 4*B*H*N*K*d."""
    return 4 * batch * heads * seqlen * topk * head_dim


def dense_flops(batch, heads, seqlen, head_dim) -> int:
    """QK^T and PV over all keys: 4*B*H*N^2*d."""
    return 4 * batch * heads * seqlen * seqlen * head_dim


def select_sweep_flops(batch, heads, seqlen, head_dim) -> int:
    """The second QK pass of the anchor step: 2*B*H*N^2*d (plus N^2 exponentials)."""
    return 2 * batch * heads * seqlen * seqlen * head_dim


def kernel_speedup(t_dense, t_sparse, density):
    """Attention-kernel speedup rho = t_dense / t_sparse and efficiency eta = rho * s
    against the ideal 1/s speedup (paper landing page, Table 6)."""
    rho = t_dense / t_sparse
    return rho, rho * density


def amortized_grouping_ms(single_ms, calls=2, steps=40):
    """Grouping cost per step when it runs ``calls`` times over ``steps`` steps
    (paper landing page, Table 7: two Fast PDDP calls per 40 steps)."""
    return calls * single_ms / steps


def amortized_kmeans_ms(init_ms, update_ms, steps=40):
    """k-means grouping amortised over the steps: one initialisation, then one
    update per remaining step (paper landing page, Table 7)."""
    return (init_ms + (steps - 1) * update_ms) / steps


def offload_ratio(sparse_tflop, volume_mib):
    """C/V: sparse FLOPs per transferred byte, with V in MiB (paper landing
    page, Table 8 reproduces only with MiB)."""
    return sparse_tflop * 1e12 / (volume_mib * MIB)


def align_ratio(seqlen, group_size, topk, key_tile):
    """Executed over nominal interactions after tiling: every group runs T rows
    and whole key tiles (paper landing page, Table 4 caption's "Align.")."""
    groups = -(-seqlen // group_size)
    exec_keys = -(-topk // key_tile) * key_tile
    return groups * group_size * exec_keys / (seqlen * topk)


def anchor_overhead_points(t_anchor_only_ms, t_dense_ms, anchors=2, steps=40):
    """Anchor-only work expressed as extra attention density, in percentage
    points, for ``anchors`` anchors over ``steps`` sparse steps."""
    return 100.0 * (anchors / steps) * t_anchor_only_ms / t_dense_ms
