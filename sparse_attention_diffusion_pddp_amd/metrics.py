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


def pddp_levels(seqlen: int, group_size: int) -> int:
    """Depth of the PDDP tree: splits until every node holds at most one tile."""
    levels, n = 0, seqlen
    while n > group_size:  # the right child, never smaller than the left, is the deepest
        G = -(-n // group_size)
        n = n - (G // 2) * group_size
        levels += 1
    return levels


def pddp_algorithmic_bytes(batch, heads, seqlen, head_dim, group_size, elem_bytes=2) -> int:
    """Bytes the grouping must move at the least: one read of every query per
    tree level, plus the int32 group order written once."""
    return batch * heads * (pddp_levels(seqlen, group_size) * seqlen * head_dim * elem_bytes + seqlen * 4)


def pddp_fp64_flops(batch, heads, seqlen, head_dim, group_size, power_iters=16) -> int:
    """float64 FLOPs of the grouping as this library computes it: the
    second moments (the upper triangle of d x d, in 16 x 16 tiles, per
    accumulated token: every token at the first level, the left children's
    (about half) below), 16 matrix-vector products per split node, and one
    projection of every token per level. 2 FLOPs per multiply-add."""
    tiles = (head_dim // 16) * (head_dim // 16 + 1) // 2
    per_token = tiles * 256
    levels = pddp_levels(seqlen, group_size)
    groups = -(-seqlen // group_size)
    accumulated = seqlen + (levels - 1) * (seqlen // 2) if levels else 0
    nodes = groups - 1  # every split node of a binary tree with `groups` leaves
    macs = accumulated * per_token + nodes * power_iters * head_dim * head_dim + levels * seqlen * head_dim
    return 2 * batch * heads * macs


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


def matched_blocks(topk: int, block: int) -> int:
    """Blocks of `block` keys that match a density of `topk` single keys:
    the nearest whole number of blocks (halves up), at least one."""
    return max(1, (topk + block // 2) // block)


def group_recall(mass, kv_idx, group_rows):
    """Per group, the mean over its query rows of the probability mass of the
    selected keys: sum_{j in S_g} A[g][j] / |g|. mass [..., G, N] and kv_idx
    [..., G, K] are torch tensors; group_rows [G] the rows of each group."""
    import torch

    sel = mass.gather(-1, kv_idx.long()).to(torch.float64).sum(-1)
    return sel / group_rows.to(torch.float64)


def rel_l1(x, ref) -> float:
    """sum |x - ref| / sum |ref| over two torch tensors of one shape."""
    import torch

    x64, r64 = x.to(torch.float64), ref.to(torch.float64)
    return float((x64 - r64).abs().sum() / r64.abs().sum())
