"""The bitmap form of the KV indices used for host offload, on the GPU:
encode matches the plain definition (bit j % 32 of word j // 32 of a row is
set iff key j is selected), decode returns the ascending index list, and
decode(encode(idx)) == idx bit for bit, on ragged key counts, word
boundaries, K = 1, K = N and the pipeline's own indices."""
import numpy as np
import pytest
import torch

from sparse_attention_diffusion_pddp_amd import binding as mcs
from sparse_attention_diffusion_pddp_amd import synth

pytestmark = pytest.mark.gpu


def bitmap_definition(idx, N):
    """uint32 words per row: bit (j % 32) of word j // 32 set iff j in the row."""
    rows = idx.reshape(-1, idx.shape[-1]).astype(np.int64)
    W = (N + 31) // 32
    out = np.zeros((rows.shape[0], W), dtype=np.uint32)
    r = np.repeat(np.arange(rows.shape[0]), rows.shape[1])
    j = rows.reshape(-1)
    np.bitwise_or.at(out, (r, j // 32), (np.uint32(1) << (j % 32).astype(np.uint32)))
    return out.reshape(idx.shape[:-1] + (W,))


def random_idx(rng, B, H, G, N, K):
    return np.stack([np.sort(rng.choice(N, size=K, replace=False)) for _ in range(B * H * G)]).reshape(B, H, G, K)


CASES = [  # (B, H, N, T, K)
    (1, 2, 1000, 128, 150),
    (2, 1, 777, 64, 200),
    (1, 1, 31, 64, 7),
    (1, 1, 32, 64, 32),
    (1, 3, 33, 64, 1),
    (1, 2, 4096, 128, 4096),
    (1, 1, 98304, 128, 14746),
]


@pytest.mark.parametrize("B,H,N,T,K", CASES)
def test_encode_decode(lib, B, H, N, T, K):
    print(f"\n[codec B={B} H={H} N={N} T={T} K={K}]", flush=True)
    rng = np.random.default_rng(N * 7 + K)
    G = (N + T - 1) // T
    idx = random_idx(rng, B, H, G, N, K).astype(np.int32)
    desc = mcs.Desc(B, H, N, 128, N * H * 128, H * 128, 128, 0.088)
    nbytes = mcs.kv_idx_bitmap_bytes(desc, T)
    W = (N + 31) // 32
    assert nbytes == B * H * G * W * 4
    bm = torch.empty((B, H, G, W), dtype=torch.int32, device="cuda")
    dev_idx = torch.from_numpy(idx).cuda()
    mcs.kv_idx_encode(desc, T, dev_idx, K, bm)
    back = torch.full_like(dev_idx, -1)
    mcs.kv_idx_decode(desc, T, bm, K, back)
    # decoding a bitmap made on the host
    host_bm = bitmap_definition(idx, N)
    back2 = torch.full_like(dev_idx, -1)
    mcs.kv_idx_decode(desc, T, torch.from_numpy(host_bm.view(np.int32)).cuda(), K, back2)
    torch.cuda.synchronize()
    assert np.array_equal(bm.cpu().numpy().view(np.uint32), host_bm)
    assert np.array_equal(back.cpu().numpy(), idx)
    assert np.array_equal(back2.cpu().numpy(), idx)


def test_pipeline_indices_roundtrip(lib):
    w = synth.small_workload(1000, heads=2, head_dim=128, group_size=128, density_pct=15)
    q, k, v = (t.cuda() for t in synth.make_qkv(w, seed=5))
    desc = mcs.desc_for(q)
    B, H, N, T, K, G = w.batch, w.heads, w.seqlen, w.group_size, w.topk, w.groups
    ws = torch.empty(mcs.pddp_workspace_size(desc, T), dtype=torch.uint8, device="cuda")
    perm = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, H, G, K), dtype=torch.int32, device="cuda")
    mcs.pddp_group(q, T, perm, ws)
    mcs.anchor_dense_lse(q, k, v, o, lse)
    mcs.anchor_select_topk(q, k, lse, perm, T, K, idx, ws=torch.empty(mcs.select_workspace_size(desc, T, K),
                                                                         dtype=torch.uint8, device="cuda"))
    bm = torch.empty(mcs.kv_idx_bitmap_bytes(desc, T) // 4, dtype=torch.int32, device="cuda")
    mcs.kv_idx_encode(desc, T, idx, K, bm)
    back = torch.empty_like(idx)
    mcs.kv_idx_decode(desc, T, bm, K, back)
    torch.cuda.synchronize()
    assert torch.equal(back, idx)
    # the decoded indices drive the reuse call exactly like the originals
    r = torch.empty_like(q)
    mcs.residual(q, k, v, o, perm, T, idx, K, r)
    o1, o2 = torch.empty_like(q), torch.empty_like(q)
    mcs.sparse_apply(q, k, v, perm, T, idx, K, r, o1)
    mcs.sparse_apply(q, k, v, perm, T, back, K, r, o2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
