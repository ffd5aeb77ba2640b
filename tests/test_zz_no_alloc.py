"""The allocation-free PDDP entry point (mcs_pddp_group_noalloc) against
mcs_pddp_group on the same inputs, through the C-ABI: bitwise equal groups on
two calls in a row, the second with a smaller input (so the library's scratch
holds the first call's contents when the second starts), plain and
whitened; and a shape whose single head needs more than the scratch is
refused before any launch."""
import numpy as np
import pytest
import torch

from sparse_attention_diffusion_pddp_amd import binding as mcs
from sparse_attention_diffusion_pddp_amd import synth

pytestmark = pytest.mark.gpu


def _groups_both_ways(w, seed, whiten):
    q = synth.make_qkv(w, seed=seed)[0].cuda()
    B, N, H, d = q.shape
    T = w.group_size
    desc = mcs.desc_for(q)
    ws = torch.empty(mcs.pddp_workspace_size(desc, T), dtype=torch.uint8, device="cuda")
    want = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    mcs.pddp_group(q, T, want, ws, whiten=whiten)
    del ws
    got = torch.full((B, H, N), -1, dtype=torch.int32, device="cuda")
    mcs.pddp_group_noalloc(q, T, got, whiten=whiten)
    torch.cuda.synchronize()
    return got.cpu().numpy(), want.cpu().numpy()


@pytest.mark.parametrize("whiten", [False, True])
def test_noalloc_matches_workspace_call_twice_second_smaller(lib, whiten):
    # first: the wan480p layer, 12 heads of N = 32760 in chunks of the scratch
    big = synth.WORKLOADS["wan480p"]
    print(f"\n[noalloc wan480p whiten={whiten}]", flush=True)
    got, want = _groups_both_ways(big, 5, whiten)
    assert np.array_equal(got, want)
    # second, right after: a smaller layer (2 batches x 3 heads, N = 5000, d = 64, T = 64)
    small = synth.small_workload(5000, heads=3, head_dim=64, group_size=64, density_pct=15, batch=2)
    print(f"[noalloc small whiten={whiten}]", flush=True)
    got, want = _groups_both_ways(small, 6, whiten)
    assert np.array_equal(got, want)
    for b in range(2):
        for h in range(3):
            assert np.array_equal(np.sort(got[b, h]), np.arange(5000))


def test_noalloc_refuses_a_head_larger_than_the_scratch(lib):
    q = torch.zeros((1, 200000, 1, 128), dtype=torch.bfloat16, device="cuda")
    perm = torch.empty((1, 1, 200000), dtype=torch.int32, device="cuda")
    with pytest.raises(mcs.McsError) as e:
        mcs.pddp_group_noalloc(q, 128, perm)
    assert e.value.status == 2 and "scratch" in str(e.value)
