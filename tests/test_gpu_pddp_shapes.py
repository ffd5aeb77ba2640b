"""PDDP groups at the shapes the full-size tests do not reach, bit-exact
against the oracle.

The full-size tests group at d = 128, T = 128. These cover:
* d = 64, whose moment kernel gives its last tile slot to two waves only
  (10 upper-triangle tiles over 4 waves);
* T = 64 trees;
* the reduce pass (units of more than 4 moment chunks) at both widths;
* register splits of 4-64 keys per thread at d = 64;
* a deep tree (N = 200,000: 11 levels, a root split beyond the register
  path, the plan's node lists in global memory).

Every head uses the clustered generator of the pages' video workloads."""
import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_diffusion_pddp_amd import binding as mcs
from sparse_attention_diffusion_pddp_amd import synth
from tests import parity_util as U

pytestmark = pytest.mark.gpu

SHAPES = [
    # (N, d, T, heads)
    (5000, 64, 64, 2),
    (9000, 128, 64, 1),
    (4500, 64, 128, 2),
    (33000, 64, 128, 1),
    # 11 levels; a root of more than 32,768 tokens (the split's LDS path) and
    # plan lists too large for the plan block's LDS
    (200000, 128, 128, 1),
]


@pytest.mark.parametrize("N,d,T,H", SHAPES)
def test_pddp_groups_exact(lib, N, d, T, H):
    print(f"\n[pddp N={N} d={d} T={T} H={H}]", flush=True)
    w = synth.small_workload(N, heads=H, head_dim=d, group_size=T, density_pct=15)
    q = synth.make_qkv(w, seed=N + d + T)[0]
    dq = q.cuda()
    desc = mcs.desc_for(dq)
    ws = torch.empty(mcs.pddp_workspace_size(desc, T), dtype=torch.uint8, device="cuda")
    perm = torch.empty((1, H, N), dtype=torch.int32, device="cuda")
    mcs.pddp_group(dq, T, perm, ws)
    torch.cuda.synchronize()
    got = perm.cpu().numpy()
    for h in range(H):
        want = O.pddp_group(U.head_np(q, 0, h), T)
        assert np.array_equal(got[0, h], want), f"head {h}: groups differ"


def _whitened_groups(q, T):
    dq = q.cuda()
    B, N, H, d = dq.shape
    desc = mcs.desc_for(dq)
    ws = torch.empty(mcs.pddp_workspace_size(desc, T), dtype=torch.uint8, device="cuda")
    perm = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    mcs.pddp_group(dq, T, perm, ws, whiten=True)
    torch.cuda.synchronize()
    return perm.cpu().numpy()


@pytest.mark.parametrize("N,d,T", [(5000, 64, 64), (4500, 64, 128), (9000, 128, 64), (1000, 128, 128)])
def test_whitened_pddp_groups_exact(lib, N, d, T):
    """Whitened grouping (per-dimension standardization) against the oracle."""
    print(f"\n[whitened pddp N={N} d={d} T={T}]", flush=True)
    w = synth.small_workload(N, heads=1, head_dim=d, group_size=T, density_pct=15)
    q = synth.make_qkv(w, seed=N + 3 * d + T)[0]
    got = _whitened_groups(q, T)
    assert np.array_equal(got[0, 0], O.pddp_group(U.head_np(q, 0, 0), T, whiten=True))


def test_whitened_pddp_full_size_wan480p(lib):
    """Two heads of the wan480p shape (N = 32760, d = 128, T = 128); the
    whitened groups also differ from the plain ones."""
    print("\n[whitened pddp wan480p]", flush=True)
    w = synth.WORKLOADS["wan480p"]
    q = synth.make_qkv(w, seed=5)[0]
    got = _whitened_groups(q, w.group_size)
    for h in (0, w.heads - 1):
        qh = U.head_np(q, 0, h)
        want = O.pddp_group(qh, w.group_size, whiten=True)
        assert np.array_equal(got[0, h], want), f"head {h}"
        assert not np.array_equal(want, O.pddp_group(qh, w.group_size))


def test_whitened_pddp_constant_dims_and_equal_queries(lib):
    """Zero-variance dimensions stay unscaled and the root starts at the
    first dimension of nonzero variance (dim 0 is constant here); with every
    query equal all variances are 0 and the groups are index order."""
    print("\n[whitened pddp constant dims]", flush=True)
    N, d, T = 1500, 64, 64
    w = synth.small_workload(N, heads=2, head_dim=d, group_size=T, density_pct=15)
    q = synth.make_qkv(w, seed=31)[0]
    q[0, :, 0, 0] = 0.75
    q[0, :, 0, 9] = -2.0
    q[0, :, 1, :] = q[0, 0, 1, :]
    got = _whitened_groups(q, T)
    assert np.array_equal(got[0, 0], O.pddp_group(U.head_np(q, 0, 0), T, whiten=True))
    assert np.array_equal(got[0, 1], np.arange(N))


@pytest.mark.parametrize("iters", [1, 3, 64])
@pytest.mark.parametrize("whiten", [False, True])
def test_pddp_power_iteration_counts(lib, iters, whiten):
    """The API's iteration count reaches the kernel. With 1 or 3 iterations
    the direction is far from converged, so the start vector and every step
    must match the oracle's."""
    print(f"\n[pddp iters={iters} whiten={whiten}]", flush=True)
    N, d, T = 3000, 128, 128
    w = synth.small_workload(N, heads=1, head_dim=d, group_size=T, density_pct=15)
    q = synth.make_qkv(w, seed=40 + iters)[0]
    dq = q.cuda()
    desc = mcs.desc_for(dq)
    ws = torch.empty(mcs.pddp_workspace_size(desc, T), dtype=torch.uint8, device="cuda")
    perm = torch.empty((1, 1, N), dtype=torch.int32, device="cuda")
    mcs.pddp_group(dq, T, perm, ws, power_iters=iters, whiten=whiten)
    torch.cuda.synchronize()
    want = O.pddp_group(U.head_np(q, 0, 0), T, power_iters=iters, whiten=whiten)
    assert np.array_equal(perm.cpu().numpy()[0, 0], want)
