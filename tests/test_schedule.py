"""Schedule logic (host only): the counts the 3D and video settings of the
paper landing page's appendix Table 9 imply."""
from sparse_attention_diffusion_pddp_amd import schedule as S


def test_hy3d_counts():
    p = S.plan(S.HY3D)
    c = S.counts(p)
    # 12 steps x 40 layers: layer 0 always dense; step 1 anchors layers 1..39;
    # steps 2..12 reuse them
    assert c == {"dense": 12, "anchor": 39, "reuse": 11 * 39}
    assert all(a == "dense" for s, l, a in p if l == 0)
    assert all(a == "anchor" for s, l, a in p if s == 1 and l > 0)
    # one store per anchor layer, one prefetch per reuse layer call
    assert sum(a == "anchor" for _, _, a in p) == 39
    assert sum(a == "reuse" for _, _, a in p) == 429


def test_video_schedule_refresh_anchor():
    p = S.plan(S.WAN_1_3B_VIDEO)
    c = S.counts(p)
    layers, sparse = 30, 29
    # steps 1..9 dense, step 10 anchor (last warm-up step), 11..25 reuse,
    # 26 anchor (refresh), 27..50 reuse; layer 0 always dense
    assert c["anchor"] == 2 * sparse
    assert c["reuse"] == (15 + 24) * sparse
    assert c["dense"] == 50 * layers - c["anchor"] - c["reuse"]
    acts = {(s, l): a for s, l, a in p}
    assert acts[(9, 5)] == "dense" and acts[(10, 5)] == "anchor" and acts[(11, 5)] == "reuse"
    assert acts[(26, 5)] == "anchor" and acts[(50, 29)] == "reuse" and acts[(26, 0)] == "dense"
    # the two anchors per 40 sparse steps that amortise grouping
    assert sum(1 for s in range(11, 51)) == 40
