"""Static broadcast of a local window to every frame (SAF_BROADCAST) on the HIP
path vs the CPU oracle, element-wise on every row (max-abs 2e-2 bf16, 1e-4
fp32).  In bf16 the patch rows run on the matrix cores in tiles of one patch
position (all frames' queries at that position share one key set) and the
special rows densely; in fp32 the row kernel enumerates each query's set.

Cases: windows on a grid and along the patch index, clipped at every border;
radius 0 (the same position in every frame); a covering radius (dense over
the patches); more frames than one query tile (two tiles per position); one
frame; no special tokens; broadcast heads mixed with every other static role.
"""
import numpy as np
import pytest
import torch

import oracle
from workload import Geometry, make_geometry_inputs, ROLE_DENSE, ROLE_POSITION, ROLE_SCANNING, ROLE_VERTICAL

from helpers import say, to_dev, to_host_f64, tol, torch_dtype

pytestmark = pytest.mark.gpu

BC = oracle.ROLE_BROADCAST


def _saf():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_wise_dynamic_amd as saf
    saf.lib()
    return saf


def _run(saf, w, rows=None):
    g = w.geom
    rows = np.arange(g.N) if rows is None else rows
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch_dtype(w))
    o = ctx.sparse_attention(w.plan, to_dev(w.q), to_dev(w.k), to_dev(w.v))
    torch.cuda.synchronize()
    outs, _, _ = oracle.layer(g, w.plan, w.q, w.k, w.v, rows=rows)
    got = to_host_f64(o)
    for h, ref in outs.items():
        err = np.max(np.abs(got[h][rows] - ref))
        assert err <= tol(w), (h, w.plan[h], err)
    ctx.close()


# (S, ns, P, grid width, dtype)
CASES = [
    (3, 2, 20, 5, "bf16"),
    (3, 2, 20, 5, "f32"),
    (5, 5, 61, 0, "bf16"),     # window along the patch index, prime P
    (2, 0, 200, 20, "bf16"),   # no special tokens
    (4, 5, 130, 13, "f32"),
    (1, 5, 36, 6, "bf16"),     # one frame
]


@pytest.mark.parametrize("S,ns,P,gw,dtype", CASES)
def test_broadcast_layer(S, ns, P, gw, dtype):
    saf = _saf()
    g = Geometry(S=S, ns=ns, P=P)
    radii = [0, 1, 2, 3, 7, P, 1, 2] * 2   # P: the window covers every patch
    w = make_geometry_inputs(g, dtype, [BC] * 16, radii, M=2 * P, Df=16, seed=81, anchors=[gw] * 16,
                             name=f"bcast_S{S}_ns{ns}_P{P}_gw{gw}_{dtype}")
    say(f"broadcast layer {w.name}")
    _run(saf, w)


def test_broadcast_two_tiles_per_position():
    """300 frames: the 300 queries of one patch position span two 256-row tiles."""
    saf = _saf()
    g = Geometry(S=300, ns=1, P=12)
    w = make_geometry_inputs(g, "bf16", [BC] * 16, [0, 1, 2, 5] * 4, M=24, Df=16, seed=82, anchors=[4] * 16,
                             name="bcast_S300_P12")
    rows = np.random.default_rng(3).choice(g.N, 1200, replace=False)
    say(f"broadcast layer {w.name}")
    _run(saf, w, np.sort(rows))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_broadcast_mixed_with_other_static_roles(dtype):
    saf = _saf()
    g = Geometry(S=4, ns=5, P=64)
    roles = [BC] * 4 + [ROLE_POSITION] * 3 + [ROLE_SCANNING] * 3 + [ROLE_VERTICAL] * 3 + [ROLE_DENSE] * 3
    budgets = [1, 0, 3, 2] + [0] * 3 + [5, 16, 3] + [32, 100, 7] + [0] * 3
    anchors = [8, 8, 0, 16] + [0, 1, 3] + [0] * 9
    w = make_geometry_inputs(g, dtype, roles, budgets, M=128, Df=16, seed=83, anchors=anchors,
                             name=f"bcast_mixed_{dtype}")
    say(f"broadcast mixed layer {w.name}")
    _run(saf, w)


def test_broadcast_pairs_match_the_oracle():
    saf = _saf()
    from oracle import profiling as oprof
    g = Geometry(S=3, ns=2, P=20)
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
    for r, gw in [(0, 0), (1, 5), (2, 0), (3, 4), (50, 10)]:
        assert ctx.head_pairs(BC, r, gw) == oprof.head_pairs(g, (BC, r, gw)), (r, gw)
    ctx.close()


def test_s100_broadcast_layer_sampled():
    """The bench's S = 100 layer with its position heads as broadcast heads
    (radius 1 on the 37 x 37 patch grid), in the bench's launch configuration:
    the broadcast heads' outputs on sampled rows (every special row, frame 0,
    frame boundaries) against the oracle."""
    saf = _saf()
    from workload import make_inputs, sample_rows
    w = make_inputs(3)
    g = w.geom
    plan = [(BC, 1, 37, 0) if p[0] == ROLE_POSITION else p for p in w.plan]
    heads = [h for h, p in enumerate(plan) if p[0] == BC]
    assert len(heads) == 4 and g.P == 37 * 37
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
    say("S=100 broadcast layer: index build")
    ctx.build_corr_index(to_dev(w.dino), w.corr_K)
    say("S=100 broadcast layer")
    o = ctx.sparse_attention(plan, to_dev(w.q), to_dev(w.k), to_dev(w.v))
    torch.cuda.synchronize()
    rows = sample_rows(g, 1024, seed=6)
    # only the broadcast heads are compared: the oracle's other heads are dense placeholders
    oplan = [p if p[0] == BC else (ROLE_DENSE, 0, 0, 0) for p in plan]
    outs, _, _ = oracle.layer(g, oplan, w.q, w.k, w.v, rows=rows, heads=heads)
    got = to_host_f64(o)
    for h in heads:
        err = np.max(np.abs(got[h][rows] - outs[h]))
        assert err <= tol(w), (h, err)
    ctx.close()
