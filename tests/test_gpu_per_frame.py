"""Per-frame correspondence index (K best patches of every other frame) on the
HIP path vs the CPU oracle, through the C ABI.

Index parity: every (row, other frame) segment of the GPU index must equal the
oracle's K best of that frame up to near-ties (band rule, 1e-5), hold only
that frame's patch tokens and be ascending.  End to end: a layer run on the
GPU-built per-frame index matches the oracle element-wise (max-abs 2e-2 bf16,
1e-4 fp32) on every row whose GPU index row equals the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
from workload import (Geometry, make_geometry_inputs, make_inputs, ROLE_CORRESPONDENCE, ROLE_DENSE,
                      ROLE_POSITION, ROLE_SCANNING, ROLE_VERTICAL)

from helpers import band_check, say, to_dev, to_host_f64, tol, torch_dtype

pytestmark = pytest.mark.gpu


def _saf():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_wise_dynamic_amd as saf
    saf.lib()
    return saf


def _workload(S, ns, P, dtype, Df=64, seed=11):
    g = Geometry(S=S, ns=ns, P=P)
    roles = [ROLE_CORRESPONDENCE, ROLE_POSITION, ROLE_VERTICAL, ROLE_SCANNING] * 3 + \
            [ROLE_CORRESPONDENCE, ROLE_DENSE, ROLE_CORRESPONDENCE, ROLE_SCANNING]
    budgets = [2, 0, 48, 5] * 3 + [2, 0, 2, 16]
    return make_geometry_inputs(g, dtype, roles, budgets, M=2 * P, Df=Df, seed=seed, corr_K=2,
                                name=f"perframe_S{S}_ns{ns}_P{P}_{dtype}_Df{Df}")


def _check_rows(w, gidx, rows, K):
    """Band rule per (row, other frame) segment of the GPU index."""
    g = w.geom
    kf = min(K, g.P)
    assert gidx.shape[1] == (g.S - 1) * kf
    sc = oracle.corr_scores(w.dino, g.S, g.P, rows)
    for i, u in enumerate(rows):
        fu = u // g.P
        for f in range(g.S):
            if f == fu:
                continue
            slot = f - (f > fu)
            seg = gidx[u, slot * kf:(slot + 1) * kf]
            assert np.all(seg // g.T == f), (u, f)
            assert np.all(seg % g.T >= g.ns), (u, f)
            band_check(sc[i, f * g.P:(f + 1) * g.P], seg % g.T - g.ns, kf)


PER_FRAME = [
    (3, 5, 300, "bf16", 64),
    (3, 5, 300, "f32", 64),
    (5, 5, 61, "bf16", 64),     # frames shorter than one wave's 64 lanes
    (2, 0, 200, "bf16", 96),    # channel count outside the 64-channel matrix tiles
    (4, 5, 130, "f32", 40),
    (3, 1, 1500, "bf16", 128),  # P > 1536: the wide selection variant
]


@pytest.mark.parametrize("S,ns,P,dtype,Df", PER_FRAME)
@pytest.mark.parametrize("K", [1, 4, 8, 9, 37, 100000])
def test_per_frame_index(S, ns, P, dtype, Df, K):
    saf = _saf()
    w = _workload(S, ns, P, dtype, Df)
    g = w.geom
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch_dtype(w))
    say(f"per-frame index {w.name} K {K}")
    ctx.build_corr_index(to_dev(w.dino), K, mode=saf.SAF_CORR_PER_FRAME)
    assert ctx.corr_k() == (g.S - 1) * min(K, g.P)
    gidx = ctx.get_corr_index().cpu().numpy()
    rows = np.arange(g.Np)
    _check_rows(w, gidx, rows, K)
    # away from near-ties the rows are the oracle's exactly
    oidx, _, _ = oracle.corr_index(w.dino, g.S, g.ns, g.P, K, rows, mode=oracle.MODE_PER_FRAME)
    same = np.mean(np.all(gidx == oidx, axis=1))
    assert same > 0.95, same
    ctx.close()


def test_per_frame_rebuild_switches_modes():
    """The cached index follows the last build: total -> per-frame -> total."""
    saf = _saf()
    w = _workload(3, 5, 300, "bf16")
    g = w.geom
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
    dino = to_dev(w.dino)
    ctx.build_corr_index(dino, 24)
    a = ctx.get_corr_index().cpu().numpy()
    ctx.build_corr_index(dino, 3, mode=saf.SAF_CORR_PER_FRAME)
    b = ctx.get_corr_index().cpu().numpy()
    ctx.build_corr_index(dino, 24)
    c = ctx.get_corr_index().cpu().numpy()
    assert a.shape == (g.Np, 24) and b.shape == (g.Np, 6)
    assert np.array_equal(a, c)
    _check_rows(w, b, np.arange(g.Np), 3)
    ctx.close()


@pytest.mark.parametrize("S,ns,P,dtype", [(3, 5, 300, "bf16"), (4, 5, 130, "f32")])
def test_per_frame_layer_end_to_end(S, ns, P, dtype):
    saf = _saf()
    w = _workload(S, ns, P, dtype)
    g = w.geom
    K = 2
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch_dtype(w))
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    say(f"per-frame end-to-end {w.name}")
    ctx.build_corr_index(to_dev(w.dino), K, mode=saf.SAF_CORR_PER_FRAME)
    o = ctx.sparse_attention(w.plan, q, k, v)
    torch.cuda.synchronize()
    gidx = ctx.get_corr_index().cpu().numpy()
    oidx, _, _ = oracle.corr_index(w.dino, g.S, g.ns, g.P, K, np.arange(g.Np), mode=oracle.MODE_PER_FRAME)
    same_rows = np.all(gidx == oidx, axis=1)
    rows = np.arange(g.N)
    t = rows % g.T
    pu = np.clip((rows // g.T) * g.P + t - g.ns, 0, g.Np - 1)
    ok_rows = rows[(t < g.ns) | same_rows[pu]]
    assert ok_rows.size > 0.95 * g.N
    heads = [h for h, p in enumerate(w.plan) if p[0] in (ROLE_CORRESPONDENCE, ROLE_POSITION,
                                                            ROLE_SCANNING, ROLE_DENSE)]
    corr = {u: oidx[u] for u in range(g.Np)}
    outs, _, _ = oracle.layer(g, w.plan, w.q, w.k, w.v, w.dino, corr_K=K, corr_mode=oracle.MODE_PER_FRAME,
                              rows=ok_rows, corr_rows=corr, heads=heads)
    got = to_host_f64(o)
    for h in heads:
        err = np.max(np.abs(got[h][ok_rows] - outs[h]))
        assert err <= tol(w), (h, err)
    ctx.close()


def test_per_frame_s100_sampled():
    """S=100 frames of 1369 patches, Df=1024: K=4 of every other frame
    (Kc = 396), sampled rows checked segment by segment."""
    saf = _saf()
    w = make_inputs(3, heads=[0])
    g = w.geom
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
    say("per-frame index S=100 K=4")
    ctx.build_corr_index(to_dev(w.dino), 4, mode=saf.SAF_CORR_PER_FRAME)
    gidx = ctx.get_corr_index().cpu().numpy()
    rows = np.sort(np.random.default_rng(5).choice(g.Np, 24, replace=False))
    rows[0], rows[-1] = 0, g.Np - 1
    _check_rows(w, gidx, rows, 4)
    ctx.close()
