"""Correspondence index at the usual feature widths, HIP path vs the oracle.

The matrix-core cosine kernel has a variant with the channel loop fixed at
compile time for 64 (an attention head's q and k), 384, 768 and 1024
channels (ViT-S/B/L features) and a run-time loop for other multiples of 64; every variant must give the
oracle's top-K (band rule, 1e-5).  The geometry (12 frames of 200 patches)
puts the symmetric square over patches [400, 2400): 2000 rows, a ragged last
tile of 208.  Per-frame mode runs the same kernel in its store mode.
"""
import numpy as np
import pytest
import torch

import oracle
from workload import Geometry, make_geometry_inputs, ROLE_CORRESPONDENCE

from helpers import band_check, say, to_dev

pytestmark = pytest.mark.gpu


def _saf():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_wise_dynamic_amd as saf
    saf.lib()
    return saf


def _workload(Df, K, seed):
    g = Geometry(S=12, ns=2, P=200)
    return make_geometry_inputs(g, "bf16", [ROLE_CORRESPONDENCE] * 16, [K] * 16, M=2 * g.P, Df=Df, seed=seed,
                                corr_K=K, name=f"widths_Df{Df}")


@pytest.mark.parametrize("Df", [64, 192, 384, 768, 1024])
def test_total_index_at_width(Df):
    saf = _saf()
    K = 24
    w = _workload(Df, K, seed=60 + Df // 64)
    g = w.geom
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
    say(f"corr index Df={Df} K={K}")
    ctx.build_corr_index(to_dev(w.dino), K)
    got = ctx.get_corr_index().cpu().numpy()
    sc = oracle.corr_scores(w.dino, g.S, g.P, np.arange(g.Np))
    frame = np.arange(g.Np) // g.P
    for u in range(g.Np):
        assert np.all(got[u] % g.T >= g.ns), u
        gp = (got[u] // g.T) * g.P + got[u] % g.T - g.ns
        band_check(np.nan_to_num(sc[u], nan=-np.inf), gp, K, valid=frame != frame[u])
    ctx.close()


@pytest.mark.parametrize("Df", [384, 1024])
def test_per_frame_index_at_width(Df):
    saf = _saf()
    K = 4
    w = _workload(Df, K, seed=70 + Df // 64)
    g = w.geom
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
    say(f"per-frame corr index Df={Df} K={K}")
    ctx.build_corr_index(to_dev(w.dino), K, mode=saf.SAF_CORR_PER_FRAME)
    gidx = ctx.get_corr_index().cpu().numpy()
    assert gidx.shape == (g.Np, (g.S - 1) * K)
    rows = np.arange(g.Np)
    sc = oracle.corr_scores(w.dino, g.S, g.P, rows)
    for u in rows:
        fu = u // g.P
        for f in range(g.S):
            if f == fu:
                continue
            slot = f - (f > fu)
            seg = gidx[u, slot * K:(slot + 1) * K]
            assert np.all(seg // g.T == f), (u, f)
            assert np.all(seg % g.T >= g.ns), (u, f)
            band_check(sc[u, f * g.P:(f + 1) * g.P], seg % g.T - g.ns, K)
    ctx.close()
