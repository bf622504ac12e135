"""Per-frame correspondence index (K best patches of every other frame) on the
HIP path vs the CPU oracle, through the C ABI.

Index parity: every (row, other frame) segment of the GPU index must equal the
oracle's K best of that frame up to near-ties (band rule, 1e-5), hold only
that frame's patch tokens and be ascending.  End to end: a layer run on the
GPU-built per-frame index matches the oracle element-wise (max-abs 2e-2 bf16,
1e-4 fp32) on every row, the oracle evaluating attention on the GPU's
band-checked index rows and vertical sets.  Full-size (S = 100) checks are in
test_gpu_full_size.py.
"""
import dataclasses

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
    # every row passes the band rule frame by frame; the oracle then evaluates
    # attention on the GPU's rows and every row of every head compares
    _check_rows(w, gidx, np.arange(g.Np), K)
    vsets = {}
    for h in w.heads(ROLE_VERTICAL):
        gv = ctx.build_vertical_index(q, k, h, w.plan[h][1]).cpu().numpy()
        _, r, _, _ = oracle.vertical_index(w.q[h], w.k[h], w.plan[h][1])
        band_check(r, gv, w.plan[h][1])
        vsets[h] = gv.astype(np.int64)
    rows = np.arange(g.N)
    corr = {u: gidx[u].astype(np.int64) for u in range(g.Np)}
    outs, _, _ = oracle.layer(g, w.plan, w.q, w.k, w.v, w.dino, corr_K=K, corr_mode=oracle.MODE_PER_FRAME,
                              rows=rows, corr_rows=corr, vert_sets=vsets)
    got = to_host_f64(o)
    for h, ref in outs.items():
        err = np.max(np.abs(got[h] - ref))
        assert err <= tol(w), (h, err)
    ctx.close()


# Geometries on the fused path (bf16, Df a multiple of 64, P >= 256, K <= 8):
# a per-(row, frame) bound from a 128-patch sample of every frame, the
# symmetric square once filtered by it, per-row frame buckets.
FUSED = [
    (2, 0, 256, 64),     # the smallest fused frame: one 256-row tile per frame
    (4, 5, 700, 64),     # 2800 rows: 11 tiles, the last ragged, tiles across frame boundaries
    (3, 1, 1500, 128),   # wide frames: 6 column tiles per frame, 128 channels
]


@pytest.mark.parametrize("S,ns,P,Df", FUSED)
@pytest.mark.parametrize("K", [1, 3, 8])
def test_fused_per_frame_matches_the_stored_build(S, ns, P, Df, K):
    """The fused build selects from the same fp32 cosines as the build that
    stores every cosine row, so the two indices agree row for row (a row that
    differs must be a near-tie, and both pass the band rule on every row)."""
    saf = _saf()
    w = _workload(S, ns, P, "bf16", Df, seed=23)
    g = w.geom
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
    dino = to_dev(w.dino)
    say(f"fused per-frame index {w.name} K {K}")
    ctx.build_corr_index(dino, K, mode=saf.SAF_CORR_PER_FRAME)
    fused = ctx.get_corr_index().cpu().numpy()
    n_rec = len(ctx.recomputed_rows())
    say(f"stored per-frame index {w.name} K {K}")
    ctx.build_corr_index(dino, K, mode=saf.SAF_CORR_PER_FRAME_STORED)
    stored = ctx.get_corr_index().cpu().numpy()
    ctx.close()
    rows = np.arange(g.Np)
    _check_rows(w, fused, rows, K)
    same = np.all(fused == stored, axis=1)
    if not same.all():
        _check_rows(w, stored, rows[~same], K)
    assert same.mean() >= 0.99, (same.mean(), n_rec)
    # random features: the bounds leave every frame its K candidates and no
    # buffer overflows
    assert n_rec == 0, n_rec


@pytest.mark.parametrize("pattern", ["identical", "zero_rows"])
def test_fused_per_frame_recomputes_flagged_rows(pattern):
    """Rows whose candidate buffer overflows are recomputed exactly: with
    identical features every cosine ties, every frame keeps all P patches and
    all 1,800 rows overflow (the first 1,024 go through cosine rows on the
    matrix cores, the other 776 through the per-row engine); with a tenth of
    the features zero, those rows' cosines are all 0 (the zero-norm rule) and
    only they overflow.  Tied scores go to the lowest patches."""
    saf = _saf()
    S, ns, P, K = 3, 5, 600, 4
    w = _workload(S, ns, P, "bf16", 64, seed=29)
    g = w.geom
    dino = w.dino.copy()
    if pattern == "identical":
        dino[:] = dino[0]
        expect_rec = np.arange(g.Np)
    else:
        expect_rec = np.sort(np.random.default_rng(5).choice(g.Np, g.Np // 10, replace=False))
        dino[expect_rec] = 0
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
    say(f"fused per-frame flagged rows ({pattern})")
    ctx.build_corr_index(to_dev(dino), K, mode=saf.SAF_CORR_PER_FRAME)
    gidx = ctx.get_corr_index().cpu().numpy()
    rec = np.sort(np.asarray(ctx.recomputed_rows(), dtype=np.int64))
    ctx.close()
    assert np.array_equal(rec, expect_rec), (rec.size, expect_rec.size)
    _check_rows(dataclasses.replace(w, dino=dino), gidx, np.arange(g.Np), K)
    # all-tied rows keep the K lowest patches of every other frame
    for u in expect_rec:
        fu = u // g.P
        exp = np.concatenate([f * g.T + g.ns + np.arange(K) for f in range(g.S) if f != fu])
        assert np.array_equal(gidx[u], exp), u
