"""Index builders and the layer at full size (S = 100 and S = 500 frames), in
the launch configuration the benchmark times, against the CPU oracle.

Index parity (SAF3R Sec. 4.1 "DINO Top-K Kernel", Sec. 4.3): every row of
every GPU index is checked for structure (length, ascending and distinct,
patch tokens of other frames only, per-frame segments in frame order); at
least 1,024 rows at S = 100 and 256 at S = 500 are checked against the
oracle's fp64 scores by the near-tie band rule (|s_K - s_K+1| < 1e-5): the
ragged last 256-row tile, rows below 4P, both sides of tile and frame
boundaries, every row the build recomputed exactly after its fast pass,
and random rows.

End to end: the layer runs on the GPU-built sets (index and vertical sets);
the sets of the sampled rows pass the band rule first, and the oracle then
evaluates attention on exactly those sets, so every sampled row of every
head is compared (max-abs 2e-2, bf16 inputs).
"""
import functools

import numpy as np
import pytest
import torch

import oracle
from workload import make_inputs, sample_rows, ROLE_CORRESPONDENCE, ROLE_VERTICAL

from helpers import (band_check, band_check_corr_rows, check_index_structure, index_rows_to_check,
                     patch_rows_of, say, to_dev, to_host_f64, token_patch, tol)

pytestmark = pytest.mark.gpu


def _saf():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_wise_dynamic_amd as saf
    saf.lib()
    return saf


@functools.lru_cache(maxsize=1)
def _s100():
    return make_inputs(3)


def _recomputed(ctx, cap=512, seed=0):
    """Rows the last build recomputed exactly; all of them up to `cap`, else
    a seeded sample of `cap` with the first and last."""
    rows = np.asarray(ctx.recomputed_rows(), dtype=np.int64)
    if rows.size > cap:
        pick = np.random.default_rng(seed).choice(rows[1:-1], cap - 2, replace=False)
        rows = np.union1d(pick, rows[[0, -1]])
    return rows


def _vertical_sets(ctx, w, q, k):
    """GPU vertical sets of every vertical head, each checked by the band rule."""
    sets = {}
    for h in w.heads(ROLE_VERTICAL):
        K = w.plan[h][1]
        gv = ctx.build_vertical_index(q, k, h, K).cpu().numpy()
        _, r, _, _ = oracle.vertical_index(w.q[h], w.k[h], K)
        band_check(r, gv, K)
        sets[h] = gv.astype(np.int64)
    return sets


def test_total_index_s100_full():
    """S = 100 (136,900 patch rows, Df = 1024), K = 256 over all other frames."""
    saf = _saf()
    w = _s100()
    g = w.geom
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
    say("S=100 total index build (K=256)")
    ctx.build_corr_index(to_dev(w.dino), w.corr_K)
    torch.cuda.synchronize()
    gidx = ctx.get_corr_index().cpu().numpy()
    fixed = _recomputed(ctx)
    say(f"S=100 total index: structure of all rows; {fixed.size} recomputed rows")
    check_index_structure(g, gidx, w.corr_K)
    rows = index_rows_to_check(g, 1024, extra=fixed, seed=3)
    assert rows.size >= 1024 and np.all(np.isin(np.arange(136704, 136900), rows))
    say(f"S=100 total index: band rule on {rows.size} rows")
    band_check_corr_rows(w, gidx, rows, w.corr_K)
    ctx.close()


def test_layer_s100_end_to_end_gpu_sets():
    """The bench's layer at S = 100: index and vertical sets built on the GPU
    (vertical sets inside the layer call), every sampled row of all 16 heads
    compared with the oracle evaluated on those band-checked sets."""
    saf = _saf()
    w = _s100()
    g = w.geom
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    say("S=100 end to end: index build + layer")
    ctx.build_corr_index(to_dev(w.dino), w.corr_K)
    o = ctx.sparse_attention(w.plan, q, k, v)
    torch.cuda.synchronize()
    gidx = ctx.get_corr_index().cpu().numpy()
    vsets = _vertical_sets(ctx, w, q, k)
    # the sets built inside the layer call are the ones checked here
    vt = torch.zeros((g.H, max(len(s) for s in vsets.values())), dtype=torch.int32)
    for h, s in vsets.items():
        vt[h, :len(s)] = torch.from_numpy(s.astype(np.int32))
    o2 = ctx.sparse_attention(w.plan, q, k, v, vert_idx=vt.cuda())
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    rows = sample_rows(g, 2048, seed=31)
    pr = patch_rows_of(g, rows)
    say(f"S=100 end to end: band rule on {pr.size} index rows, oracle on {rows.size} rows")
    corr = band_check_corr_rows(w, gidx, pr, w.corr_K)
    outs, _, _ = oracle.layer(g, w.plan, w.q, w.k, w.v, w.dino, corr_K=w.corr_K, rows=rows,
                              corr_rows=corr, vert_sets=vsets)
    got = to_host_f64(o)
    for h, ref in outs.items():
        err = float(np.max(np.abs(got[h][rows] - ref)))
        assert err <= tol(w), f"head {h} role {w.plan[h][0]}: max-abs {err:.3g}"
    ctx.close()


def test_per_frame_index_s100_full():
    """S = 100, K = 4 of every other frame (rows of 396 tokens), fused build
    (sampled per-(row, frame) bounds, one filtered symmetric pass): every row
    equals the build that stores every cosine row, bar near-ties."""
    saf = _saf()
    w = _s100()
    g = w.geom
    K = 4
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
    dino = to_dev(w.dino)
    say("S=100 per-frame index build (K=4, fused)")
    ctx.build_corr_index(dino, K, mode=saf.SAF_CORR_PER_FRAME)
    gidx = ctx.get_corr_index().cpu().numpy()
    rec = _recomputed(ctx)
    check_index_structure(g, gidx, (g.S - 1) * K, per_frame_k=K)
    say("S=100 per-frame index build (K=4, stored cosine rows)")
    ctx.build_corr_index(dino, K, mode=saf.SAF_CORR_PER_FRAME_STORED)
    sidx = ctx.get_corr_index().cpu().numpy()
    ctx.close()
    check_index_structure(g, sidx, (g.S - 1) * K, per_frame_k=K)
    same = np.all(gidx == sidx, axis=1)
    differ = np.flatnonzero(~same)
    say(f"S=100 per-frame: {differ.size} rows differ between the builds, {rec.size} recomputed")
    assert same.mean() >= 0.999, same.mean()
    rows = np.union1d(np.union1d(index_rows_to_check(g, 1024, seed=4), rec), differ[:256])
    say(f"S=100 per-frame index: band rule on {rows.size} rows x 99 frames")
    band_check_corr_rows(w, gidx, rows, K, per_frame=True)
    if differ.size:
        band_check_corr_rows(w, sidx, differ[:256], K, per_frame=True)


def test_qk_index_s100_full():
    """S = 100: the index from the first correspondence head's logits, K = 256
    (band 1e-4 on the fp64 logits: fp32 sums of 64 bf16 products ~10)."""
    saf = _saf()
    w = _s100()
    g = w.geom
    h = w.heads(ROLE_CORRESPONDENCE)[0]
    K = 256
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
    say(f"S=100 qk index build (head {h}, K={K})")
    ctx.build_corr_index_qk(to_dev(w.q), to_dev(w.k), h, K)
    gidx = ctx.get_corr_index().cpu().numpy()
    fixed = _recomputed(ctx)
    check_index_structure(g, gidx, K)
    rows = index_rows_to_check(g, 1024, extra=fixed, seed=5)
    say(f"S=100 qk index: band rule on {rows.size} rows ({fixed.size} recomputed)")
    dec = lambda a: (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    Q, Kf = dec(w.q[h]), dec(w.k[h])
    tok = g.patch_token(np.arange(g.Np))
    Kp = Kf[tok]
    frame = np.arange(g.Np) // g.P
    for c0 in range(0, rows.size, 256):
        part = rows[c0:c0 + 256]
        s = Kp @ Q[tok[part]].T
        for i, u in enumerate(part):
            sc = np.where(frame == frame[u], -np.inf, s[:, i])
            band_check(sc, token_patch(g, gidx[u]), K, valid=frame != frame[u], eps=1e-4)
    ctx.close()


def test_block_index_s100_blocks():
    """S = 100, blocks of one patch row (b = 37), 7 blocks per query block:
    structure of every row; 48 query blocks (both ends, frame boundaries,
    random) against the oracle's literal block averages."""
    saf = _saf()
    w = _s100()
    g = w.geom
    b, K = 37, 7
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
    say("S=100 block index build (b=37, K=7)")
    ctx.build_corr_index_blocks(to_dev(w.dino), b, K, 0)
    gidx = ctx.get_corr_index().cpu().numpy()
    check_index_structure(g, gidx, K * b)
    per = g.P // b
    nb = g.Np // b
    rng = np.random.default_rng(9)
    qb = np.unique(np.concatenate([[0, 1, per - 1, per, nb // 2, nb - per, nb - 2, nb - 1],
                                   rng.choice(nb, 40, replace=False)]))
    say(f"S=100 block index: {qb.size} query blocks")
    sc = oracle.block_scores(w.dino, g.S, g.P, b, qb)
    bframe = np.arange(nb) // per
    for i, A in enumerate(qb):
        first = gidx[A * b]
        for u in range(A * b + 1, (A + 1) * b):
            np.testing.assert_array_equal(gidx[u], first)
        patch = token_patch(g, first)
        sel = patch[::b] // b
        np.testing.assert_array_equal(patch, (sel[:, None] * b + np.arange(b)[None, :]).reshape(-1))
        band_check(np.nan_to_num(sc[i], nan=-np.inf), sel, K, valid=bframe != bframe[A])
    ctx.close()


def test_s500_index_and_layer_end_to_end():
    """S = 500 frames of 36 x 36 patches (N = 650,500), one head per role,
    K = 128: structure of all 648,000 index rows; the band rule on at least
    256 rows (the ragged last tile, boundaries, recomputed rows, and every
    patch row of the layer sample); the layer on the GPU-built sets against
    the oracle on every sampled row."""
    saf = _saf()
    heads = [0, 4, 7, 10]  # position, vertical, correspondence, scanning
    w = make_inputs(5, heads=heads)
    g = w.geom
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    say("S=500 index build (K=128)")
    ctx.build_corr_index(to_dev(w.dino), w.corr_K)
    torch.cuda.synchronize()
    gidx = ctx.get_corr_index().cpu().numpy()
    fixed = _recomputed(ctx, cap=64)
    check_index_structure(g, gidx, w.corr_K)
    rng = np.random.default_rng(55)
    rows = np.unique(np.concatenate([[0, 4, g.T, g.N - g.T, g.N - 1], np.arange(g.ns, g.ns + 8),
                                     g.N - 1 - np.arange(g.P // 2), rng.choice(g.N, 96, replace=False)]))
    pr = patch_rows_of(g, rows)
    check = index_rows_to_check(g, 256, extra=np.concatenate([fixed, pr]), seed=6)
    assert np.all(np.isin(np.arange(647936, 648000), check))
    say(f"S=500 index: band rule on {check.size} rows ({fixed.size} recomputed)")
    corr = band_check_corr_rows(w, gidx, check, w.corr_K)
    say("S=500 layer on GPU-built sets")
    o = ctx.sparse_attention(w.plan, q, k, v)
    torch.cuda.synchronize()
    vsets = _vertical_sets(ctx, w, q, k)
    outs, _, _ = oracle.layer(g, w.plan, w.q, w.k, w.v, w.dino, corr_K=w.corr_K, rows=rows,
                              corr_rows={u: corr[u] for u in pr}, heads=heads, vert_sets=vsets)
    got = to_host_f64(o)
    for h in heads:
        err = float(np.max(np.abs(got[h][rows] - outs[h])))
        assert err <= tol(w), f"head {h}: max-abs {err:.3g}"
    ctx.close()
