"""Block-wise correspondence index on the HIP path vs the CPU oracle.

Blocks are b consecutive patches of a frame; block similarity is the token
cosine averaged over the b x b patch pairs.  Index parity: for every query
block, the blocks the GPU selected must be the oracle's top blocks up to
near-ties (band rule, 1e-5, on the oracle's fp64 block scores), per other
frame in per-frame mode; every patch of the block must get exactly the
patches of those blocks, ascending.  End to end: a layer on the GPU-built
block index matches the oracle element-wise (max-abs 2e-2 bf16, 1e-4 fp32)
on every row, the oracle evaluating attention on the GPU's band-checked
index rows.  The S = 100 check is in test_gpu_full_size.py.
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


def _workload(S, ns, P, dtype, Df=64, seed=21):
    g = Geometry(S=S, ns=ns, P=P)
    roles = [ROLE_CORRESPONDENCE, ROLE_POSITION, ROLE_SCANNING, ROLE_DENSE] * 4
    budgets = [0, 0, 7, 0] * 4
    return make_geometry_inputs(g, dtype, roles, budgets, M=2 * P, Df=Df, seed=seed, corr_K=8,
                                name=f"block_S{S}_ns{ns}_P{P}_{dtype}")


def _check_blocks(w, gidx, b, K, mode, qblocks):
    g = w.geom
    per = g.P // b
    kb = (g.S - 1) * min(K, per) if mode == oracle.MODE_PER_FRAME else min(K, (g.S - 1) * per)
    assert gidx.shape[1] == kb * b
    sc = oracle.block_scores(w.dino, g.S, g.P, b, qblocks)
    bframe = np.arange(g.S * per) // per
    for i, A in enumerate(qblocks):
        rows = np.arange(A * b, (A + 1) * b)
        first = gidx[rows[0]]
        for u in rows[1:]:
            np.testing.assert_array_equal(gidx[u], first)
        assert np.all(np.diff(first) > 0)
        patch = (first // g.T) * g.P + first % g.T - g.ns
        assert np.all(first % g.T >= g.ns)
        sel = patch[::b] // b
        np.testing.assert_array_equal(patch, (sel[:, None] * b + np.arange(b)[None, :]).reshape(-1))
        s = np.nan_to_num(sc[i], nan=-np.inf)
        if mode == oracle.MODE_TOTAL:
            band_check(s, sel, kb, valid=bframe != bframe[A])
        else:
            kf = min(K, per)
            fa = A // per
            for f in range(g.S):
                if f == fa:
                    continue
                slot = f - (f > fa)
                seg = sel[slot * kf:(slot + 1) * kf]
                assert np.all(seg // per == f)
                band_check(s[f * per:(f + 1) * per], seg - f * per, kf)


BLOCKS = [
    (3, 5, 300, "bf16", 64, 30),
    (3, 5, 300, "bf16", 64, 1),     # one-patch blocks: the token index through the block path
    (4, 5, 130, "f32", 40, 13),
    (5, 5, 61, "bf16", 64, 61),     # one block per frame
    (40, 1, 64, "bf16", 128, 8),
]


@pytest.mark.parametrize("S,ns,P,dtype,Df,b", BLOCKS)
@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("K", [1, 3, 100])
def test_block_index(S, ns, P, dtype, Df, b, mode, K):
    saf = _saf()
    w = _workload(S, ns, P, dtype, Df)
    g = w.geom
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch_dtype(w))
    say(f"block index {w.name} b {b} mode {mode} K {K}")
    ctx.build_corr_index_blocks(to_dev(w.dino), b, K, mode)
    gidx = ctx.get_corr_index().cpu().numpy()
    _check_blocks(w, gidx, b, K, mode, np.arange(g.Np // b))
    oidx, _ = oracle.block_corr_index(w.dino, g.S, g.ns, g.P, b, K, np.arange(g.Np), mode)
    assert np.mean(np.all(gidx == oidx, axis=1)) > 0.9
    ctx.close()


@pytest.mark.parametrize("mode", [0, 1])
def test_block_layer_end_to_end(mode):
    saf = _saf()
    w = _workload(3, 5, 300, "bf16")
    g = w.geom
    b, K = 20, 2
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    say(f"block end-to-end mode {mode}")
    ctx.build_corr_index_blocks(to_dev(w.dino), b, K, mode)
    o = ctx.sparse_attention(w.plan, q, k, v)
    torch.cuda.synchronize()
    gidx = ctx.get_corr_index().cpu().numpy()
    # every query block passes the band rule; the oracle then evaluates
    # attention on the GPU's rows and every row of every head compares
    _check_blocks(w, gidx, b, K, mode, np.arange(g.Np // b))
    rows = np.arange(g.N)
    corr = {u: gidx[u].astype(np.int64) for u in range(g.Np)}
    outs, _, _ = oracle.layer(g, w.plan, w.q, w.k, w.v, w.dino, rows=rows, corr_rows=corr)
    got = to_host_f64(o)
    for h in outs:
        err = np.max(np.abs(got[h] - outs[h]))
        assert err <= tol(w), (h, err)
    ctx.close()
