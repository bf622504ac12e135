"""Both softmax shifts of the matrix-core attention kernel against the oracle.

A wave whose logits are bounded by |q| max|k| <= 56 (log2 units) subtracts a
fixed per-query shift; any other wave keeps a running maximum.  Scaling a
head's Q and K by 4 (exact in bf16) lifts its bound to ~250, so its waves take
the running maximum; scaling only some query rows mixes the two paths within
one launch and within one wave.  Every row of the listed heads is compared
with the oracle (max-abs 2e-2, bf16 inputs)."""
import numpy as np
import pytest
import torch

import oracle
from workload import (Geometry, bf16_round, bf16_to_f32, make_geometry_inputs, ROLE_CORRESPONDENCE, ROLE_DENSE,
                      ROLE_POSITION, ROLE_SCANNING, ROLE_VERTICAL)

from helpers import say, to_dev, to_host_f64

pytestmark = pytest.mark.gpu


def _saf():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_wise_dynamic_amd as saf
    saf.lib()
    return saf


def _scale(a, f, rows=None):
    x = bf16_to_f32(a).copy()
    if rows is None:
        x *= f
    else:
        x[rows] *= f
    return bf16_round(x)


def test_dense_kernel_both_shifts():
    saf = _saf()
    g = Geometry(S=3, ns=5, P=600)
    w = make_geometry_inputs(g, "bf16", [ROLE_DENSE] * 16, [0] * 16, M=1800, Df=32, seed=21, dino=False)
    q, k = w.q.copy(), w.k.copy()
    for h in range(4):          # whole heads beyond the bound
        q[h], k[h] = _scale(q[h], 4.0), _scale(k[h], 4.0)
    for h in range(4, 8):       # rows 0..99 beyond it: waves of one tile mixed
        q[h] = _scale(q[h], 8.0, np.arange(100))
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
    say(f"dense kernel, both softmax shifts, N={g.N}")
    o = ctx.dense_attention(to_dev(q), to_dev(k), to_dev(w.v))
    torch.cuda.synchronize()
    got = to_host_f64(o)
    rows = np.arange(g.N)
    for h in (0, 3, 4, 7, 8, 15):
        ref = oracle.attention(q[h], k[h], w.v[h], rows, rows)
        err = float(np.max(np.abs(got[h] - ref)))
        assert err <= 2e-2, (h, err)
    ctx.close()


def test_layer_both_shifts():
    saf = _saf()
    g = Geometry(S=3, ns=5, P=300)
    roles = [ROLE_POSITION, ROLE_POSITION, ROLE_VERTICAL, ROLE_VERTICAL, ROLE_SCANNING, ROLE_SCANNING,
             ROLE_CORRESPONDENCE, ROLE_CORRESPONDENCE, ROLE_DENSE, ROLE_DENSE, ROLE_POSITION, ROLE_VERTICAL,
             ROLE_SCANNING, ROLE_SCANNING, ROLE_POSITION, ROLE_SCANNING]
    budgets = [0, 0, 64, 200, 8, 3, 24, 24, 0, 0, 0, 7, 1, 64, 0, 16]
    w = make_geometry_inputs(g, "bf16", roles, budgets, M=900, Df=64, seed=5, corr_K=24)
    q, k = w.q.copy(), w.k.copy()
    for h in (0, 2, 4, 6, 8):   # one head of every role beyond the bound
        q[h], k[h] = _scale(q[h], 4.0), _scale(k[h], 4.0)
    for h in (1, 3, 5, 7, 9):   # some query rows beyond it (specials of frame 0 and the first patches)
        q[h] = _scale(q[h], 8.0, np.arange(70))
    vert = {}
    ld = 200
    vt = np.zeros((g.H, ld), dtype=np.int32)
    for h in range(g.H):
        if roles[h] == ROLE_VERTICAL:
            ids, _, _, _ = oracle.vertical_index(q[h], k[h], budgets[h])
            vert[h] = ids.astype(np.int64)
            vt[h, :ids.size] = ids
    corr_idx, _, _ = oracle.corr_index(w.dino, g.S, g.ns, g.P, w.corr_K, np.arange(g.Np))
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
    ctx.set_corr_index(torch.from_numpy(corr_idx.astype(np.int32)).cuda())
    say(f"layer, both softmax shifts, N={g.N}")
    o = ctx.sparse_attention(w.plan, to_dev(q), to_dev(k), to_dev(w.v), vert_idx=torch.from_numpy(vt).cuda())
    torch.cuda.synchronize()
    got = to_host_f64(o)
    rows = np.arange(g.N)
    outs, _, _ = oracle.layer(g, w.plan, q, k, w.v, w.dino, corr_K=w.corr_K, rows=rows,
                              corr_rows={u: corr_idx[u].astype(np.int64) for u in range(g.Np)}, vert_sets=vert)
    for h, ref in outs.items():
        err = float(np.max(np.abs(got[h] - ref)))
        assert err <= 2e-2, f"head {h} role {roles[h]}: max-abs {err:.3g}"
    ctx.close()
