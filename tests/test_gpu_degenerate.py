"""Degenerate geometries through every role: one patch per frame, two frames,
no special tokens, budgets far beyond the candidate sets.  The GPU builds its
own sets (vertical, correspondence); outputs compare element-wise with the
oracle on the oracle's own sets (max-abs 2e-2 bf16, 1e-4 fp32), and the
GPU-built index rows must equal the oracle's exactly where no near-tie exists
(checked by the band rule)."""
import numpy as np
import pytest
import torch

import oracle
from workload import Geometry, make_geometry_inputs, ROLE_CORRESPONDENCE, ROLE_DENSE, ROLE_POSITION, \
    ROLE_SCANNING, ROLE_VERTICAL

from helpers import band_check, say, to_dev, to_host_f64, tol, torch_dtype

pytestmark = pytest.mark.gpu

CASES = [(2, 0, 1, "bf16"), (3, 1, 1, "bf16"), (2, 5, 3, "f32"), (4, 2, 2, "bf16"), (2, 0, 7, "f32")]


@pytest.mark.parametrize("S,ns,P,dtype", CASES)
def test_degenerate_geometry(S, ns, P, dtype):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_wise_dynamic_amd as saf
    g = Geometry(S=S, ns=ns, P=P)
    roles = [ROLE_POSITION, ROLE_POSITION, ROLE_VERTICAL, ROLE_VERTICAL, ROLE_CORRESPONDENCE,
             ROLE_CORRESPONDENCE, ROLE_SCANNING, ROLE_SCANNING, ROLE_DENSE, ROLE_VERTICAL,
             ROLE_SCANNING, ROLE_POSITION, ROLE_CORRESPONDENCE, ROLE_SCANNING, ROLE_VERTICAL, ROLE_DENSE]
    budgets = [0, 0, 1, 1000, 0, 0, 1, 3, 0, 2, 10 ** 6, 0, 0, 2, 5, 0]
    anchors = [0, S - 1, 0, 0, 0, 0, 0, 0, 0, 0, 0, S - 1, 0, 0, 0, 0]
    K = 3
    w = make_geometry_inputs(g, dtype, roles, budgets, M=max(2 * P, 4), Df=64, seed=51, corr_K=K,
                             anchors=anchors, name=f"deg_S{S}_ns{ns}_P{P}_{dtype}")
    # correspondence heads: budget 0 = the cached index (imported below)
    plan = [(r, (0 if r == ROLE_CORRESPONDENCE else b), a, 0) for r, b, a in zip(roles, budgets, anchors)]
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch_dtype(w))
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    say(f"degenerate {w.name}")
    ctx.build_corr_index(to_dev(w.dino), K)
    gidx = ctx.get_corr_index().cpu().numpy()
    kc = min(K, (S - 1) * P)
    assert gidx.shape == (g.Np, kc)
    sc = oracle.corr_scores(w.dino, g.S, g.P, np.arange(g.Np))
    frame = np.arange(g.Np) // g.P
    for u in range(g.Np):
        gp = (gidx[u] // g.T) * g.P + gidx[u] % g.T - g.ns
        band_check(np.nan_to_num(sc[u], nan=-np.inf), gp, K, valid=frame != frame[u])
    # outputs on the oracle's sets
    oidx, _, _ = oracle.corr_index(w.dino, g.S, g.ns, g.P, K, np.arange(g.Np))
    ctx.set_corr_index(torch.from_numpy(oidx.astype(np.int32)).cuda())
    vert = {}
    for h, r in enumerate(roles):
        if r == ROLE_VERTICAL:
            vert[h] = oracle.vertical_index(w.q[h], w.k[h], plan[h][1])[0]
    ld = max(len(x) for x in vert.values())
    vt = np.zeros((g.H, ld), dtype=np.int32)
    for h, ids in vert.items():
        vt[h, :len(ids)] = ids
    o = ctx.sparse_attention(plan, q, k, v, vert_idx=torch.from_numpy(vt).cuda())
    torch.cuda.synchronize()
    corr = {u: oidx[u] for u in range(g.Np)}
    outs, _, _ = oracle.layer(g, plan, w.q, w.k, w.v, w.dino, corr_K=K, corr_rows=corr)
    got = to_host_f64(o)
    for h, ref in outs.items():
        err = np.max(np.abs(got[h] - ref))
        assert err <= tol(w), (h, plan[h], err)
    # the GPU's own vertical sets
    for h, ids in vert.items():
        gv = ctx.build_vertical_index(q, k, h, plan[h][1]).cpu().numpy()
        r = oracle.vertical_index(w.q[h], w.k[h], plan[h][1])[1]
        band_check(r, gv, plan[h][1])
    ctx.close()
