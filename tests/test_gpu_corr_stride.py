"""Correspondence top-K united with the stride set (SAF_CORR_STRIDE) on the
HIP path vs the CPU oracle: the GPU runs with the oracle's correspondence
index imported, so the key sets are the oracle's and the outputs compare
element-wise (max-abs 2e-2 bf16, 1e-4 fp32).  In bf16 the stride set runs on
the matrix cores and the gathered keys on the row kernel, merged as softmax
partial records; in fp32 one row kernel walks both lists."""
import numpy as np
import pytest
import torch

import oracle
from workload import Geometry, make_geometry_inputs, make_inputs, sample_rows, ROLE_CORRESPONDENCE, \
    ROLE_POSITION, ROLE_SCANNING, ROLE_VERTICAL

from helpers import say, to_dev, to_host_f64, tol, torch_dtype

pytestmark = pytest.mark.gpu

CS = oracle.ROLE_CORR_STRIDE


def _saf():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_wise_dynamic_amd as saf
    saf.lib()
    return saf


def _run(saf, w, plan, rows, corr_K):
    g = w.geom
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch_dtype(w))
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    idx, _, _ = oracle.corr_index(w.dino, g.S, g.ns, g.P, corr_K, np.arange(g.Np))
    ctx.set_corr_index(torch.from_numpy(idx.astype(np.int32)).cuda())
    o = ctx.sparse_attention(plan, q, k, v)
    torch.cuda.synchronize()
    corr = {u: idx[u] for u in range(g.Np)}
    outs, _, _ = oracle.layer(g, plan, w.q, w.k, w.v, w.dino, corr_K=corr_K, rows=rows, corr_rows=corr)
    got = to_host_f64(o)
    for h, ref in outs.items():
        err = np.max(np.abs(got[h][rows] - ref))
        assert err <= tol(w), (h, plan[h], err)
    ctx.close()


@pytest.mark.parametrize("S,ns,P,dtype", [(3, 5, 300, "bf16"), (3, 5, 300, "f32"), (5, 5, 61, "bf16"),
                                          (2, 0, 200, "bf16"), (4, 5, 130, "f32")])
def test_corr_stride_layer(S, ns, P, dtype):
    saf = _saf()
    g = Geometry(S=S, ns=ns, P=P)
    roles = [ROLE_CORRESPONDENCE] * 6 + [ROLE_SCANNING] * 4 + [ROLE_POSITION] * 2 + [ROLE_VERTICAL] * 4
    w = make_geometry_inputs(g, dtype, roles, [24] * 6 + [8] * 4 + [0] * 2 + [32] * 4, M=3 * P, Df=64,
                             seed=31, corr_K=24, name=f"cs_S{S}_P{P}_{dtype}")
    # strides: 1 (union = every key), 2, 7 (with specials off the stride), 16, a stride beyond N
    plan = [(CS, 1, 0, 0), (CS, 2, 0, 0), (CS, 7, 0, 0), (CS, 16, 0, 0), (CS, g.N + 3, 0, 0),
            (ROLE_CORRESPONDENCE, 24, 0, 0)] + [(ROLE_SCANNING, 8, 0, 0)] * 4 + [(ROLE_POSITION, 0, 0, 0)] * 2 + \
        [(CS, 3, 0, 0)] * 4
    say(f"corr+stride layer {w.name}")
    _run(saf, w, plan, np.arange(g.N), 24)


def test_corr_stride_s100_sampled():
    """S=100, the metric's layer with its correspondence heads switched to
    correspondence top-256 united with stride 64; sampled rows."""
    saf = _saf()
    w = make_inputs(3)
    g = w.geom
    plan = [(CS, 64, 0, 0) if r == ROLE_CORRESPONDENCE else (r, b, a, f) for (r, b, a, f) in w.plan]
    rows = sample_rows(g, 200, seed=5)
    say("corr+stride layer S=100 sampled")
    t = rows % g.T
    pr = np.unique((rows[t >= g.ns] // g.T) * g.P + t[t >= g.ns] - g.ns)
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    ctx.build_corr_index(to_dev(w.dino), w.corr_K)
    gidx = ctx.get_corr_index().cpu().numpy()
    oidx, _, _ = oracle.corr_index(w.dino, g.S, g.ns, g.P, w.corr_K, pr)
    full = gidx.copy()
    for u, r in zip(pr, oidx):
        full[u] = r
    ctx.set_corr_index(torch.from_numpy(full.astype(np.int32)).cuda())
    vert = {}
    for h in w.heads(ROLE_VERTICAL):
        ids, _, _, _ = oracle.vertical_index(w.q[h], w.k[h], w.plan[h][1])
        vert[h] = ids
    ld = max(len(x) for x in vert.values())
    vt = np.zeros((g.H, ld), dtype=np.int32)
    for h, ids in vert.items():
        vt[h, :len(ids)] = ids
    o = ctx.sparse_attention(plan, q, k, v, vert_idx=torch.from_numpy(vt).cuda())
    torch.cuda.synchronize()
    corr = {int(u): r for u, r in zip(pr, oidx)}
    heads = [h for h in range(g.H) if plan[h][0] in (CS, ROLE_SCANNING, ROLE_POSITION)]
    outs, _, _ = oracle.layer(g, plan, w.q, w.k, w.v, w.dino, corr_K=w.corr_K, rows=rows, corr_rows=corr,
                              heads=heads)
    got = to_host_f64(o)
    for h in heads:
        err = np.max(np.abs(got[h][rows] - outs[h]))
        assert err <= 2e-2, (h, err)
    ctx.close()
