"""Correspondence index from one head's logits (q_i . k_j) on the HIP path vs
the CPU oracle.  Index parity: band rule on the oracle's fp64 logits with a
band of 1e-4 (fp32 accumulation of d = 64 products of |q|, |k| ~ 10 carries
errors ~1e-5); end to end: a layer whose correspondence heads use the index matches the
oracle element-wise on every row, the oracle evaluating attention on the
GPU's band-checked rows.  The S = 100 check is in test_gpu_full_size.py."""
import numpy as np
import pytest
import torch

import oracle
from workload import Geometry, make_geometry_inputs, make_inputs, ROLE_CORRESPONDENCE, ROLE_DENSE, \
    ROLE_POSITION, ROLE_SCANNING

from helpers import band_check, say, to_dev, to_host_f64, tol, torch_dtype

pytestmark = pytest.mark.gpu
BAND = 1e-4


def _saf():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_wise_dynamic_amd as saf
    saf.lib()
    return saf


def _logits(w, h, rows):
    g = w.geom
    dec = lambda a: (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64) if a.dtype == np.uint16 \
        else a.astype(np.float64)
    Q, K = dec(w.q[h]), dec(w.k[h])
    tok = np.array([(v // g.P) * g.T + g.ns + v % g.P for v in range(g.Np)])
    return K[tok] @ Q[tok[rows]].T, tok      # [Np, nrows]


def _check(w, h, gidx, rows, K, mode):
    g = w.geom
    s, tok = _logits(w, h, rows)
    frame = np.arange(g.Np) // g.P
    for i, u in enumerate(rows):
        gp = (gidx[u] // g.T) * g.P + gidx[u] % g.T - g.ns
        assert np.all(gidx[u] % g.T >= g.ns)
        if mode == 0:
            sc = np.where(frame == frame[u], -np.inf, s[:, i])
            band_check(sc, gp, K, valid=frame != frame[u], eps=BAND)
        else:
            kf = min(K, g.P)
            fu = u // g.P
            for f in range(g.S):
                if f == fu:
                    continue
                slot = f - (f > fu)
                seg = gp[slot * kf:(slot + 1) * kf]
                assert np.all(seg // g.P == f)
                band_check(s[f * g.P:(f + 1) * g.P, i], seg - f * g.P, kf, eps=BAND)


@pytest.mark.parametrize("S,ns,P,dtype", [(3, 5, 300, "bf16"), (3, 5, 300, "f32"), (5, 5, 61, "bf16"),
                                          (2, 0, 200, "bf16"), (4, 5, 130, "f32")])
@pytest.mark.parametrize("mode,K", [(0, 1), (0, 24), (0, 10000), (1, 3), (1, 9)])
def test_qk_index(S, ns, P, dtype, mode, K):
    saf = _saf()
    g = Geometry(S=S, ns=ns, P=P)
    roles = [ROLE_CORRESPONDENCE] * 8 + [ROLE_SCANNING] * 8
    w = make_geometry_inputs(g, dtype, roles, [24] * 8 + [8] * 8, M=3 * P, Df=64, seed=41, corr_K=24,
                             name=f"qk_S{S}_P{P}_{dtype}")
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch_dtype(w))
    h = 2
    say(f"qk index {w.name} head {h} mode {mode} K {K}")
    ctx.build_corr_index_qk(to_dev(w.q), to_dev(w.k), h, K, mode)
    gidx = ctx.get_corr_index().cpu().numpy()
    _check(w, h, gidx, np.arange(g.Np), K, mode)
    ctx.close()


def test_qk_index_layer_end_to_end():
    saf = _saf()
    g = Geometry(S=3, ns=5, P=300)
    roles = [ROLE_CORRESPONDENCE] * 6 + [ROLE_SCANNING] * 6 + [ROLE_POSITION] * 2 + [ROLE_DENSE] * 2
    w = make_geometry_inputs(g, "bf16", roles, [16] * 6 + [8] * 6 + [0] * 4, M=900, Df=64, seed=43, corr_K=16)
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    say("qk index end-to-end")
    ctx.build_corr_index_qk(q, k, 0, 16)
    o = ctx.sparse_attention(w.plan, q, k, v)
    torch.cuda.synchronize()
    gidx = ctx.get_corr_index().cpu().numpy()
    # every row passes the band rule; the oracle then evaluates attention on
    # the GPU's rows and every row of every head compares
    _check(w, 0, gidx, np.arange(g.Np), 16, 0)
    rows = np.arange(g.N)
    corr = {u: gidx[u].astype(np.int64) for u in range(g.Np)}
    outs, _, _ = oracle.layer(g, w.plan, w.q, w.k, w.v, w.dino, rows=rows, corr_rows=corr)
    got = to_host_f64(o)
    for h in outs:
        err = np.max(np.abs(got[h] - outs[h]))
        assert err <= tol(w), (h, err)
    ctx.close()
