"""Seeded sweep of small geometries and mixed plans, HIP path vs the oracle.

Each case draws a geometry (2-6 frames, 0-5 special tokens, 16-400 patches),
a dtype, and sixteen heads with roles and budgets drawn from every role the
library knows: position (any anchor), vertical (K from 1 to beyond N),
correspondence, scanning (strides from 1 to beyond N), dense, correspondence
united with a stride, broadcast (radius 0-5, grid width any divisor of P or
0).  The GPU runs with the oracle's vertical sets and correspondence index,
so every row of every head compares element-wise (max-abs 2e-2 bf16, 1e-4
fp32).

A second sweep builds the correspondence index itself on random geometries,
feature widths (multiples of 64 including the unrolled 384 / 768 / 1024, and
one off the matrix-core tiles), K up to 1024, both modes and both dtypes,
checked row by row against the oracle's scores with the band rule.
"""
import numpy as np
import pytest
import torch

import oracle
from workload import Geometry, make_geometry_inputs

from helpers import band_check, say, to_dev, to_host_f64, tol, torch_dtype

pytestmark = pytest.mark.gpu


def _saf():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_wise_dynamic_amd as saf
    saf.lib()
    return saf


def _draw(seed):
    rng = np.random.default_rng(7000 + seed)
    S, ns, P = int(rng.integers(2, 7)), int(rng.integers(0, 6)), int(rng.integers(16, 401))
    dtype = "bf16" if rng.random() < 0.6 else "f32"
    g = Geometry(S=S, ns=ns, P=P)
    N = g.N
    corr_K = int(rng.integers(1, min(64, (S - 1) * P) + 1))
    widths = [0] + [x for x in range(2, P + 1) if P % x == 0]
    roles, budgets, anchors = [], [], []
    for _ in range(16):
        r = int(rng.integers(0, 7))
        a = 0
        if r == 0:
            b, a = 0, int(rng.integers(0, S))
        elif r == 1:
            b = int(rng.integers(1, N + 10))
        elif r == 2:
            b = corr_K
        elif r == 3:
            b = int(rng.integers(1, N + 5))
        elif r == 4:
            b = 0
        elif r == 5:
            b = int(rng.integers(1, 50))
        else:
            b, a = int(rng.integers(0, 6)), int(rng.choice(widths))
        roles.append(r)
        budgets.append(b)
        anchors.append(a)
    w = make_geometry_inputs(g, dtype, roles, budgets, M=max(2 * P, 32), Df=64, seed=7000 + seed,
                             corr_K=corr_K, anchors=anchors, name=f"rand{seed}_S{S}_ns{ns}_P{P}_{dtype}")
    return w


@pytest.mark.parametrize("seed", range(48))
def test_random_plan_matches_oracle(seed):
    saf = _saf()
    w = _draw(seed)
    g = w.geom
    say(f"random plan {w.name}: roles {[p[0] for p in w.plan]}")
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch_dtype(w))
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    # the oracle's vertical sets, passed in
    vheads = [h for h, p in enumerate(w.plan) if p[0] == oracle.ROLE_VERTICAL]
    vt = None
    if vheads:
        ids = {h: oracle.vertical_index(w.q[h], w.k[h], w.plan[h][1])[0] for h in vheads}
        ld = max(len(x) for x in ids.values())
        arr = np.zeros((g.H, ld), dtype=np.int32)
        for h, x in ids.items():
            arr[h, :len(x)] = x
        vt = torch.from_numpy(arr).cuda()
    # the oracle's correspondence index, imported
    corr = None
    if any(p[0] in (oracle.ROLE_CORRESPONDENCE, oracle.ROLE_CORR_STRIDE) for p in w.plan):
        idx, _, _ = oracle.corr_index(w.dino, g.S, g.ns, g.P, w.corr_K, np.arange(g.Np))
        ctx.set_corr_index(torch.from_numpy(idx.astype(np.int32)).cuda())
        corr = {u: idx[u] for u in range(g.Np)}
    o = ctx.sparse_attention(w.plan, q, k, v, vert_idx=vt)
    torch.cuda.synchronize()
    rows = np.arange(g.N)
    outs, _, _ = oracle.layer(g, w.plan, w.q, w.k, w.v, w.dino, corr_K=w.corr_K, rows=rows, corr_rows=corr)
    got = to_host_f64(o)
    for h, ref in outs.items():
        err = np.max(np.abs(got[h][rows] - ref))
        assert err <= tol(w), (h, w.plan[h], err)
    ctx.close()


@pytest.mark.parametrize("seed", range(16))
def test_random_index_matches_oracle(seed):
    saf = _saf()
    rng = np.random.default_rng(9000 + seed)
    S, ns, P = int(rng.integers(2, 7)), int(rng.integers(0, 6)), int(rng.integers(16, 401))
    dtype = "bf16" if rng.random() < 0.7 else "f32"
    Df = int(rng.choice([64, 128, 192, 384, 768, 1024, 96]))
    mode = saf.SAF_CORR_PER_FRAME if rng.random() < 0.3 else saf.SAF_CORR_TOTAL
    g = Geometry(S=S, ns=ns, P=P)
    cand = P if mode == saf.SAF_CORR_PER_FRAME else (S - 1) * P
    K = int(rng.integers(1, min(1024, cand) + 1))
    w = make_geometry_inputs(g, dtype, [oracle.ROLE_CORRESPONDENCE] * 16, [K] * 16, M=max(2 * P, 32), Df=Df,
                             seed=9000 + seed, corr_K=K, name=f"ridx{seed}_S{S}_P{P}_Df{Df}_{dtype}")
    say(f"random index {w.name} K {K} mode {mode}")
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch_dtype(w))
    ctx.build_corr_index(to_dev(w.dino), K, mode=mode)
    got = ctx.get_corr_index().cpu().numpy()
    sc = oracle.corr_scores(w.dino, g.S, g.P, np.arange(g.Np))
    frame = np.arange(g.Np) // g.P
    for u in range(g.Np):
        assert np.all(got[u] % g.T >= g.ns), u
        gp = (got[u] // g.T) * g.P + got[u] % g.T - g.ns
        if mode == saf.SAF_CORR_TOTAL:
            band_check(np.nan_to_num(sc[u], nan=-np.inf), gp, K, valid=frame != frame[u])
        else:
            kf = min(K, g.P)
            for f in range(g.S):
                if f == frame[u]:
                    continue
                slot = f - (f > frame[u])
                seg = got[u, slot * kf:(slot + 1) * kf]
                assert np.all(seg // g.T == f), (u, f)
                band_check(sc[u, f * g.P:(f + 1) * g.P], seg % g.T - g.ns, kf)
    ctx.close()
