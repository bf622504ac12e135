"""Pins for the oracle's offline head profiling (SAF3R Sec. 4.2, Eq. 1-2)."""
import types

import numpy as np
import pytest

import oracle
from oracle import profiling
from workload import Geometry, make_geometry_inputs, ROLE_CORRESPONDENCE, ROLE_DENSE, ROLE_POSITION, \
    ROLE_SCANNING, ROLE_VERTICAL


def test_nmse_definition():
    a = np.array([[1.0, 2.0], [3.0, 4.0]])
    assert profiling.nmse(a, a) == 0.0
    assert profiling.nmse(a, np.zeros_like(a)) == 1.0
    assert profiling.nmse(a, 0.25 * a) == pytest.approx(0.75 ** 2, abs=1e-15)
    b = np.array([[1.0, 0.0], [3.0, 4.0]])
    assert profiling.nmse(a, b) == pytest.approx(4.0 / 30.0, abs=1e-15)     # hand computed


@pytest.mark.parametrize("sigma,stride", [(0.0, 1), (0.5, 2), (0.75, 4), (0.85, 7), (0.9, 10), (0.97, 34)])
def test_baseline_stride(sigma, stride):
    s = profiling.baseline_stride(sigma)
    assert s == stride
    assert 1.0 / s <= 1.0 - sigma + 1e-12          # keeps at most 1 - sigma of the keys
    assert s == 1 or 1.0 / (s - 1) > 1.0 - sigma    # and is the smallest such stride


@pytest.mark.parametrize("cfg", [(ROLE_POSITION, 0, 0), (ROLE_POSITION, 0, 2), (ROLE_SCANNING, 3, 0),
                                 (ROLE_SCANNING, 7, 0), (ROLE_VERTICAL, 9, 0), (ROLE_VERTICAL, 10000, 0),
                                 (ROLE_CORRESPONDENCE, 5, 0), (ROLE_CORRESPONDENCE, 10000, 0),
                                 (ROLE_DENSE, 0, 0), (6, 0, 0), (6, 1, 5), (6, 2, 0), (6, 7, 5)])
def test_head_pairs_count_the_actual_key_sets(cfg):
    geom = Geometry(S=3, ns=2, P=10)
    w = make_geometry_inputs(geom, "f32", [ROLE_DENSE] * 16, [0] * 16, M=40, Df=16, seed=4)
    role, budget, anchor = cfg
    plan = [(role, budget, anchor, 0)] * 16
    sets, _, _ = oracle.layer_sets(geom, plan, w.q, w.k, w.v, w.dino, corr_K=budget)
    row_set, s = sets[0]
    brute = sum(len(np.unique(s[i])) for i in row_set)
    assert profiling.head_pairs(geom, cfg) == brute
    assert profiling.head_flops(geom, cfg) == 4 * geom.d * brute


def test_select_is_constrained_progressive_argmin():
    # entry 0 is the baseline
    assert profiling.select([0.5, 0.1, 0.3], [10, 20, 10]) == 2      # 1 is cheaper-error but too costly
    assert profiling.select([0.5, 0.5, 0.6], [10, 5, 5]) == 0        # ties keep the current choice
    assert profiling.select([0.5, 0.4, 0.2, 0.3], [10, 1, 10, 2]) == 2
    assert profiling.select([0.5], [10]) == 0


def _planted_sample():
    """Head 0: every query attends to keys 5, 20 and 30 (vertical lines).
    Head 1: patch p of frame 0 attends to patch p of frame 1 and back, and
    the DINO features (one-hot by patch position) rank exactly that pair
    first (correspondence).  Other heads: N(0, 1)."""
    g = Geometry(S=2, ns=1, P=16)
    rng = np.random.default_rng(0)
    H, N, d = g.H, g.N, g.d
    q = rng.standard_normal((H, N, d)).astype(np.float32)
    k = rng.standard_normal((H, N, d)).astype(np.float32)
    v = rng.standard_normal((H, N, d)).astype(np.float32)
    q[0] = 0.0
    q[0][:, 0] = 10.0
    k[0] = 0.1 * k[0]
    k[0][[5, 20, 30], 0] = 10.0
    q[1] = 0.0
    k[1] = 0.0
    for f in range(2):
        for p in range(16):
            t = f * g.T + g.ns + p
            q[1][t, (16 if f == 0 else 0) + p] = 10.0
            k[1][t, (0 if f == 0 else 16) + p] = 10.0
    dino = np.zeros((g.Np, 16), dtype=np.float32)
    dino[np.arange(g.Np), np.arange(g.Np) % 16] = 1.0
    return types.SimpleNamespace(geom=g, q=q, k=k, v=v, dino=dino)


def test_profile_recovers_planted_heads():
    w = _planted_sample()
    cands = [(ROLE_VERTICAL, 3, 0), (ROLE_CORRESPONDENCE, 1, 0), (ROLE_POSITION, 0, 0),
             (ROLE_SCANNING, 4, 0)]
    res = profiling.profile([w], cands, sigma=0.5)
    cfg = res["configs"]
    assert cfg[0] == (ROLE_SCANNING, 2, 0)
    assert cfg[res["choice"][0]] == (ROLE_VERTICAL, 3, 0)
    assert cfg[res["choice"][1]] == (ROLE_CORRESPONDENCE, 1, 0)
    assert res["errors"][0, 1] < 1e-6 and res["errors"][1, 2] < 1e-6
    # position (specials + frame 0 + own frame) costs more than stride 2 here
    assert res["costs"][3] > res["costs"][0]
    assert not np.any(res["choice"] == 3)
    for h in range(w.geom.H):
        c = res["choice"][h]
        assert res["costs"][c] <= res["costs"][0]
        assert res["errors"][h, c] <= res["errors"][h, 0]


def test_profile_averages_over_samples():
    g = Geometry(S=2, ns=1, P=12)
    ws = [make_geometry_inputs(g, "f32", [ROLE_VERTICAL] * 16, [4] * 16, M=30, Df=16, seed=s) for s in (1, 2)]
    cands = [(ROLE_VERTICAL, 4, 0)]
    both = profiling.profile(ws, cands, sigma=0.5)
    one = [profiling.profile([w], cands, sigma=0.5) for w in ws]
    np.testing.assert_allclose(both["errors"], 0.5 * (one[0]["errors"] + one[1]["errors"]), rtol=1e-12)
