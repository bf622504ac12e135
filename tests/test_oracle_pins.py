"""Pins of the CPU oracle against things other than itself.

Each check below would fail on a plausible slip in the oracle (a dropped term,
a wrong sign or index, a transposed operand, a set with repeats, a wrong tie
order): brute force with library routines (numpy, scipy, torch CPU), closed
forms, printed values from the pages, and invariants of softmax attention.
"""
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from workload import (Geometry, bf16_round, bf16_to_f32, make_geometry_inputs, make_inputs,
                      ROLE_CORRESPONDENCE, ROLE_POSITION, ROLE_SCANNING, ROLE_VERTICAL)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def _masked_dense(q, k, v, mask):
    """Brute force: dense softmax(QK^T/sqrt(d) + M) V with -inf outside the set."""
    q64, k64, v64 = (np.asarray(a, np.float64) for a in (q, k, v))
    logits = q64 @ k64.T / math.sqrt(q.shape[1])
    logits = np.where(mask, logits, -np.inf)
    return scipy.special.softmax(logits, axis=1) @ v64


# ---------------------------------------------------------------- attention
def test_attention_matches_masked_dense_softmax():
    N, d = 300, 64
    q, k, v = _rand((N, d), 1), _rand((N, d), 2), _rand((N, d), 3)
    rng = np.random.default_rng(4)
    rows = np.sort(rng.choice(N, 40, replace=False))
    sets = [np.sort(rng.choice(N, rng.integers(1, N), replace=False)) for _ in range(7)]
    row_set = rng.integers(0, len(sets), rows.size)
    got = oracle.attention_sets(q, k, v, rows, row_set, sets)
    mask = np.zeros((rows.size, N), dtype=bool)
    for r, s in enumerate(row_set):
        mask[r, sets[s]] = True
    want = _masked_dense(q[rows], k, v, mask)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    # torch CPU scaled-dot-product attention (float64, boolean mask)
    tq = torch.from_numpy(q[rows].astype(np.float64))[None]
    tk = torch.from_numpy(k.astype(np.float64))[None]
    tv = torch.from_numpy(v.astype(np.float64))[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(mask)[None])
    np.testing.assert_allclose(got, ref[0].numpy(), rtol=0, atol=1e-12)


def test_attention_bf16_decodes_exactly():
    N, d = 200, 64
    qf, kf, vf = _rand((N, d), 5), _rand((N, d), 6), _rand((N, d), 7)
    qb, kb, vb = bf16_round(qf), bf16_round(kf), bf16_round(vf)
    keys = np.arange(0, N, 3)
    rows = np.arange(N)
    got = oracle.attention(qb, kb, vb, rows, keys)
    mask = np.zeros((N, N), dtype=bool)
    mask[:, keys] = True
    want = _masked_dense(bf16_to_f32(qb), bf16_to_f32(kb), bf16_to_f32(vb), mask)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_attention_special_cases():
    N, d = 128, 64
    q, k, v = _rand((N, d), 8), _rand((N, d), 9), _rand((N, d), 10)
    rows = np.arange(N)
    # one key: the output is that value row exactly
    got = oracle.attention(q, k, v, rows, [37])
    np.testing.assert_array_equal(got, np.broadcast_to(v[37].astype(np.float64), got.shape))
    # all logits equal (zero query): the mean of V over the set
    keys = np.array([3, 5, 8, 13, 21, 34, 55, 89])
    got = oracle.attention(np.zeros_like(q), k, v, rows, keys)
    np.testing.assert_allclose(got, np.broadcast_to(v[keys].astype(np.float64).mean(0), got.shape),
                               rtol=0, atol=1e-15)
    # every key: plain dense attention (torch, no mask)
    got = oracle.attention(q, k, v, rows, np.arange(N))
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(a.astype(np.float64))[None] for a in (q, k, v)))[0].numpy()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    # the order of the keys in the set does not matter
    keys = np.random.default_rng(11).choice(N, 50, replace=False)
    a = oracle.attention(q, k, v, rows, np.sort(keys))
    b = oracle.attention(q, k, v, rows, keys)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_attention_large_logits_are_stable():
    N, d = 64, 64
    q, k, v = _rand((N, d), 12, 30.0), _rand((N, d), 13, 30.0), _rand((N, d), 14)
    got = oracle.attention(q, k, v, np.arange(N), np.arange(N))
    assert np.all(np.isfinite(got))
    want = _masked_dense(q, k, v, np.ones((N, N), dtype=bool))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-10)


# ------------------------------------------------------------ static sets
@pytest.mark.parametrize("S,ns,P,anchor", [(4, 5, 256, 0), (3, 5, 7, 2), (5, 0, 11, 1), (1, 5, 9, 0)])
def test_position_set_brute_force_and_size(S, ns, P, anchor):
    T = ns + P
    N = S * T
    j = np.arange(N)
    for f in range(S):
        want = j[((j % T) < ns) | (j // T == anchor) | (j // T == f)]
        got = oracle.position_set(S, ns, P, anchor, f)
        np.testing.assert_array_equal(got, want)
        assert len(np.unique(got)) == len(got)
        assert len(got) == (ns * S + 2 * P if f != anchor else ns * S + P)


@pytest.mark.parametrize("S,ns,P,s", [(4, 5, 256, 8), (100, 5, 1369, 16), (32, 5, 1369, 16),
                                      (500, 5, 1296, 32), (3, 0, 10, 4), (6, 5, 3, 7)])
def test_scan_set_closed_form(S, ns, P, s):
    T = ns + P
    N = S * T
    got = oracle.scan_set(S, ns, P, s)
    on_stride = -(-N // s)
    specials_on_stride = sum(1 for f in range(S) for t in range(ns) if (f * T + t) % s == 0)
    assert len(got) == on_stride + ns * S - specials_on_stride
    assert np.all(np.diff(got) > 0)
    j = np.arange(N)
    np.testing.assert_array_equal(got, j[(j % s == 0) | (j % T < ns)])


def test_scan_set_size_at_measured_configs():
    # |scan| at the tiny config (S=4, stride 8) and the S=100 config (stride 16)
    assert len(oracle.scan_set(4, 5, 256, 8)) == 148
    assert len(oracle.scan_set(100, 5, 1369, 16)) == 9049


def _golden_rows():
    rows = []
    with open(os.path.join(GOLDEN, "table6_keys.txt")) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if line:
                kind, param, pct = line.split()
                rows.append((kind, int(param), float(pct)))
    return rows


@pytest.mark.parametrize("kind,param,pct", _golden_rows())
def test_table6_keys_column(kind, param, pct):
    """Printed #Keys fractions (Table 6/7) from the oracle's own key sets."""
    S, ns, P = 128, 0, 1036
    N = S * (ns + P)
    if kind == "full":
        frac = N / N
    elif kind == "skip":
        frac = 0.0
    elif kind == "uniform_stride":
        frac = len(oracle.scan_set(S, ns, P, param)) / N
    else:
        F = _rand((S * P, 4), 15)
        idx, _, _ = oracle.corr_index(F, S, ns, P, param, [0], mode=oracle.MODE_PER_FRAME)
        assert len(np.unique(idx[0])) == idx.shape[1] == (S - 1) * param
        frac = idx.shape[1] / N
    assert round(100 * frac, 1) == pytest.approx(pct, abs=1e-9)


# ---------------------------------------------------------------- top-K
def test_topk_ties_take_lower_index_and_output_is_ascending():
    scores = np.array([0.5, 0.9, 0.5, 0.1, 0.9, 0.5, -1.0])
    ids, kth, nxt = oracle.topk(scores, 4)
    np.testing.assert_array_equal(ids, [0, 1, 2, 4])
    assert kth == 0.5 and nxt == 0.5
    ids, kth, nxt = oracle.topk(scores, 100)
    np.testing.assert_array_equal(ids, np.arange(7))
    assert nxt == -np.inf
    # agrees with a stable argsort on random data with many repeats
    r = np.random.default_rng(16).integers(0, 50, 1000).astype(np.float64)
    want = np.sort(np.argsort(-r, kind="stable")[:137])
    np.testing.assert_array_equal(oracle.topk(r, 137)[0], want)


# ---------------------------------------------------------------- vertical probe
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_probe_equals_column_mean_of_scores(dtype):
    N, d = 700, 64
    q, k = _rand((N, d), 17), _rand((N, d), 18)
    if dtype == "bf16":
        q, k = bf16_round(q), bf16_round(k)
        qf, kf = bf16_to_f32(q), bf16_to_f32(k)
    else:
        qf, kf = q, k
    qbar = oracle.mean_query(q)
    np.testing.assert_allclose(qbar, qf.astype(np.float64).mean(0), rtol=0, atol=1e-15)
    r = oracle.probe_scores(k, qbar)
    full = qf.astype(np.float64) @ kf.astype(np.float64).T / math.sqrt(d)   # N x N
    colmean = full.mean(axis=0)
    np.testing.assert_allclose(r, colmean, rtol=0, atol=1e-12)
    ids, _, _, _ = oracle.vertical_index(q, k, 64)
    np.testing.assert_array_equal(ids, np.sort(np.argsort(-colmean, kind="stable")[:64]))
    # budget >= N keeps every key
    ids_all, _, _, _ = oracle.vertical_index(q, k, N + 5)
    np.testing.assert_array_equal(ids_all, np.arange(N))


def test_probe_recovers_planted_salient_keys():
    w = make_inputs(1, dino=False)
    for h in w.heads(ROLE_VERTICAL):
        ids, _, _, _ = oracle.vertical_index(w.q[h], w.k[h], w.plan[h][1])
        # a salient key scores ~ (4 +- 1)/8 against ~N(0, 1/8^2) for the rest, so
        # only a rare one falls below the 64th score
        assert len(set(w.salient[h]) & set(ids)) >= 20


# ---------------------------------------------------------------- correspondence
def _brute_corr(F, S, ns, P, K, mode):
    Ff = F.astype(np.float64) if F.dtype == np.float32 else bf16_to_f32(F).astype(np.float64)
    n = np.linalg.norm(Ff, axis=1)
    cos = (Ff @ Ff.T) / np.outer(n, n)
    frame = np.arange(S * P) // P
    tok = frame * (ns + P) + ns + np.arange(S * P) % P
    rows = []
    for u in range(S * P):
        if mode == oracle.MODE_TOTAL:
            cand = np.nonzero(frame != frame[u])[0]
            order = np.lexsort((tok[cand], -cos[u, cand]))
            rows.append(np.sort(tok[cand[order[:K]]]))
        else:
            sel = []
            for g in range(S):
                if g == frame[u]:
                    continue
                cand = np.nonzero(frame == g)[0]
                order = np.lexsort((tok[cand], -cos[u, cand]))
                sel.append(tok[cand[order[:K]]])
            rows.append(np.sort(np.concatenate(sel)))
    return np.array(rows), cos


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", [oracle.MODE_TOTAL, oracle.MODE_PER_FRAME])
def test_corr_index_matches_brute_force(dtype, mode):
    geom = Geometry(S=4, ns=5, P=30)
    w = make_geometry_inputs(geom, dtype, [ROLE_CORRESPONDENCE] * 16, [8] * 16, M=80, Df=48, seed=3)
    want, cos = _brute_corr(w.dino, geom.S, geom.ns, geom.P, 8, mode)
    got, tau, _ = oracle.corr_index(w.dino, geom.S, geom.ns, geom.P, 8, np.arange(geom.Np), mode)
    np.testing.assert_array_equal(got, want)
    sc = oracle.corr_scores(w.dino, geom.S, geom.P, [0, 31, 119])
    for r, u in enumerate([0, 31, 119]):
        same = (np.arange(geom.Np) // geom.P) == u // geom.P
        assert np.all(np.isnan(sc[r, same]))
        np.testing.assert_allclose(sc[r, ~same], cos[u, ~same], rtol=0, atol=1e-12)


def test_corr_index_budget_clamps_to_candidates():
    geom = Geometry(S=3, ns=5, P=6)
    F = _rand((geom.Np, 16), 19)
    got, _, _ = oracle.corr_index(F, 3, 5, 6, 1000, np.arange(geom.Np))
    assert got.shape == (geom.Np, 12)
    for u in range(geom.Np):
        f = u // 6
        want = [g * geom.T + 5 + p for g in range(3) if g != f for p in range(6)]
        np.testing.assert_array_equal(got[u], want)


def test_corr_generator_closed_form():
    """Same-latent DINO pairs have cosine ~ 1/(1 + 0.3^2); the copies rank first."""
    w = make_inputs(1)
    geom = w.geom
    rows = np.arange(0, geom.Np, 17)
    sc = oracle.corr_scores(w.dino, geom.S, geom.P, rows)
    idx, _, _ = oracle.corr_index(w.dino, geom.S, geom.ns, geom.P, w.corr_K, rows)
    same_cos = []
    for r, u in enumerate(rows):
        copies = np.nonzero((w.lat == w.lat[u]) & (np.arange(geom.Np) // geom.P != u // geom.P))[0]
        same_cos.extend(sc[r, copies])
        if 0 < copies.size <= w.corr_K:
            assert set(geom.patch_token(copies)).issubset(set(idx[r]))
    assert abs(np.mean(same_cos) - 1 / 1.09) < 0.01


def test_generator_is_deterministic_and_bf16_is_rne():
    a = make_geometry_inputs(Geometry(S=2, ns=5, P=8), "bf16", [ROLE_POSITION] * 16, [0] * 16, 40, 16, seed=9)
    b = make_geometry_inputs(Geometry(S=2, ns=5, P=8), "bf16", [ROLE_POSITION] * 16, [0] * 16, 40, 16, seed=9)
    np.testing.assert_array_equal(a.q, b.q)
    np.testing.assert_array_equal(a.dino, b.dino)
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5], dtype=np.float32)   # ties to even
    np.testing.assert_array_equal(bf16_to_f32(bf16_round(x)), [1.0, 1.0, 1.015625, -2.5])


# ---------------------------------------------------------------- layer
def test_layer_with_every_key_equals_dense():
    """A vertical budget >= N, a stride of 1 and the dense role all give dense attention."""
    geom = Geometry(S=3, ns=5, P=20)
    w = make_geometry_inputs(geom, "f32", [ROLE_VERTICAL, ROLE_SCANNING, 4] + [ROLE_POSITION] * 13,
                             [10 ** 6, 1, 0] + [0] * 13, M=80, Df=16, seed=21)
    outs, _, _ = oracle.layer(geom, w.plan, w.q, w.k, w.v, heads=[0, 1, 2])
    for h in (0, 1, 2):
        want = _masked_dense(w.q[h], w.k[h], w.v[h], np.ones((geom.N, geom.N), dtype=bool))
        np.testing.assert_allclose(outs[h], want, rtol=0, atol=1e-12)


def test_layer_position_heads_against_brute_force_mask():
    geom = Geometry(S=3, ns=5, P=20)
    w = make_geometry_inputs(geom, "f32", [ROLE_POSITION] * 16, [0] * 16, M=80, Df=16, seed=22,
                             anchors=[1] * 16)
    outs, _, _ = oracle.layer(geom, w.plan, w.q, w.k, w.v, heads=[0])
    j = np.arange(geom.N)
    f, t = j // geom.T, j % geom.T
    mask = (t[None, :] < geom.ns) | (f[None, :] == 1) | (f[None, :] == f[:, None])
    want = _masked_dense(w.q[0], w.k[0], w.v[0], mask)
    np.testing.assert_allclose(outs[0], want, rtol=0, atol=1e-12)


def test_layer_corr_heads_specials_attend_everything():
    geom = Geometry(S=3, ns=5, P=20)
    w = make_geometry_inputs(geom, "f32", [ROLE_CORRESPONDENCE] * 16, [6] * 16, M=80, Df=16, seed=23,
                             corr_K=6)
    outs, corr, _ = oracle.layer(geom, w.plan, w.q, w.k, w.v, w.dino, corr_K=6, heads=[0])
    want_idx, _ = _brute_corr(w.dino, geom.S, geom.ns, geom.P, 6, oracle.MODE_TOTAL)
    j = np.arange(geom.N)
    mask = np.zeros((geom.N, geom.N), dtype=bool)
    for i in j:
        if i % geom.T < geom.ns:
            mask[i, :] = True
        else:
            u = (i // geom.T) * geom.P + i % geom.T - geom.ns
            mask[i, want_idx[u]] = True
    want = _masked_dense(w.q[0], w.k[0], w.v[0], mask)
    np.testing.assert_allclose(outs[0], want, rtol=0, atol=1e-12)


# ---- block-wise DINO similarity (Sec. 4.3 "block-wise implementation")
@pytest.mark.parametrize("mode", [oracle.MODE_TOTAL, oracle.MODE_PER_FRAME])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_index_with_one_patch_blocks_is_the_token_index(mode, dtype):
    geom = Geometry(S=4, ns=5, P=30)
    w = make_geometry_inputs(geom, dtype, [ROLE_CORRESPONDENCE] * 16, [8] * 16, M=80, Df=48, seed=5)
    rows = np.arange(geom.Np)
    want, _, _ = oracle.corr_index(w.dino, geom.S, geom.ns, geom.P, 8, rows, mode)
    got, _ = oracle.block_corr_index(w.dino, geom.S, geom.ns, geom.P, 1, 8, rows, mode)
    np.testing.assert_array_equal(got, want)


def test_block_scores_equal_dot_of_mean_unit_vectors():
    # mean over a x b pairs of u.v/(|u||v|) = (mean of unit u) . (mean of unit v)
    S, P, b, Df = 3, 12, 4, 20
    F = _rand((S * P, Df), 23)
    F[5] = 0.0                        # a zero feature contributes cosine 0
    F64 = F.astype(np.float64)
    n = np.linalg.norm(F64, axis=1)
    U = np.divide(F64, n[:, None], out=np.zeros_like(F64), where=n[:, None] > 0)
    M = U.reshape(S * P // b, b, Df).mean(axis=1)
    sc = oracle.block_scores(F, S, P, b, np.arange(S * P // b))
    want = M @ M.T
    per = P // b
    own = (np.arange(S * per)[:, None] // per) == (np.arange(S * per)[None, :] // per)
    assert np.all(np.isnan(sc[own]))
    np.testing.assert_allclose(sc[~own], want[~own], rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode", [oracle.MODE_TOTAL, oracle.MODE_PER_FRAME])
def test_block_index_recovers_planted_block_matches(mode):
    # one-hot features: block j of frame 0 is e_j in all its patches; block k
    # of frame 1 is e_perm[k].  The only block of frame 1 with similarity 1 to
    # frame-0 block j is perm^-1(j); everything else scores 0 against it.
    S, ns, P, b = 2, 3, 24, 6
    per = P // b
    perm = np.array([2, 0, 3, 1])
    F = np.zeros((S * P, 8), dtype=np.float32)
    for j in range(per):
        F[j * b:(j + 1) * b, j] = 1.0
        F[P + j * b:P + (j + 1) * b, perm[j]] = 1.0
    rows = np.arange(S * P)
    got, sel = oracle.block_corr_index(F, S, ns, P, b, 1, rows, mode)
    T = ns + P
    for j in range(per):
        k = int(np.where(perm == j)[0][0])            # frame-1 block holding e_j
        assert sel[j][0].tolist() == [per + k]
        assert sel[per + k][0].tolist() == [j]
        want = [T + ns + k * b + i for i in range(b)]
        for u in range(j * b, (j + 1) * b):
            assert got[u].tolist() == want


def test_block_index_shares_sets_within_a_block_and_clamps():
    geom = Geometry(S=5, ns=2, P=16)
    w = make_geometry_inputs(geom, "f32", [ROLE_CORRESPONDENCE] * 16, [8] * 16, M=40, Df=24, seed=8)
    rows = np.arange(geom.Np)
    got, _ = oracle.block_corr_index(w.dino, 5, 2, 16, 4, 3, rows)
    assert got.shape == (geom.Np, 12)
    for u in rows:
        np.testing.assert_array_equal(got[u], got[(u // 4) * 4])
        assert np.all(np.diff(got[u]) > 0)
        assert np.all(got[u] // geom.T != u // 16)            # other frames only
    pf, _ = oracle.block_corr_index(w.dino, 5, 2, 16, 4, 100, rows, oracle.MODE_PER_FRAME)
    assert pf.shape == (geom.Np, 4 * 16)                       # clamps to every other patch
    with pytest.raises(ValueError):
        oracle.block_corr_index(w.dino, 5, 2, 16, 3, 3, rows)


# ---- correspondence top-K united with the stride set
def test_corr_stride_sets_are_the_union():
    geom = Geometry(S=3, ns=2, P=20)
    w = make_geometry_inputs(geom, "f32", [ROLE_CORRESPONDENCE] * 16, [6] * 16, M=50, Df=16, seed=12)
    idx, _, _ = oracle.corr_index(w.dino, 3, 2, 20, 6, np.arange(geom.Np))
    for s in (1, 4, 7, 10 ** 6):
        plan = [(oracle.ROLE_CORR_STRIDE, s, 0, 0)] * 16
        sets, _, _ = oracle.layer_sets(geom, plan, w.q, w.k, w.v, w.dino, corr_K=6)
        row_set, ss = sets[0]
        scan = {j for j in range(geom.N) if j % s == 0} | {f * geom.T + t for f in range(3) for t in range(2)}
        for i in range(geom.N):
            got = ss[row_set[i]]
            if i % geom.T < 2:
                assert len(got) == geom.N                      # special queries: every key
                continue
            u = (i // geom.T) * 20 + i % geom.T - 2
            want = sorted(scan | set(idx[u].tolist()))
            assert got.tolist() == want
            assert len(got) == len(scan) + len(set(idx[u].tolist()) - scan)


def test_corr_stride_with_stride_one_is_dense():
    geom = Geometry(S=2, ns=1, P=12)
    w = make_geometry_inputs(geom, "f32", [ROLE_CORRESPONDENCE] * 16, [4] * 16, M=30, Df=16, seed=13)
    u_plan = [(oracle.ROLE_CORR_STRIDE, 1, 0, 0)] * 16
    d_plan = [(oracle.ROLE_DENSE, 0, 0, 0)] * 16
    a, _, _ = oracle.layer(geom, u_plan, w.q, w.k, w.v, w.dino, corr_K=4)
    b, _, _ = oracle.layer(geom, d_plan, w.q, w.k, w.v)
    for h in range(16):
        np.testing.assert_allclose(a[h], b[h], rtol=0, atol=1e-14)


# ---- correspondence index from one head's logits
@pytest.mark.parametrize("mode", [oracle.MODE_TOTAL, oracle.MODE_PER_FRAME])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_qk_index_matches_brute_force(mode, dtype):
    S, ns, P, d, K = 3, 2, 14, 16, 5
    T, N = ns + P, S * (ns + P)
    rng = np.random.default_rng(21)
    q = rng.standard_normal((N, d)).astype(np.float32)
    k = rng.standard_normal((N, d)).astype(np.float32)
    k[[T + ns + 3, 2 * T + ns + 3]] = k[ns + 3]              # exact ties between frames
    if dtype == "bf16":
        q, k = bf16_round(q), bf16_round(k)
        qf, kf = bf16_to_f32(q).astype(np.float64), bf16_to_f32(k).astype(np.float64)
    else:
        qf, kf = q.astype(np.float64), k.astype(np.float64)
    got, _ = oracle.qk_index(q, k, S, ns, P, K, np.arange(S * P), mode)
    tok = np.array([(v // P) * T + ns + v % P for v in range(S * P)])
    for u in range(S * P):
        fu = u // P
        s = kf[tok] @ qf[tok[u]]
        if mode == oracle.MODE_TOTAL:
            cand = [v for v in range(S * P) if v // P != fu]
            order = sorted(cand, key=lambda v: (-s[v], tok[v]))[:K]
        else:
            order = []
            for f in range(S):
                if f != fu:
                    order += sorted(range(f * P, (f + 1) * P), key=lambda v: (-s[v], tok[v]))[:K]
        np.testing.assert_array_equal(got[u], np.sort(tok[order]))


def test_qk_index_on_unit_features_is_the_cosine_index():
    # with Q = K = the unit-normalised features, q.k is the cosine; one-hot
    # features with distinct magnitudes keep every ranking free of near-ties
    S, ns, P = 3, 1, 8
    T, N = ns + P, S * (ns + P)
    F = np.zeros((S * P, 8), dtype=np.float32)
    for v in range(S * P):
        F[v, v % 8] = 1.0 + 0.1 * (v // 8)
        F[v, (v + 3) % 8] = 0.5
    rng = np.random.default_rng(3)
    F += 0.01 * rng.standard_normal(F.shape).astype(np.float32)
    U = (F / np.linalg.norm(F, axis=1, keepdims=True)).astype(np.float32)
    q = np.zeros((N, 8), dtype=np.float32)
    tok = np.array([(v // P) * T + ns + v % P for v in range(S * P)])
    q[tok] = U
    want, _, _ = oracle.corr_index(F, S, ns, P, 4, np.arange(S * P))
    got, _ = oracle.qk_index(q, q, S, ns, P, 4, np.arange(S * P))
    np.testing.assert_array_equal(got, want)


# ---- static broadcast of a local window (Sec. 4.1 "Static Kernel")
def _bcast_mask(geom, radius, grid_w):
    """Brute force over token pairs: patch query (f, p) sees token (f', p') iff
    p' is within `radius` of p on the grid (or along the patch index), in any
    frame; every special token; special queries see everything."""
    T, ns = geom.T, geom.ns
    j = np.arange(geom.N)
    t = j % T
    sp = t < ns
    p = t - ns
    if grid_w > 0:
        dy = np.abs(p[:, None] // grid_w - p[None, :] // grid_w)
        dx = np.abs(p[:, None] % grid_w - p[None, :] % grid_w)
        near = (dy <= radius) & (dx <= radius)
    else:
        near = np.abs(p[:, None] - p[None, :]) <= radius
    return sp[:, None] | sp[None, :] | near


@pytest.mark.parametrize("S,ns,P", [(3, 2, 12), (1, 0, 7), (4, 5, 20)])
@pytest.mark.parametrize("grid_w", [0, 1, 4])
def test_broadcast_radius_zero_is_the_same_position_in_every_frame(S, ns, P, grid_w):
    if grid_w and P % grid_w:
        pytest.skip("grid width must divide P")
    T = ns + P
    for p in range(P):
        want = sorted([f * T + t for f in range(S) for t in range(ns)] + [f * T + ns + p for f in range(S)])
        np.testing.assert_array_equal(oracle.broadcast_set(S, ns, P, 0, grid_w, p), want)


def test_broadcast_window_sizes_closed_form():
    S, ns, P, gw = 3, 2, 20, 5          # a 4 x 5 grid
    size = lambda r, p, g=gw: oracle.broadcast_set(S, ns, P, r, g, p).size - ns * S
    assert size(1, 0) == S * 4          # corner: 2 x 2
    assert size(1, 2) == S * 6          # top edge: 2 x 3
    assert size(1, 6) == S * 9          # interior: 3 x 3
    assert size(2, 12) == S * 4 * 5     # rows 0..3, columns 0..4: the whole grid
    assert size(0, 13) == S
    assert size(2, 0, 0) == S * 3       # along the index: 0..2
    assert size(2, 10, 0) == S * 5      # 8..12
    assert size(3, 19, 0) == S * 4      # 16..19


def test_broadcast_window_moves_with_the_query():
    S, ns, P, gw = 2, 1, 30, 6          # a 5 x 6 grid
    T = ns + P
    a = oracle.broadcast_set(S, ns, P, 1, gw, 8)   # (1, 2)
    b = oracle.broadcast_set(S, ns, P, 1, gw, 9)   # (1, 3): one column right
    c = oracle.broadcast_set(S, ns, P, 1, gw, 14)  # (2, 2): one row down
    pa, pb, pc = (x[x % T >= ns] for x in (a, b, c))
    np.testing.assert_array_equal(pb, pa + 1)
    np.testing.assert_array_equal(pc, pa + gw)


@pytest.mark.parametrize("radius,grid_w", [(0, 0), (1, 4), (2, 0), (1, 5)])
def test_layer_broadcast_heads_against_brute_force_mask(radius, grid_w):
    geom = Geometry(S=3, ns=2, P=20)
    w = make_geometry_inputs(geom, "f32", [oracle.ROLE_BROADCAST] * 16, [radius] * 16, M=80, Df=16,
                             seed=31, anchors=[grid_w] * 16)
    outs, _, _ = oracle.layer(geom, w.plan, w.q, w.k, w.v, heads=[0, 5])
    mask = _bcast_mask(geom, radius, grid_w)
    for h in (0, 5):
        want = _masked_dense(w.q[h], w.k[h], w.v[h], mask)
        np.testing.assert_allclose(outs[h], want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("radius,grid_w", [(4, 5), (19, 0)])
def test_broadcast_covering_window_is_dense(radius, grid_w):
    geom = Geometry(S=3, ns=5, P=20)
    w = make_geometry_inputs(geom, "f32", [oracle.ROLE_BROADCAST] * 16, [radius] * 16, M=80, Df=16, seed=32,
                             anchors=[grid_w] * 16)
    outs, _, _ = oracle.layer(geom, w.plan, w.q, w.k, w.v, heads=[0])
    want = _masked_dense(w.q[0], w.k[0], w.v[0], np.ones((geom.N, geom.N), dtype=bool))
    np.testing.assert_allclose(outs[0], want, rtol=0, atol=1e-12)
