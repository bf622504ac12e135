"""Scanning heads with their key set packed into contiguous rows, and without.

A bf16 scanning set (the stride tokens, then the special tokens off the
stride) is gathered once per layer into contiguous K and V rows when the
geometry has at most 4,096 special tokens; beyond that the matrix-core kernel
enumerates the set per tile and masks the specials already on the stride.
Both sides of that limit, with strides that put no, some and every special on
the stride, are compared with the oracle on every row (max-abs 2e-2)."""
import numpy as np
import pytest
import torch

import oracle
from workload import Geometry, make_geometry_inputs, ROLE_POSITION, ROLE_SCANNING

from helpers import say, to_dev, to_host_f64

pytestmark = pytest.mark.gpu


def _saf():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_wise_dynamic_amd as saf
    saf.lib()
    return saf


@pytest.mark.parametrize("S,ns,P", [
    (819, 5, 16),   # 4,095 specials: packed
    (821, 5, 16),   # 4,105 specials: enumerated per tile
    (7, 3, 200),    # a few specials, packed
])
def test_scanning_sets_packed_and_enumerated(S, ns, P):
    saf = _saf()
    g = Geometry(S=S, ns=ns, P=P)
    # strides: 1 (every special on the stride), T (the first special of every
    # frame), 7, 64 and beyond N (only token 0 and the specials off it)
    strides = [1, g.T, 7, 64, g.N + 3, 16, 5, 1000]
    roles = [ROLE_SCANNING] * 8 + [ROLE_POSITION] * 8
    budgets = strides + [0] * 8
    w = make_geometry_inputs(g, "bf16", roles, budgets, M=4 * P, Df=32, seed=17, dino=False)
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
    say(f"scanning sets S={S} ns={ns} P={P} N={g.N} specials={ns * S}")
    o = ctx.sparse_attention(w.plan, to_dev(w.q), to_dev(w.k), to_dev(w.v))
    torch.cuda.synchronize()
    got = to_host_f64(o)
    rows = np.arange(g.N) if g.N <= 3000 else np.unique(np.concatenate([
        np.arange(0, 600), np.arange(g.N - 600, g.N), np.random.default_rng(3).integers(0, g.N, 1500)]))
    heads = [0, 1, 2, 3, 4, 5, 6, 7, 8]
    outs, _, _ = oracle.layer(g, w.plan, w.q, w.k, w.v, None, rows=rows, heads=heads)
    for h in heads:
        err = float(np.max(np.abs(got[h][rows] - outs[h])))
        assert err <= 2e-2, f"head {h} (stride {budgets[h]}): max-abs {err:.3g}"
    ctx.close()
