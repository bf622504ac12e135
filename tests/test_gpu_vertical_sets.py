"""Vertical heads on both sides of the LDS staging limit of their key lists.

The matrix-core kernel stages a vertical head's key list (ascending token
ids) in LDS once per work-group when it holds at most 4,096 entries, and reads
it from memory per tile otherwise.  Budgets 4,095 / 4,096 / 4,097 / 4,200 /
5,000 / 6,000 and one above N (every key) on a geometry of 6,020 tokens, with
the sets built by the library's probe and top-K (checked by the band rule) and
the oracle evaluated on exactly those sets: every row compared (max-abs
2e-2), for the layer that builds its own sets and for the same sets handed in
by the caller."""
import numpy as np
import pytest
import torch

import oracle
from workload import Geometry, make_geometry_inputs, ROLE_DENSE, ROLE_VERTICAL

from helpers import band_check, say, to_dev, to_host_f64

pytestmark = pytest.mark.gpu


def _saf():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_wise_dynamic_amd as saf
    saf.lib()
    return saf


def test_vertical_lists_staged_and_read_per_tile():
    saf = _saf()
    g = Geometry(S=4, ns=5, P=1500)   # N = 6,020
    budgets_v = [4095, 4096, 4097, 5000, 64, 10 ** 6, 4200, 6000]   # 10^6: clamped to all N keys
    roles = [ROLE_VERTICAL] * 8 + [ROLE_DENSE] * 8
    budgets = budgets_v + [0] * 8
    w = make_geometry_inputs(g, "bf16", roles, budgets, M=3000, Df=32, seed=29, dino=False)
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    say(f"vertical sets around the staging limit, N={g.N}")
    o = ctx.sparse_attention(w.plan, q, k, v)
    sets = {h: ctx.build_vertical_index(q, k, h, budgets[h]).cpu().numpy().astype(np.int64) for h in range(8)}
    ld = max(ids.size for ids in sets.values())
    vt = torch.zeros((g.H, ld), dtype=torch.int32)
    for h, ids in sets.items():
        vt[h, :ids.size] = torch.from_numpy(ids.astype(np.int32))
    o2 = ctx.sparse_attention(w.plan, q, k, v, vert_idx=vt.cuda())
    torch.cuda.synchronize()
    got, got2 = to_host_f64(o), to_host_f64(o2)
    for h, ids in sets.items():
        _, r, _, _ = oracle.vertical_index(w.q[h], w.k[h], budgets[h])
        band_check(r, ids, budgets[h])
    rows = np.arange(g.N)
    outs, _, _ = oracle.layer(g, w.plan, w.q, w.k, w.v, None, rows=rows, heads=list(range(8)), vert_sets=sets)
    for h in range(8):
        for name, a in (("own sets", got), ("caller's sets", got2)):
            err = float(np.max(np.abs(a[h] - outs[h])))
            assert err <= 2e-2, f"{name}, head {h} (K = {budgets[h]}): max-abs {err:.3g}"
    ctx.close()
