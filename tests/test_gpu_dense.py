"""The dense attention kernel (every key, the speedup baseline) against the
oracle at shapes around its tiles: 256 queries per work-group, 64 keys per
tile.  Exactly one key tile, fewer keys than one tile, exact multiples of
both tiles, ragged in both, and the [N, H, d] layout; every row of four heads
is compared (max-abs 2e-2, bf16 inputs)."""
import numpy as np
import pytest
import torch

import oracle
from workload import Geometry, make_geometry_inputs, ROLE_DENSE

from helpers import say, to_dev, to_host_f64

pytestmark = pytest.mark.gpu


def _saf():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_wise_dynamic_amd as saf
    saf.lib()
    return saf


@pytest.mark.parametrize("S,ns,P,nhd", [
    (2, 0, 32, False),     # N = 64: one key tile, one partial query tile
    (1, 5, 20, False),     # N = 25: fewer keys than one tile
    (4, 5, 251, False),    # N = 1024: four query tiles, sixteen key tiles exactly
    (3, 3, 600, False),    # N = 1809: ragged queries and keys
    (3, 3, 600, True),     # the same in the [N, H, d] layout
    (2, 5, 1400, False),   # N = 2810: 44 key tiles with a ragged one, eleven query tiles
])
def test_dense_kernel_against_oracle(S, ns, P, nhd):
    saf = _saf()
    g = Geometry(S=S, ns=ns, P=P)
    w = make_geometry_inputs(g, "bf16", [ROLE_DENSE] * 16, [0] * 16, M=4 * P, Df=32, seed=13, dino=False)
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    if nhd:
        q, k, v = (t.transpose(0, 1).contiguous() for t in (q, k, v))
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
    say(f"dense kernel N={g.N} nhd={nhd}")
    o = ctx.dense_attention(q, k, v)
    torch.cuda.synchronize()
    got = to_host_f64(o.transpose(0, 1) if nhd else o)
    rows, keys = np.arange(g.N), np.arange(g.N)
    for h in (0, 5, 10, 15):
        ref = oracle.attention(w.q[h], w.k[h], w.v[h], rows, keys)
        err = float(np.max(np.abs(got[h] - ref)))
        assert err <= 2e-2, (h, err)
    ctx.close()
