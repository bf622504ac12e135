"""A failed index rebuild leaves the cached index intact (GPU).

The allocation hook makes the rebuild's allocations fail at each step a
rebuild allocates (the index buffer, the build scratch, the second of the
two); the call must return SAF_ENOMEM, and the previously built index must
keep its row length and contents and still serve a layer bit for bit.
"""
import numpy as np
import pytest
import torch

from workload import Geometry, make_geometry_inputs, ROLE_CORRESPONDENCE, ROLE_SCANNING, ROLE_VERTICAL

from helpers import say, to_dev

pytestmark = pytest.mark.gpu


def _saf():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_wise_dynamic_amd as saf
    saf.lib()
    return saf


def test_failed_rebuild_keeps_the_cached_index():
    saf = _saf()
    g = Geometry(S=3, ns=5, P=300)
    roles = [ROLE_CORRESPONDENCE] * 4 + [ROLE_SCANNING] * 8 + [ROLE_VERTICAL] * 4
    w = make_geometry_inputs(g, "bf16", roles, [24] * 4 + [8] * 8 + [64] * 4, M=900, Df=64, seed=17, corr_K=24)
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
    q, k, v, dino = to_dev(w.q), to_dev(w.k), to_dev(w.v), to_dev(w.dino)
    say("error paths: reference build and layer")
    ctx.build_corr_index(dino, 24)
    ref_idx = ctx.get_corr_index().cpu().numpy()
    ref_o = ctx.sparse_attention(w.plan, q, k, v).clone()
    torch.cuda.synchronize()

    def still_intact():
        assert ctx.corr_k() == 24
        assert np.array_equal(ctx.get_corr_index().cpu().numpy(), ref_idx)
        o = ctx.sparse_attention(w.plan, q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o)

    # (allowance, K): 48 needs a new index buffer only (same scratch); 200
    # needs a larger scratch first; 300 gets its scratch and then fails on
    # the index buffer
    try:
        for allowance, K in [(0, 48), (0, 200), (1, 300)]:
            say(f"error paths: rebuild K={K} with {allowance} allocations allowed")
            saf.saf_debug_fail_alloc(allowance)
            with pytest.raises(saf.SafError) as ei:
                ctx.build_corr_index(dino, K)
            saf.saf_debug_fail_alloc(-1)
            assert ei.value.status == saf.SAF_ENOMEM, ei.value
            assert "hipMalloc" in ei.value.message
            still_intact()
    finally:
        saf.saf_debug_fail_alloc(-1)
    # with allocations allowed again the rebuild goes through
    say("error paths: rebuild K=48")
    ctx.build_corr_index(dino, 48)
    assert ctx.corr_k() == 48
    ctx.close()
