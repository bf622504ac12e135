"""saf_sparse_attention_noalloc against saf_sparse_attention, through the C ABI.

The no-allocation variant takes its workspace from the library's static
device scratch instead of the caller and runs every launch on the caller's
stream; it runs the same kernels, so its output must equal the regular entry
point's bit for bit.  Two calls in a row share the scratch, the second with a
smaller input (it must not depend on what the first left there); a plan
whose workspace exceeds the scratch is rejected before anything runs.
"""
import ctypes as C

import numpy as np
import pytest
import torch

from workload import (Geometry, make_geometry_inputs, ROLE_BROADCAST, ROLE_CORR_STRIDE, ROLE_CORRESPONDENCE,
                      ROLE_DENSE, ROLE_POSITION, ROLE_SCANNING, ROLE_VERTICAL)

from helpers import say, to_dev

pytestmark = pytest.mark.gpu


def _saf():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_wise_dynamic_amd as saf
    saf.lib()
    return saf


def _noalloc(saf, ctx, plan, q, k, v, o):
    lay = ctx.layout_of(q)
    st = torch.cuda.current_stream()
    return saf.saf_sparse_attention_noalloc(ctx._ctx, saf.make_plan(plan), C.c_void_p(q.data_ptr()),
                                            C.c_void_p(k.data_ptr()), C.c_void_p(v.data_ptr()),
                                            C.c_void_p(o.data_ptr()), lay, None, 0, C.c_void_p(st.cuda_stream))


def _compare(saf, S, ns, P, seed, grid_w):
    g = Geometry(S=S, ns=ns, P=P)
    roles = ([ROLE_POSITION] * 2 + [ROLE_VERTICAL] * 3 + [ROLE_CORRESPONDENCE] * 3 + [ROLE_SCANNING] * 3 +
             [ROLE_DENSE, ROLE_BROADCAST, ROLE_BROADCAST, ROLE_CORR_STRIDE, ROLE_CORR_STRIDE])
    budgets = [0, 0, 64, 200, 7, 24, 24, 24, 8, 1, 33, 0, 1, 0, 16, 5]
    anchors = [0, S - 1] + [0] * 10 + [grid_w, 0, 0, 0]
    w = make_geometry_inputs(g, "bf16", roles, budgets, M=3 * P, Df=64, seed=seed, corr_K=24, anchors=anchors)
    ctx = saf.Context(g.S, g.ns, g.P, g.H, g.d, torch.bfloat16)
    q, k, v = to_dev(w.q), to_dev(w.k), to_dev(w.v)
    ctx.build_corr_index(to_dev(w.dino), w.corr_K)
    ref = ctx.sparse_attention(w.plan, q, k, v)
    out = torch.full_like(q, float("nan"))
    say(f"no-alloc layer S={S} ns={ns} P={P}")
    assert _noalloc(saf, ctx, w.plan, q, k, v, out) == saf.SAF_OK, saf.saf_last_error(ctx._ctx)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), float((out.float() - ref.float()).abs().max())
    ctx.close()


def test_noalloc_matches_the_regular_entry_point_on_two_calls():
    saf = _saf()
    _compare(saf, 3, 5, 300, seed=7, grid_w=20)   # first call on this GPU
    _compare(saf, 2, 5, 120, seed=8, grid_w=12)   # second call, smaller input, same scratch


def test_noalloc_rejects_a_plan_beyond_the_static_scratch():
    saf = _saf()
    # S = 500 frames of 1296 patches: three vertical sets and the split dense
    # rows of three correspondence heads need far more than 64 MiB
    ctx = saf.Context(500, 5, 1296, 16, 64, torch.bfloat16)
    plan = [(ROLE_POSITION, 0, 0, 0)] * 4 + [(ROLE_VERTICAL, 4096, 0, 0)] * 3 + \
        [(ROLE_CORRESPONDENCE, 0, 0, 0)] * 3 + [(ROLE_SCANNING, 32, 0, 0)] * 6
    x = torch.empty(16, 16, dtype=torch.bfloat16, device="cuda")
    lay = saf.saf_layout_t(650500 * 64, 64)
    st = saf.saf_sparse_attention_noalloc(ctx._ctx, saf.make_plan(plan), C.c_void_p(x.data_ptr()),
                                          C.c_void_p(x.data_ptr()), C.c_void_p(x.data_ptr()),
                                          C.c_void_p(x.data_ptr()), lay, None, 0, None)
    assert st == saf.SAF_EUNSUPPORTED
    assert "static scratch" in saf.saf_last_error(ctx._ctx)
    ctx.close()
