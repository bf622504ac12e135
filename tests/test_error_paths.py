"""Error paths that need no GPU.

* Every SAF_ENOMEM return of the library, forced through its allocation
  hook (saf_debug_fail_alloc) so that no device is touched: the status, the
  message, and that a failed build leaves no index behind on a fresh context.
* The Python binding's tensor checks: q, k, v and o must share one shape,
  one set of strides and the context's dtype, and live on the GPU; row counts
  of DINO features, imported indices and vertical sets must match the
  geometry.  A mismatch raises ValueError before anything reaches the
  library, which takes one layout and dtype for all four tensors and would
  otherwise read or write out of bounds.
"""
import ctypes as C

import pytest
import torch

import head_wise_dynamic_amd as saf

FAKE = 0x10000  # aligned, never dereferenced: the hook fails the first allocation
S, NS, P, H, D = 4, 5, 256, 16, 64
N = S * (NS + P)
LAY = saf.saf_layout_t(N * D, D)


@pytest.fixture
def ctx():
    c = C.c_void_p()
    assert saf.saf_create(saf.saf_geometry_t(S, NS, P, H, D, saf.SAF_BF16), c) == saf.SAF_OK
    saf.saf_debug_fail_alloc(0)
    try:
        yield c
    finally:
        saf.saf_debug_fail_alloc(-1)
        saf.saf_destroy(c)


def _enomem(c, st, what):
    assert st == saf.SAF_ENOMEM, (st, saf.saf_last_error(c))
    msg = saf.saf_last_error(c)
    assert "hipMalloc" in msg and what in msg, msg


def test_index_builds_report_enomem(ctx):
    kc = C.c_int32()
    _enomem(ctx, saf.saf_build_corr_index(ctx, FAKE, 1, 64, 64, 8, 0, None), "index scratch")
    assert saf.saf_get_corr_index(ctx, None, kc, None) == saf.SAF_ESTATE
    # per-frame: the fused build (bf16, P = 256, K = 8) and the stored-row build
    _enomem(ctx, saf.saf_build_corr_index(ctx, FAKE, 1, 64, 64, 8, 1, None), "index scratch")
    _enomem(ctx, saf.saf_build_corr_index(ctx, FAKE, 1, 64, 64, 8, 2, None), "index scratch")
    _enomem(ctx, saf.saf_build_corr_index_blocks(ctx, FAKE, 1, 64, 64, 4, 8, 0, None), "index scratch")
    _enomem(ctx, saf.saf_build_corr_index_qk(ctx, FAKE, FAKE, LAY, 0, 8, 0, None), "index scratch")
    _enomem(ctx, saf.saf_set_corr_index(ctx, FAKE, 8, None), "correspondence index")
    assert saf.saf_get_corr_index(ctx, None, kc, None) == saf.SAF_ESTATE
    cnt = C.c_int32()
    assert saf.saf_corr_recomputed_rows(ctx, None, 0, cnt, None) == saf.SAF_ESTATE


def test_error_kernels_report_enomem(ctx):
    _enomem(ctx, saf.saf_head_nmse(ctx, FAKE, FAKE, LAY, FAKE, None), "error partials")
    _enomem(ctx, saf.saf_head_nmse_accumulate(ctx, FAKE, FAKE, LAY, 0.5, FAKE, 1, None), "error partials")


def test_accumulate_argument_checks(ctx):
    f = saf.saf_head_nmse_accumulate
    assert f(ctx, None, FAKE, LAY, 1.0, FAKE, 1, None) == saf.SAF_EINVAL
    assert f(ctx, FAKE, FAKE, LAY, 1.0, None, 1, None) == saf.SAF_EINVAL
    assert f(ctx, FAKE, FAKE, LAY, 1.0, FAKE, 0, None) == saf.SAF_EINVAL       # stride
    assert f(ctx, FAKE, FAKE, LAY, -1.0, FAKE, 1, None) == saf.SAF_EINVAL      # weight
    assert f(ctx, FAKE, FAKE, LAY, float("nan"), FAKE, 1, None) == saf.SAF_EINVAL
    assert f(ctx, FAKE, FAKE, LAY, float("inf"), FAKE, 1, None) == saf.SAF_EINVAL
    assert f(ctx, FAKE, FAKE, LAY, 1.0, FAKE + 4, 1, None) == saf.SAF_EINVAL   # misaligned accumulator
    assert f(ctx, FAKE + 2, FAKE, LAY, 1.0, FAKE, 1, None) == saf.SAF_EINVAL   # misaligned output
    cnt = C.c_int32()
    assert saf.lib().saf_corr_recomputed_rows(ctx, None, 0, None, None) == saf.SAF_EINVAL
    assert saf.saf_corr_recomputed_rows(ctx, None, 4, cnt, None) == saf.SAF_EINVAL
    assert saf.saf_corr_recomputed_rows(ctx, None, -1, cnt, None) == saf.SAF_EINVAL


# ---------------------------------------------------------------------------
# binding checks
def _c(dtype=torch.bfloat16):
    return saf.Context(S, NS, P, H, D, dtype)


def _qkvo(dtype=torch.bfloat16, shape=(H, N, D)):
    return [torch.zeros(shape, dtype=dtype) for _ in range(4)]


PLAN = [(saf.SAF_SCANNING, 8, 0, 0)] * H


@pytest.mark.parametrize("which", [1, 2, 3])
def test_binding_rejects_mismatched_shapes(which):
    ctx = _c()
    t = _qkvo()
    t[which] = torch.zeros((H, N - 1, D), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="shape"):
        ctx.sparse_attention(PLAN, t[0], t[1], t[2], o=t[3])
    with pytest.raises(ValueError, match="shape"):
        ctx.dense_attention(t[0], t[1], t[2], o=t[3])
    ctx.close()


def test_binding_rejects_layout_mix():
    """q in [H, N, d] with o in [N, H, d]: same element count, other layout."""
    ctx = _c()
    q, k, v, _ = _qkvo()
    o = torch.zeros((N, H, D), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="shape"):
        ctx.sparse_attention(PLAN, q, k, v, o=o)
    kt = torch.zeros((N, H, D), dtype=torch.bfloat16).transpose(0, 1)   # [H, N, d] view, other strides
    with pytest.raises(ValueError, match="strides"):
        ctx.sparse_attention(PLAN, q, kt, v, o=torch.zeros_like(q))
    ctx.close()


def test_binding_rejects_wrong_dtype():
    ctx = _c()
    q, k, v, o = _qkvo()
    with pytest.raises(ValueError, match="dtype"):
        ctx.sparse_attention(PLAN, q, k.float(), v, o=o)
    qf, kf, vf, of = _qkvo(torch.float32)
    with pytest.raises(ValueError, match="dtype"):   # fp32 tensors, bf16 context
        ctx.dense_attention(qf, kf, vf, o=of)
    with pytest.raises(ValueError, match="dtype"):
        ctx.head_nmse_accumulate(qf, kf, torch.zeros(H, dtype=torch.float64), 1.0)
    ctx.close()


def test_binding_rejects_host_tensors():
    ctx = _c()
    q, k, v, o = _qkvo()
    with pytest.raises(ValueError, match="GPU"):
        ctx.sparse_attention(PLAN, q, k, v, o=o)
    with pytest.raises(ValueError, match="GPU"):
        ctx.build_corr_index_qk(q, k, 0, 8)
    with pytest.raises(ValueError, match="GPU"):
        ctx.build_vertical_index(q, k, 0, 8)
    ctx.close()


def test_binding_rejects_wrong_row_counts():
    ctx = _c()
    with pytest.raises(ValueError, match="rows"):
        ctx.build_corr_index(torch.zeros((S * P - 1, 64), dtype=torch.bfloat16), 8)
    with pytest.raises(ValueError, match="rows"):
        ctx.build_corr_index_blocks(torch.zeros((S * P + 1, 64), dtype=torch.bfloat16), 4, 8)
    with pytest.raises(ValueError, match="rows"):
        ctx.set_corr_index(torch.zeros((S * P - 1, 8), dtype=torch.int32))
    with pytest.raises(ValueError, match="plan"):
        q, k, v, o = _qkvo()
        ctx.sparse_attention(PLAN[:-1], q, k, v, o=o)
    ctx.close()
