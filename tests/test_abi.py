"""C-ABI checks that need no GPU: the library loads, exports every declared
entry point, and rejects bad arguments on the host with the documented codes
before anything is enqueued."""
import ctypes as C
import os
import re

import pytest

import head_wise_dynamic_amd as saf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "saf3r.h")
FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(saf_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = saf.lib()
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(saf.exported_symbols())


def _ctx(S=4, ns=5, P=256, H=16, dtype=saf.SAF_BF16):
    c = C.c_void_p()
    st = saf.saf_create(saf.saf_geometry_t(S, ns, P, H, 64, dtype), c)
    assert st == saf.SAF_OK, saf.saf_last_error(None)
    return c


@pytest.mark.parametrize("geom,code", [
    ((0, 5, 256, 16, 64, 1), saf.SAF_EINVAL),
    ((4, -1, 256, 16, 64, 1), saf.SAF_EINVAL),
    ((4, 5, 0, 16, 64, 1), saf.SAF_EINVAL),
    ((4, 5, 256, 0, 64, 1), saf.SAF_EINVAL),
    ((4, 5, 256, 16, 64, 7), saf.SAF_EINVAL),
    ((4, 5, 256, 16, 32, 1), saf.SAF_EUNSUPPORTED),
    ((100000, 5, 30000, 16, 64, 1), saf.SAF_EINVAL),
    ((1 << 20, 0, 1 << 10, 16, 64, 1), saf.SAF_EINVAL),   # N = 2^30: key-slot counts must stay below 2^31
])
def test_create_rejects_bad_geometry(geom, code):
    c = C.c_void_p()
    assert saf.saf_create(saf.saf_geometry_t(*geom), c) == code
    assert not c.value
    assert saf.saf_last_error(None)


def _plan(roles):
    return saf.make_plan(roles)


GOOD = [(0, 0, 0, 0)] * 4 + [(1, 64, 0, 0)] * 4 + [(4, 0, 0, 0)] * 4 + [(3, 8, 0, 0)] * 4
LAY = saf.saf_layout_t(4 * 1044 * 64 * 0 + 1044 * 64, 64)


def _call(c, plan, ws_bytes=1 << 30, lay=LAY, q=FAKE, o=FAKE, ws=FAKE):
    return saf.saf_sparse_attention(c, _plan(plan), q, FAKE, FAKE, o, lay, None, 0, ws, ws_bytes, None)


@pytest.mark.parametrize("bad,code", [
    ((9, 0, 0, 0), saf.SAF_EINVAL),          # unknown role
    ((1, 0, 0, 0), saf.SAF_EINVAL),          # vertical K < 1
    ((3, 0, 0, 0), saf.SAF_EINVAL),          # stride < 1
    ((0, 0, 4, 0), saf.SAF_EINVAL),          # anchor outside [0, S)
    ((0, 0, -1, 0), saf.SAF_EINVAL),
    ((6, -1, 0, 0), saf.SAF_EINVAL),         # broadcast radius < 0
    ((6, 1, 3, 0), saf.SAF_EINVAL),          # broadcast grid width not dividing P = 256
    ((6, 1, -16, 0), saf.SAF_EINVAL),
    ((0, 0, 0, 1), saf.SAF_EUNSUPPORTED),    # flags
    ((2, 0, 0, 0), saf.SAF_ESTATE),          # correspondence head, no index yet
])
def test_sparse_attention_rejects_bad_plans(bad, code):
    c = _ctx()
    try:
        plan = list(GOOD)
        plan[5] = bad
        assert _call(c, plan) == code
        assert saf.saf_last_error(c)
    finally:
        saf.saf_destroy(c)


def test_sparse_attention_rejects_bad_pointers_layouts_and_workspace():
    c = _ctx()
    try:
        assert _call(c, GOOD, q=None) == saf.SAF_EINVAL
        assert _call(c, GOOD, o=FAKE + 2) == saf.SAF_EINVAL          # misaligned
        assert _call(c, GOOD, lay=saf.saf_layout_t(1044 * 64, 60)) == saf.SAF_EINVAL
        assert _call(c, GOOD, lay=saf.saf_layout_t(64, 64)) == saf.SAF_EINVAL  # heads overlap tokens
        need = C.c_size_t()
        assert saf.saf_workspace_size(c, _plan(GOOD), need) == saf.SAF_OK
        assert need.value > 0
        assert _call(c, GOOD, ws_bytes=need.value - 1) == saf.SAF_EINVAL
        assert _call(c, GOOD, ws=None) == saf.SAF_EINVAL
        assert saf.saf_sparse_attention(c, None, FAKE, FAKE, FAKE, FAKE, LAY, None, 0, FAKE, 1 << 30,
                                        None) == saf.SAF_EINVAL
    finally:
        saf.saf_destroy(c)


def test_correspondence_needs_two_frames():
    c = _ctx(S=1)
    try:
        plan = list(GOOD)
        plan[8] = (2, 0, 0, 0)
        assert _call(c, plan, lay=saf.saf_layout_t(261 * 64, 64)) == saf.SAF_EINVAL
        assert saf.saf_build_corr_index(c, FAKE, 1, 64, 64, 8, 0, None) == saf.SAF_EINVAL
        assert saf.saf_set_corr_index(c, FAKE, 8, None) == saf.SAF_EINVAL
    finally:
        saf.saf_destroy(c)


def test_build_corr_index_validation():
    c = _ctx()
    try:
        b = saf.saf_build_corr_index
        assert b(c, None, 1, 64, 64, 8, 0, None) == saf.SAF_EINVAL
        assert b(c, FAKE, 1, 64, 64, 0, 0, None) == saf.SAF_EINVAL       # K < 1
        assert b(c, FAKE, 1, 0, 64, 8, 0, None) == saf.SAF_EINVAL        # Df < 1
        assert b(c, FAKE, 1, 64, 32, 8, 0, None) == saf.SAF_EINVAL       # stride < Df
        assert b(c, FAKE, 5, 64, 64, 8, 0, None) == saf.SAF_EINVAL       # dtype
        assert b(c, FAKE, 1, 64, 64, 8, 7, None) == saf.SAF_EINVAL
        assert b(c, FAKE, 1, 64, 68, 8, 0, None) == saf.SAF_EINVAL       # rows not 16-byte aligned
        kc = C.c_int32()
        assert saf.saf_get_corr_index(c, None, kc, None) == saf.SAF_ESTATE
        assert saf.saf_set_corr_index(c, FAKE, 0, None) == saf.SAF_EINVAL
        assert saf.saf_set_corr_index(c, FAKE, 3 * 256 + 1, None) == saf.SAF_EINVAL
    finally:
        saf.saf_destroy(c)
    c = _ctx(S=2, P=4097)
    try:   # the per-frame selection holds at most 4096 patches per frame
        assert saf.saf_build_corr_index(c, FAKE, 1, 64, 64, 8, 1, None) == saf.SAF_EUNSUPPORTED
        assert saf.saf_build_corr_index(c, FAKE, 1, 64, 64, 2000, 0, None) == saf.SAF_EUNSUPPORTED
    finally:
        saf.saf_destroy(c)


def test_build_corr_index_blocks_validation():
    c = _ctx()
    try:
        b = saf.saf_build_corr_index_blocks
        assert b(c, None, 1, 64, 64, 4, 8, 0, None) == saf.SAF_EINVAL
        assert b(c, FAKE, 1, 64, 64, 0, 8, 0, None) == saf.SAF_EINVAL       # block < 1
        assert b(c, FAKE, 1, 64, 64, 3, 8, 0, None) == saf.SAF_EINVAL       # 3 does not divide P = 256
        assert b(c, FAKE, 1, 64, 64, 4, 0, 0, None) == saf.SAF_EINVAL       # K < 1
        assert b(c, FAKE, 1, 64, 64, 4, 8, 2, None) == saf.SAF_EINVAL       # mode
        assert b(c, FAKE, 1, 64, 32, 4, 8, 0, None) == saf.SAF_EINVAL       # stride < Df
        assert b(c, FAKE, 1, 8192, 8192, 4, 8, 0, None) == saf.SAF_EUNSUPPORTED  # Df
    finally:
        saf.saf_destroy(c)
    c = _ctx(S=9)
    try:   # 2000 of the 8 x 256 one-patch blocks in one row
        assert saf.saf_build_corr_index_blocks(c, FAKE, 1, 64, 64, 1, 2000, 0, None) == saf.SAF_EUNSUPPORTED
    finally:
        saf.saf_destroy(c)


def test_build_corr_index_qk_validation():
    c = _ctx()
    try:
        b = saf.saf_build_corr_index_qk
        assert b(c, None, FAKE, LAY, 0, 8, 0, None) == saf.SAF_EINVAL
        assert b(c, FAKE, FAKE, LAY, 16, 8, 0, None) == saf.SAF_EINVAL     # head
        assert b(c, FAKE, FAKE, LAY, -1, 8, 0, None) == saf.SAF_EINVAL
        assert b(c, FAKE, FAKE, LAY, 0, 0, 0, None) == saf.SAF_EINVAL      # K
        assert b(c, FAKE, FAKE, LAY, 0, 8, 3, None) == saf.SAF_EINVAL      # mode
    finally:
        saf.saf_destroy(c)
    c = _ctx(S=9)
    try:   # 2000 of 8 x 256 candidates in one total-mode row
        lay = saf.saf_layout_t(9 * 261 * 64, 64)
        assert saf.saf_build_corr_index_qk(c, FAKE, FAKE, lay, 0, 2000, 0, None) == saf.SAF_EUNSUPPORTED
    finally:
        saf.saf_destroy(c)


def test_vertical_index_validation():
    c = _ctx()
    try:
        f = saf.saf_build_vertical_index
        assert f(c, FAKE, FAKE, LAY, 16, 8, FAKE, FAKE, 1 << 30, None) == saf.SAF_EINVAL   # head
        assert f(c, FAKE, FAKE, LAY, 0, 0, FAKE, FAKE, 1 << 30, None) == saf.SAF_EINVAL    # K
        assert f(c, FAKE, FAKE, LAY, 0, 8, None, FAKE, 1 << 30, None) == saf.SAF_EINVAL
        assert f(c, FAKE, FAKE, LAY, 0, 8, FAKE, FAKE, 16, None) == saf.SAF_EINVAL        # workspace
    finally:
        saf.saf_destroy(c)


def test_context_wrapper_raises_on_error():
    with pytest.raises(saf.SafError) as ei:
        saf.Context(4, 5, 256, d=32)
    assert ei.value.status == saf.SAF_EUNSUPPORTED
    ctx = saf.Context(4, 5, 256, dtype=__import__("torch").float32)
    assert ctx.workspace_size(None) == 0  # fp32 dense: the row kernel needs none
    assert ctx.workspace_size(GOOD) > 0
    ctx.close()
    # bf16 dense: room for the key-norm maxima of one launch group
    ctx = saf.Context(4, 5, 256, dtype=__import__("torch").bfloat16)
    assert ctx.workspace_size(None) >= 24 * 256 * 4
    with pytest.raises(saf.SafError):
        ctx.workspace_size([(9, 0, 0, 0)] * 16)
    ctx.close()


def test_create_accepts_n_just_below_the_limit():
    c = C.c_void_p()
    assert saf.saf_create(saf.saf_geometry_t((1 << 20) - 1, 0, 1 << 10, 16, 64, 1), c) == saf.SAF_OK
    saf.saf_destroy(c)


def test_dense_attention_needs_workspace_for_bf16():
    """bf16 dense: the key-norm maxima live in the workspace (no device touched
    before the check)."""
    c = _ctx()
    try:
        need = C.c_size_t()
        assert saf.saf_workspace_size(c, None, need) == saf.SAF_OK and need.value > 0
        f = saf.saf_dense_attention
        assert f(c, FAKE, FAKE, FAKE, FAKE, LAY, None, 0, None) == saf.SAF_EINVAL
        assert "workspace" in saf.saf_last_error(c)
        assert f(c, FAKE, FAKE, FAKE, FAKE, LAY, FAKE, need.value - 1, None) == saf.SAF_EINVAL
        assert f(c, FAKE, FAKE, FAKE, FAKE, LAY, FAKE + 8, need.value, None) == saf.SAF_EINVAL  # misaligned
    finally:
        saf.saf_destroy(c)
    c = _ctx(dtype=saf.SAF_F32)
    try:
        need = C.c_size_t()
        assert saf.saf_workspace_size(c, None, need) == saf.SAF_OK and need.value == 0
    finally:
        saf.saf_destroy(c)


@pytest.mark.parametrize("S,ns,P,stride", [(4, 5, 256, 8), (4, 5, 256, 1), (4, 5, 256, 261), (7, 3, 200, 7),
                                           (3, 0, 100, 16), (100, 5, 1369, 16), (819, 5, 16, 5)])
def test_workspace_holds_the_packed_scanning_set(S, ns, P, stride):
    """A bf16 scanning head's packed key set (the stride tokens, then the
    specials off the stride, plus their token list) is in the workspace: the
    size grows by exactly that over the same plan with a dense head, which
    needs none.  Brute-force count of the specials on the stride."""
    T, N = ns + P, S * (ns + P)
    on = sum(1 for f in range(S) for t in range(ns) if (f * T + t) % stride == 0)
    rows = (N + stride - 1) // stride + ns * S - on
    a256 = lambda x: (x + 255) // 256 * 256
    expect = 2 * a256(rows * 128) + a256(4 * ns * S + 4)
    c = _ctx(S, ns, P)
    try:
        base = [(0, 0, 0, 0)] * 15
        ws, wd = C.c_size_t(), C.c_size_t()
        assert saf.saf_workspace_size(c, _plan(base + [(3, stride, 0, 0)]), ws) == saf.SAF_OK
        assert saf.saf_workspace_size(c, _plan(base + [(4, 0, 0, 0)]), wd) == saf.SAF_OK
        assert ws.value - wd.value == expect
    finally:
        saf.saf_destroy(c)
    c = _ctx(S, ns, P, dtype=saf.SAF_F32)   # fp32: the row kernel enumerates the set, nothing packed
    try:
        ws, wd = C.c_size_t(), C.c_size_t()
        assert saf.saf_workspace_size(c, _plan(base + [(3, stride, 0, 0)]), ws) == saf.SAF_OK
        assert saf.saf_workspace_size(c, _plan(base + [(4, 0, 0, 0)]), wd) == saf.SAF_OK
        assert ws.value == wd.value
    finally:
        saf.saf_destroy(c)
