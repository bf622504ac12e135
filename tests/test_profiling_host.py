"""Host logic of the offline head profiler (C ABI, no GPU needed) against
the oracle: pair counts and Eq. 2's cost per configuration, the baseline
stride and the selection rule of Eq. 2."""
import ctypes as C

import numpy as np
import pytest

import head_wise_dynamic_amd as saf
from oracle import profiling
from workload import Geometry


def _ctx(S, ns, P):
    c = C.c_void_p()
    assert saf.saf_create(saf.saf_geometry_t(S, ns, P, 16, 64, saf.SAF_BF16), c) == saf.SAF_OK
    return c


@pytest.mark.parametrize("S,ns,P", [(3, 2, 10), (4, 5, 256), (100, 5, 1369), (500, 5, 1296), (2, 0, 7)])
def test_head_pairs_match_oracle(S, ns, P):
    geom = Geometry(S=S, ns=ns, P=P)
    c = _ctx(S, ns, P)
    try:
        cfgs = [(saf.SAF_DENSE, 0, 0), (saf.SAF_POSITION, 0, 0), (saf.SAF_POSITION, 0, S - 1),
                (saf.SAF_VERTICAL, 64, 0), (saf.SAF_VERTICAL, 10 ** 9, 0), (saf.SAF_CORRESPONDENCE, 32, 0),
                (saf.SAF_CORRESPONDENCE, 10 ** 9, 0)] + [(saf.SAF_SCANNING, s, 0) for s in (1, 2, 3, 7, 16, 33)]
        gw = {10: 5, 256: 16, 1369: 37, 1296: 36, 7: 7}[P]   # the patch grid's width
        cfgs += [(saf.SAF_BROADCAST, 0, 0), (saf.SAF_BROADCAST, 1, gw), (saf.SAF_BROADCAST, 2, 0)]
        if P <= 256:
            cfgs += [(saf.SAF_BROADCAST, P, gw), (saf.SAF_BROADCAST, 3, 1)]
        for role, budget, anchor in cfgs:
            n = C.c_int64()
            h = saf.saf_head_plan_t(role, budget, anchor, 0)
            assert saf.saf_head_pairs(c, C.byref(h), budget, C.byref(n)) == saf.SAF_OK
            assert n.value == profiling.head_pairs(geom, (role, budget, anchor)), (role, budget, anchor)
            # Eq. 2's cost: the oracle's FLOP count of the configuration
            f = C.c_double()
            assert saf.saf_head_cost(c, C.byref(h), budget, C.byref(f)) == saf.SAF_OK
            assert f.value == float(profiling.head_flops(geom, (role, budget, anchor))), (role, budget, anchor)
        n = C.c_int64()
        bad = saf.saf_head_plan_t(saf.SAF_POSITION, 0, S, 0)
        assert saf.saf_head_pairs(c, C.byref(bad), 0, C.byref(n)) == saf.SAF_EINVAL
        for bad_b in (saf.saf_head_plan_t(saf.SAF_BROADCAST, -1, 0, 0),
                      saf.saf_head_plan_t(saf.SAF_BROADCAST, 1, -2, 0)):
            assert saf.saf_head_pairs(c, C.byref(bad_b), 0, C.byref(n)) == saf.SAF_EINVAL
        if P % 3:
            b3 = saf.saf_head_plan_t(saf.SAF_BROADCAST, 1, 3, 0)   # grid width not dividing P
            assert saf.saf_head_pairs(c, C.byref(b3), 0, C.byref(n)) == saf.SAF_EINVAL
        corr = saf.saf_head_plan_t(saf.SAF_CORRESPONDENCE, 0, 0, 0)
        assert saf.saf_head_pairs(c, C.byref(corr), 0, C.byref(n)) == saf.SAF_ESTATE    # no cached index
        f = C.c_double()
        assert saf.saf_head_cost(c, C.byref(corr), 0, C.byref(f)) == saf.SAF_ESTATE
        assert saf.saf_head_cost(c, C.byref(bad), 0, C.byref(f)) == saf.SAF_EINVAL
        assert saf.lib().saf_head_cost(c, C.byref(corr), 8, None) == saf.SAF_EINVAL
    finally:
        saf.saf_destroy(c)


def test_baseline_stride_matches_oracle():
    for sigma in np.concatenate([np.linspace(0, 0.99, 199), [0.5, 0.75, 0.8, 0.85, 0.9, 0.95, 0.875]]):
        assert saf.saf_baseline_stride(float(sigma)) == profiling.baseline_stride(float(sigma)), sigma
    assert saf.saf_baseline_stride(1.0) == -1 and saf.saf_baseline_stride(-0.1) == -1


def test_select_matches_oracle():
    rng = np.random.default_rng(1)
    P = C.POINTER(C.c_double)
    for _ in range(2000):
        n = int(rng.integers(1, 9))
        e = np.round(rng.random(n), 1)          # coarse values: ties happen
        cst = rng.integers(1, 5, n).astype(np.float64)
        got = saf.saf_profile_select(e.ctypes.data_as(P), cst.ctypes.data_as(P), n)
        assert got == profiling.select(e, cst)
    assert saf.saf_profile_select(None, None, 0) == -1
