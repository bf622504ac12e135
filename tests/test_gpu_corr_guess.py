"""Correspondence index: rows whose best matches sit in the first frames.

The symmetric pass of the index build filters with a per-row guess of the
K-th best cosine taken from the first frames; a row whose guess turns out too
high (fewer than K candidates reach it) must be recomputed exactly.  These
features put near-copies of some late patches into the first frames, so
those rows take that path; every row must still match the oracle's top-K
(band rule, 1e-5).
"""
import numpy as np
import pytest
import torch

import oracle
from workload import make_front_loaded_dino

from helpers import band_check, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("K", [32, 100])
def test_front_loaded_rows_stay_exact(K):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_wise_dynamic_amd as saf
    S, ns, P, Df = 40, 1, 64, 128          # Np = 2560: the symmetric pass covers patches [256, 2560)
    dino, special = make_front_loaded_dino(S, P, Df, first_frames=4, n_rows=20, copies=12, seed=3)
    ctx = saf.Context(S, ns, P, 16, 64, torch.bfloat16)
    say(f"front-loaded corr index K={K}")
    ctx.build_corr_index(to_dev(dino), K)
    got = ctx.get_corr_index().cpu().numpy()
    Np, T = S * P, ns + P
    sc = oracle.corr_scores(dino, S, P, np.arange(Np))
    frame = np.arange(Np) // P
    for u in range(Np):
        gp = (got[u] // T) * P + got[u] % T - ns
        band_check(np.nan_to_num(sc[u], nan=-np.inf), gp, K, valid=frame != frame[u])
    # the special rows' copies all rank first
    for u in special:
        gp = (got[u] // T) * P + got[u] % T - ns
        top = np.argsort(-np.nan_to_num(sc[u], nan=-np.inf), kind="stable")[:12]
        assert np.all(np.isin(top, gp))
    ctx.close()


def test_more_flagged_rows_than_the_matrix_core_batches():
    """1,200 late patches in 60 groups, each group with 8 near-copies in the
    first two frames (the columns the guess is taken from): every one of them
    fails the guess check.  The first 1,024 flagged rows are recomputed by
    the row-list GEMM, the rest by the per-row engine; all rows must match
    the oracle's top-K."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_wise_dynamic_amd as saf
    from workload import make_grouped_front_dino
    S, ns, P, Df, K = 30, 1, 256, 128, 32
    dino, late = make_grouped_front_dino(S, P, Df, first_frames=2, groups=60, group_size=20, copies=8, seed=5)
    ctx = saf.Context(S, ns, P, 16, 64, torch.bfloat16)
    say("corr index with 1200 flagged rows")
    ctx.build_corr_index(to_dev(dino), K)
    got = ctx.get_corr_index().cpu().numpy()
    Np, T = S * P, ns + P
    frame = np.arange(Np) // P
    for r0 in range(0, Np, 1024):
        rows = np.arange(r0, min(Np, r0 + 1024))
        sc = oracle.corr_scores(dino, S, P, rows)
        for i, u in enumerate(rows):
            gp = (got[u] // T) * P + got[u] % T - ns
            band_check(np.nan_to_num(sc[i], nan=-np.inf), gp, K, valid=frame != frame[u])
    ctx.close()
