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
