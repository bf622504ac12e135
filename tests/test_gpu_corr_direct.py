"""Correspondence index, direct square (SAF3R Sec. 4.1 "DINO Top-K Kernel").

When the two seed frames hold on average at least five of a row's K best
(K 2P >= 5 (S-1) P, with 4 K + 128 <= P), the build guesses every row's K-th
best from the seed frames' lane maxima and filters the whole square once with
that guess; a row whose exact K-th best falls below its guess is recomputed.
S = 8, P = 256, K = 32 takes that path (guess rank 23 of 448 lane maxima, 12
for rows of the seed frames themselves).  Every row must match the oracle's
top-K (band rule, 1e-5).
"""
import numpy as np
import pytest
import torch

import oracle
from workload import make_front_loaded_dino

from helpers import band_check, say, to_dev

pytestmark = pytest.mark.gpu

S, NS, P, DF, K = 8, 1, 256, 128, 32


def _check_all_rows(dino, got):
    Np, T = S * P, NS + P
    sc = oracle.corr_scores(dino, S, P, np.arange(Np))
    frame = np.arange(Np) // P
    for u in range(Np):
        gp = (got[u] // T) * P + got[u] % T - NS
        band_check(np.nan_to_num(sc[u], nan=-np.inf), gp, K, valid=frame != frame[u])


def test_direct_square_random_features():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_wise_dynamic_amd as saf
    dino, _ = make_front_loaded_dino(S, P, DF, first_frames=2, n_rows=0, copies=0, seed=11)
    ctx = saf.Context(S, NS, P, 16, 64, torch.bfloat16)
    say(f"direct-square corr index S={S} P={P} K={K}")
    ctx.set_kernel_timing(True)
    ctx.build_corr_index(to_dev(dino), K)
    torch.cuda.synchronize()
    gemms = [n for n, _ in ctx.read_kernel_timing() if n == "cosine_gemm"]
    ctx.set_kernel_timing(False)
    # the schedule taken: the seed frames' lane maxima, then the square
    assert len(gemms) == 2, gemms
    got = ctx.get_corr_index().cpu().numpy()
    _check_all_rows(dino, got)
    ctx.close()


def test_direct_square_guess_failures_are_recomputed():
    """16 late patches, each with 28 near-copies in the two seed frames: at
    least 23 distinct lane maxima of the seed reach copy level, so the guess
    sits at copy level while the row's 32nd best is an ordinary patch (only
    28 copies exist).  Those rows fail the check and are recomputed."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_wise_dynamic_amd as saf
    dino, special = make_front_loaded_dino(S, P, DF, first_frames=2, n_rows=16, copies=28, seed=12)
    ctx = saf.Context(S, NS, P, 16, 64, torch.bfloat16)
    say(f"direct-square corr index with front-loaded rows S={S} P={P} K={K}")
    ctx.build_corr_index(to_dev(dino), K)
    got = ctx.get_corr_index().cpu().numpy()
    redone = set(ctx.recomputed_rows())
    assert len(redone & set(int(u) for u in special)) >= len(special) // 2, sorted(redone)[:20]
    _check_all_rows(dino, got)
    T = NS + P
    sc = oracle.corr_scores(dino, S, P, special)
    for i, u in enumerate(special):  # the copies all rank first
        gp = (got[u] // T) * P + got[u] % T - NS
        top = np.argsort(-np.nan_to_num(sc[i], nan=-np.inf), kind="stable")[:28]
        assert np.all(np.isin(top, gp))
    ctx.close()
