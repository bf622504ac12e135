"""Shared test utilities: device upload/download and the near-tie band rule."""
import sys

import numpy as np
import torch

from workload import bf16_to_f32

NEAR_TIE = 1e-5


def say(msg: str) -> None:
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_host_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return bf16_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def torch_dtype(w) -> torch.dtype:
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def tol(w) -> float:
    """Max-abs output tolerance: 2e-2 for bf16 inputs, 1e-4 for fp32."""
    return 2e-2 if w.dtype == "bf16" else 1e-4


def band_check(scores: np.ndarray, gpu_set: np.ndarray, K: int, valid: np.ndarray = None,
               eps: float = NEAR_TIE) -> None:
    """GPU top-K set vs oracle scores (fp64), modulo near-ties.

    scores: oracle score per candidate id (ids = positions); valid: mask of
    candidates (None = all).  The set must have min(K, n) distinct valid ids,
    contain every id scoring above tau + eps and none scoring below tau - eps,
    tau being the oracle's K-th best score."""
    ids = np.arange(scores.size)
    cand = ids if valid is None else ids[valid]
    n = cand.size
    kk = min(K, n)
    g = np.asarray(gpu_set, dtype=np.int64)
    assert g.size == kk, (g.size, kk)
    assert np.unique(g).size == kk, "repeated ids in the GPU set"
    assert np.all(np.diff(g) > 0), "GPU set is not ascending"
    if valid is not None:
        assert np.all(valid[g]), "GPU set holds a non-candidate"
    s = scores[cand]
    tau = np.sort(s)[::-1][kk - 1]
    must = cand[s > tau + eps]
    assert np.all(np.isin(must, g)), f"missing {np.setdiff1d(must, g)[:8]} (tau={tau})"
    assert np.all(scores[g] >= tau - eps), f"kept a key below tau - eps (tau={tau})"
