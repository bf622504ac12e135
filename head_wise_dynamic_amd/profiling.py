"""Offline head profiling on the GPU (SAF3R Sec. 4.2).

For every head, the error E(c) of Eq. 1 (normalised squared error of the
head's sparse output against its full-attention output, averaged over
calibration samples) is measured for the uniform-sampling baseline and for
each candidate configuration; Eq. 2 then keeps, by progressive
substitution, the lowest-error configuration whose floating-point work does
not exceed the baseline's.  Every attention output and every error sum is
computed by the library's kernels (dense and sparse attention, the per-head
error of Eq. 1 averaged over the samples, the pair counts, the Eq. 2
selection); this module only sequences the calls.
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

import ctypes as C
import numpy as np
import torch

from . import SAF_CORRESPONDENCE, SAF_SCANNING, Context, saf_baseline_stride, saf_profile_select

Config = Tuple[int, int, int]   # (role, budget, anchor frame)


def baseline(sigma: float) -> Config:
    """Uniform sampling with sparsity ratio sigma (stride from the library)."""
    s = saf_baseline_stride(float(sigma))
    if s < 1:
        raise ValueError("sigma must lie in [0, 1)")
    return (SAF_SCANNING, s, 0)


def config_flops(ctx: Context, cfg: Config) -> float:
    role, budget, anchor = cfg
    return ctx.head_cost(role, budget, anchor, corr_kc=budget if role == SAF_CORRESPONDENCE else 0)


def select(errors: Sequence[float], costs: Sequence[float]) -> int:
    e = np.ascontiguousarray(errors, dtype=np.float64)
    c = np.ascontiguousarray(costs, dtype=np.float64)
    r = saf_profile_select(e.ctypes.data_as(C.POINTER(C.c_double)), c.ctypes.data_as(C.POINTER(C.c_double)),
                           e.size)
    if r < 0:
        raise ValueError("empty configuration list")
    return r


def profile_heads(ctx: Context, samples: Sequence[Dict[str, torch.Tensor]], candidates: Sequence[Config],
                  sigma: float, stream=None) -> Dict[str, object]:
    """samples: dicts of device tensors q, k, v ([H, N, d] or [N, H, d]) and
    dino ([S*P, Df]); all share the context's geometry.

    Returns configs (baseline first), errors [H, n], costs [n] (FLOPs) and
    the chosen configuration index per head."""
    configs: List[Config] = [baseline(sigma)] + [tuple(c) for c in candidates]
    H = ctx.H
    err = None
    for smp in samples:
        q, k, v = smp["q"], smp["k"], smp["v"]
        full = ctx.dense_attention(q, k, v, stream=stream)
        out = torch.empty_like(full)
        if err is None:
            err = torch.zeros((H, len(configs)), dtype=torch.float64, device=full.device)
        built = None
        for j, (role, budget, anchor) in enumerate(configs):
            if role == SAF_CORRESPONDENCE and built != budget:
                ctx.build_corr_index(smp["dino"], budget, stream=stream)
                built = budget
            # a correspondence head's budget 0 means "the cached index"
            b = 0 if role == SAF_CORRESPONDENCE else budget
            ctx.sparse_attention([(role, b, anchor, 0)] * H, q, k, v, o=out, stream=stream)
            ctx.head_nmse_accumulate(full, out, err[:, j], 1.0 / len(samples), stream=stream)
    err = err.cpu().numpy() if err is not None else np.zeros((H, len(configs)), dtype=np.float64)
    costs = np.array([config_flops(ctx, c) for c in configs], dtype=np.float64)
    choice = np.array([select(err[h], costs) for h in range(H)], dtype=np.int64)
    return dict(configs=configs, errors=err, costs=costs, choice=choice)
