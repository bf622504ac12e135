"""Offline head profiling (SAF3R Sec. 4.2), the oracle's version.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the tests, the
smoke check and the benchmark's CPU-baseline leg are the only callers.

* E(c), Eq. (1): the normalised squared error of a head's sparse output under
  configuration c against its full-attention output, averaged over the
  calibration samples;
* Omega(c): the floating-point work of the configuration, 4 d per (query,
  key) pair (one multiply-add each for q.k and p.v);
* Eq. (2) by progressive substitution: start from the uniform-sampling
  baseline c_base and take a candidate whenever its error is strictly lower
  than the current choice's and its cost does not exceed the baseline's.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

from . import (ROLE_BROADCAST, ROLE_CORRESPONDENCE, ROLE_DENSE, ROLE_POSITION, ROLE_SCANNING,
               ROLE_VERTICAL, MODE_TOTAL, broadcast_set, corr_index, layer)

Config = Tuple[int, int, int]   # (role, budget, anchor frame)


def nmse(o_full: np.ndarray, o_sparse: np.ndarray) -> float:
    """||O_full - O_sparse||^2 / ||O_full||^2 (Frobenius), in float64."""
    a = np.asarray(o_full, dtype=np.float64)
    b = np.asarray(o_sparse, dtype=np.float64)
    return float(np.sum((a - b) ** 2) / np.sum(a * a))


def baseline_stride(sigma: float) -> int:
    """Stride of the uniform-sampling baseline with sparsity ratio sigma: the
    smallest stride that keeps at most a fraction 1 - sigma of the keys."""
    if not 0.0 <= sigma < 1.0:
        raise ValueError("sigma must lie in [0, 1)")
    return max(1, math.ceil(1.0 / (1.0 - sigma) - 1e-12))


def head_pairs(geom, cfg: Config) -> int:
    """(query, key) pairs one head computes under cfg at this geometry."""
    role, budget, anchor = cfg
    S, ns, P, T, N = geom.S, geom.ns, geom.P, geom.T, geom.N
    if role == ROLE_DENSE:
        return N * N
    if role == ROLE_POSITION:
        return sum(T * (ns * S + (P if f == anchor else 2 * P)) for f in range(S))
    if role == ROLE_SCANNING:
        on = (N + budget - 1) // budget
        on_special = sum(1 for f in range(S) for t in range(ns) if (f * T + t) % budget == 0)
        return N * (on + ns * S - on_special)
    if role == ROLE_VERTICAL:
        return N * min(budget, N)
    if role == ROLE_CORRESPONDENCE:
        return S * P * min(budget, (S - 1) * P) + ns * S * N
    if role == ROLE_BROADCAST:
        # a patch query's set depends on its position only; special rows see all
        return S * sum(broadcast_set(S, ns, P, budget, anchor, p).size for p in range(P)) + ns * S * N
    raise ValueError(f"unknown role {role}")


def head_flops(geom, cfg: Config) -> int:
    return 4 * geom.d * head_pairs(geom, cfg)


def select(errors: Sequence[float], costs: Sequence[float]) -> int:
    """Eq. (2) by progressive substitution over entries 0 (the baseline), 1, 2, ...

    Returns the index of the chosen configuration."""
    best = 0
    for i in range(1, len(errors)):
        if costs[i] <= costs[0] and errors[i] < errors[best]:
            best = i
    return best


def profile(samples, candidates: Sequence[Config], sigma: float,
            rows: np.ndarray = None) -> Dict[str, object]:
    """Run the search on calibration samples (workloads sharing one geometry).

    Every head is scored under the baseline (uniform sampling at sigma) and
    every candidate; rows: the query rows the errors are taken over (default
    all).  Returns errors [H, 1 + len(candidates)], costs, the configuration
    list and the chosen index per head."""
    g = samples[0].geom
    configs: List[Config] = [(ROLE_SCANNING, baseline_stride(sigma), 0)] + list(candidates)
    rows = np.arange(g.N, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    err = np.zeros((g.H, len(configs)), dtype=np.float64)
    for w in samples:
        dense_plan = [(ROLE_DENSE, 0, 0, 0)] * g.H
        full, _, _ = layer(g, dense_plan, w.q, w.k, w.v, rows=rows)
        for j, (role, budget, anchor) in enumerate(configs):
            plan = [(role, budget, anchor, 0)] * g.H
            corr_rows = None
            if role == ROLE_CORRESPONDENCE:
                t = rows % g.T
                pr = np.unique((rows[t >= g.ns] // g.T) * g.P + t[t >= g.ns] - g.ns)
                idx, _, _ = corr_index(w.dino, g.S, g.ns, g.P, budget, pr, MODE_TOTAL)
                corr_rows = {int(u): r for u, r in zip(pr, idx)}
            out, _, _ = layer(g, plan, w.q, w.k, w.v, w.dino, corr_K=budget, rows=rows, corr_rows=corr_rows)
            for h in range(g.H):
                err[h, j] += nmse(full[h], out[h]) / len(samples)
    costs = np.array([head_flops(g, c) for c in configs], dtype=np.float64)
    choice = np.array([select(err[h], costs) for h in range(g.H)], dtype=np.int64)
    return dict(configs=configs, errors=err, costs=costs, choice=choice)
