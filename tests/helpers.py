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
    tau = np.partition(s, s.size - kk)[s.size - kk]   # the kk-th largest
    must = cand[s > tau + eps]
    assert np.all(np.isin(must, g)), f"missing {np.setdiff1d(must, g)[:8]} (tau={tau})"
    assert np.all(scores[g] >= tau - eps), f"kept a key below tau - eps (tau={tau})"


# ---------------------------------------------------------------------------
# Correspondence index rows at full size
def token_patch(g, tok) -> np.ndarray:
    """Patch number of global patch token ids."""
    tok = np.asarray(tok, dtype=np.int64)
    return (tok // g.T) * g.P + tok % g.T - g.ns


def check_index_structure(g, gidx: np.ndarray, kc: int, per_frame_k: int = 0, chunk: int = 1 << 14) -> None:
    """Every row of an index: kc entries, strictly ascending (hence distinct),
    patch tokens only, none from the query's own frame.  Per-frame mode
    (per_frame_k > 0): kc = (S-1) per_frame_k and the entries come frame by
    frame, per_frame_k from each other frame in ascending frame order."""
    assert gidx.shape == (g.Np, kc), (gidx.shape, (g.Np, kc))
    for r0 in range(0, g.Np, chunk):
        blk = gidx[r0:r0 + chunk].astype(np.int64)
        own = (np.arange(r0, r0 + blk.shape[0]) // g.P)[:, None]
        assert blk.min() >= 0 and blk.max() < g.N, f"token id outside [0, N) in rows {r0}.."
        if kc > 1:
            bad = np.nonzero(np.any(np.diff(blk, axis=1) <= 0, axis=1))[0]
            assert bad.size == 0, f"rows not strictly ascending: {r0 + bad[:8]}"
        bad = np.nonzero(np.any(blk % g.T < g.ns, axis=1))[0]
        assert bad.size == 0, f"special token in rows {r0 + bad[:8]}"
        f = blk // g.T
        bad = np.nonzero(np.any(f == own, axis=1))[0]
        assert bad.size == 0, f"own-frame token in rows {r0 + bad[:8]}"
        if per_frame_k:
            seg = np.arange(kc)[None, :] // per_frame_k
            want = seg + (seg >= own)
            bad = np.nonzero(np.any(f != want, axis=1))[0]
            assert bad.size == 0, f"per-frame segments out of order in rows {r0 + bad[:8]}"


def index_rows_to_check(g, n: int, extra=(), seed: int = 0, tile: int = 256) -> np.ndarray:
    """At least n patch rows to band-check at full size, always including:
    every row of the ragged last tile of `tile` rows; rows below 4P (the
    rows of the build's first column phases, which also stay in its doubling
    phases) sampled, with both ends; both sides of tile boundaries at the
    start, around each doubling of 2P (2P, 4P, 8P, ...), around 4P + k tile
    (the tile grid of the pair square that starts there), mid-range and at
    the end; both sides of frame boundaries; the listed extra rows; then
    random rows up to n."""
    Np = g.Np
    rng = np.random.default_rng(seed)
    sel = set(range((Np - 1) // tile * tile, Np))
    lo = min(Np, 4 * g.P)
    sel.update(int(x) for x in rng.choice(lo, min(lo, 96), replace=False))
    sel.update([0, 1, lo - 1])
    bounds = [tile, 2 * tile, (Np // 2) // tile * tile, (Np - 1) // tile * tile - tile]
    b = 2 * g.P
    while b < Np:
        bounds += [b, b // tile * tile, (b // tile + 1) * tile]
        b *= 2
    bounds += [lo + k * tile for k in (0, 1, 2, 7)]
    for b in bounds:
        sel.update(r for r in (b - 2, b - 1, b, b + 1) if 0 <= r < Np)
    for f in sorted({1, 2, g.S // 2, g.S - 1}):
        sel.update(r for r in (f * g.P - 1, f * g.P, f * g.P + 1) if 0 <= r < Np)
    sel.update(int(x) for x in extra)
    rows = np.array(sorted(sel), dtype=np.int64)
    if rows.size < n:
        rest = np.setdiff1d(np.arange(Np), rows)
        rows = np.union1d(rows, rng.choice(rest, min(rest.size, n - rows.size), replace=False))
    return rows


def band_check_corr_rows(w, gidx: np.ndarray, rows, K: int, per_frame: bool = False, chunk: int = 128):
    """Band rule for the listed rows of a DINO-cosine index against the
    oracle's fp64 cosines (total mode over all other frames, or per other
    frame).  Returns {patch number: the GPU row (token ids)} for the rows,
    all of which passed."""
    import oracle
    g = w.geom
    frame = np.arange(g.Np) // g.P
    rows = np.asarray(rows, dtype=np.int64)
    for c0 in range(0, rows.size, chunk):
        part = rows[c0:c0 + chunk]
        sc = oracle.corr_scores(w.dino, g.S, g.P, part)
        for i, u in enumerate(part):
            if not per_frame:
                band_check(np.nan_to_num(sc[i], nan=-np.inf), token_patch(g, gidx[u]), K,
                           valid=frame != frame[u])
                continue
            kf = min(K, g.P)
            fu = u // g.P
            for f in range(g.S):
                if f == fu:
                    continue
                slot = f - (f > fu)
                seg = gidx[u, slot * kf:(slot + 1) * kf].astype(np.int64)
                assert np.all(seg // g.T == f), (u, f)
                band_check(sc[i, f * g.P:(f + 1) * g.P], seg % g.T - g.ns, kf)
    return {int(u): gidx[u].astype(np.int64) for u in rows}


def patch_rows_of(g, rows) -> np.ndarray:
    """Patch numbers of the patch-token rows among the given token rows."""
    rows = np.asarray(rows, dtype=np.int64)
    t = rows % g.T
    return np.unique((rows[t >= g.ns] // g.T) * g.P + t[t >= g.ns] - g.ns)
