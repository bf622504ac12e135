"""CPU oracle for SAF3R head-wise dynamic sparse global attention.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product library never imports,
links or runs anything here, and nothing here imports the product package.

The arithmetic lives in ``oracle.c`` (plain C, double precision, OpenMP over
independent rows); this module builds it with gcc, binds it with ctypes and
assembles per-head key sets the way the pages describe them:

* position heads  -- static set: all special tokens, the anchor frame and the
  query's own frame (Sec. 4.1 "Static Kernel"; Sec. 3 Obs. #2);
* vertical heads  -- top-K of the mean-query probe qbar K^T / sqrt(D), shared by
  all queries (Sec. 4.1 "Query-Probe Top-K", Sec. 4.3);
* correspondence  -- per-patch top-K of DINO cosine similarity against other
  frames (Sec. 4.1 "DINO Top-K", Sec. 4.3); special-token queries, which have
  no DINO feature, attend to every key;
* scanning heads  -- fixed stride of the token index plus all special tokens
  (Sec. 4.1 "Uniform Sampling Kernel");
* dense           -- every key (full global attention);
* corr + stride   -- a patch query's correspondence keys united with the
  scanning set of a given stride (the combination the paper proposes for
  scenes where DINO features miss regions); special queries attend to all;
* broadcast       -- the static pattern that broadcasts the first frame's
  local attention map to the other frames (Sec. 4.1 "Static Kernel", named
  there as an example): a patch query attends, in every frame, to the patches
  within a window around its own grid position, plus every special token;
  special queries attend to all.

Parity pins: see tests/test_oracle_pins.py.  Every function has at least one
pin independent of its own code (brute force, closed form, printed values).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Dict, Iterable, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ROLE_POSITION, ROLE_VERTICAL, ROLE_CORRESPONDENCE, ROLE_SCANNING, ROLE_DENSE = 0, 1, 2, 3, 4
# correspondence top-K united with the uniform stride set (Sec. 5, the second
# direction named for the DINO Top-K kernel): budget = the stride
ROLE_CORR_STRIDE = 5
# static broadcast of a local window to every frame: budget = the window
# radius r, anchor = the patch grid's width in patches (0: a window along the
# patch index)
ROLE_BROADCAST = 6
MODE_TOTAL, MODE_PER_FRAME = 0, 1


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc -O2 -fopenmp)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    """The oracle library.  SAF_ORACLE_LIB names another build of oracle.c to
    load instead (the sanitizer test runs the pins against such a build)."""
    global _lib
    if _lib is None:
        path = os.environ.get("SAF_ORACLE_LIB")
        if not path:
            build(force=False)
            path = _LIB
        L = C.CDLL(path)
        P = C.c_void_p
        i32, i64, dbl = C.c_int32, C.c_int64, C.c_double
        L.oracle_num_threads.restype = C.c_int
        L.oracle_num_threads.argtypes = []
        L.oracle_position_set.restype = i64
        L.oracle_position_set.argtypes = [i32, i32, i32, i32, i32, P]
        L.oracle_scan_set.restype = i64
        L.oracle_scan_set.argtypes = [i32, i32, i32, i32, P]
        L.oracle_topk.restype = i64
        L.oracle_topk.argtypes = [P, P, i64, i64, P, P, P]
        L.oracle_mean_query.restype = C.c_int
        L.oracle_mean_query.argtypes = [P, C.c_int, i64, i32, i64, P]
        L.oracle_probe_scores.restype = C.c_int
        L.oracle_probe_scores.argtypes = [P, C.c_int, i64, i32, i64, P, P]
        L.oracle_feature_norms.restype = C.c_int
        L.oracle_feature_norms.argtypes = [P, C.c_int, i64, i32, i64, P]
        L.oracle_corr_scores.restype = C.c_int
        L.oracle_corr_scores.argtypes = [P, C.c_int, i32, i32, i32, i64, P, P, i64, P]
        L.oracle_corr_index.restype = i64
        L.oracle_corr_index.argtypes = [P, C.c_int, i32, i32, i32, i32, i64, i32, i32, P, i64, P, P, P]
        L.oracle_attention.restype = C.c_int
        L.oracle_attention.argtypes = [P, P, P, C.c_int, i32, i64, i64, i64, P, P, P, P, P]
        _lib = L
    return _lib


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:
        return 1
    raise TypeError("oracle inputs are float32 or bfloat16 bits (uint16)")


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _i64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def num_threads() -> int:
    return int(lib().oracle_num_threads())


# ---------------------------------------------------------------------------
# Key sets
# ---------------------------------------------------------------------------
def position_set(S: int, ns: int, P: int, anchor: int, frame: int) -> np.ndarray:
    n = lib().oracle_position_set(S, ns, P, anchor, frame, None)
    out = np.empty(n, dtype=np.int64)
    lib().oracle_position_set(S, ns, P, anchor, frame, _p(out))
    return out


def scan_set(S: int, ns: int, P: int, stride: int) -> np.ndarray:
    n = lib().oracle_scan_set(S, ns, P, stride, None)
    out = np.empty(n, dtype=np.int64)
    lib().oracle_scan_set(S, ns, P, stride, _p(out))
    return out


def broadcast_set(S: int, ns: int, P: int, radius: int, grid_w: int, patch: int) -> np.ndarray:
    """Keys of the patch query at position `patch` under the broadcast static
    pattern (Sec. 4.1 "Static Kernel": the first frame's local attention map
    broadcast to the other frames).  Reading: frame 0's local map lets patch p
    see the patches near p; broadcast, every frame contributes its patches
    near p, so the query meets the same spatial neighbourhood in every view.
    Near = Chebyshev distance <= radius on a grid `grid_w` patches wide (rows
    of grid_w patches, row-major), or |p' - p| <= radius along the patch index
    when grid_w = 0.  Every special token is included, as in every static set.
    Written as a filter over all patches, not as a window walk."""
    T = ns + P
    pp = np.arange(P)
    if grid_w > 0:
        y, x = divmod(patch, grid_w)
        near = (np.abs(pp // grid_w - y) <= radius) & (np.abs(pp % grid_w - x) <= radius)
    else:
        near = np.abs(pp - patch) <= radius
    frames = np.arange(S, dtype=np.int64)[:, None] * T
    specials = (frames + np.arange(ns, dtype=np.int64)[None, :]).ravel()
    patches = (frames + ns + pp[near][None, :]).ravel()
    return np.union1d(specials, patches)


def topk(scores: np.ndarray, K: int, ids: Optional[np.ndarray] = None):
    """(ids ascending, score of the K-th kept, best dropped score)."""
    s = np.ascontiguousarray(scores, dtype=np.float64)
    idv = None if ids is None else _i64(ids)
    out = np.empty(min(K, s.size), dtype=np.int64)
    kth, nxt = C.c_double(), C.c_double()
    n = lib().oracle_topk(_p(s), _p(idv), s.size, K, _p(out), C.byref(kth), C.byref(nxt))
    if n < 0:
        raise MemoryError("oracle_topk")
    return out[:n], kth.value, nxt.value


def mean_query(q: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q)
    N, d = q.shape
    out = np.empty(d, dtype=np.float64)
    lib().oracle_mean_query(_p(q), _dt(q), N, d, d, _p(out))
    return out


def probe_scores(k: np.ndarray, qbar: np.ndarray) -> np.ndarray:
    k = np.ascontiguousarray(k)
    N, d = k.shape
    qb = np.ascontiguousarray(qbar, dtype=np.float64)
    out = np.empty(N, dtype=np.float64)
    lib().oracle_probe_scores(_p(k), _dt(k), N, d, d, _p(qb), _p(out))
    return out


def vertical_index(q: np.ndarray, k: np.ndarray, K: int):
    """Top-K keys of the mean-query probe: (ids, scores r, kth, next)."""
    r = probe_scores(k, mean_query(q))
    ids, kth, nxt = topk(r, K)
    return ids, r, kth, nxt


def feature_norms(F: np.ndarray) -> np.ndarray:
    F = np.ascontiguousarray(F)
    Np, Df = F.shape
    out = np.empty(Np, dtype=np.float64)
    lib().oracle_feature_norms(_p(F), _dt(F), Np, Df, Df, _p(out))
    return out


def corr_scores(F: np.ndarray, S: int, P: int, rows: Sequence[int]) -> np.ndarray:
    """Cosines of the listed patches against all patches (NaN in own frame)."""
    F = np.ascontiguousarray(F)
    Np, Df = F.shape
    rows = _i64(rows)
    norms = feature_norms(F)
    out = np.empty((rows.size, Np), dtype=np.float64)
    lib().oracle_corr_scores(_p(F), _dt(F), S, P, Df, Df, _p(norms), _p(rows), rows.size, _p(out))
    return out


def corr_index(F: np.ndarray, S: int, ns: int, P: int, K: int, rows: Sequence[int],
               mode: int = MODE_TOTAL):
    """Correspondence key rows for the listed patch numbers.

    Returns (idx [nrows, kc] global token ids ascending, tau, next)."""
    F = np.ascontiguousarray(F)
    Np, Df = F.shape
    rows = _i64(rows)
    if mode == MODE_TOTAL:
        kc = min(K, (S - 1) * P)
    else:
        kc = (S - 1) * min(K, P)
    out = np.empty((rows.size, kc), dtype=np.int64)
    tau = np.empty(rows.size, dtype=np.float64)
    nxt = np.empty(rows.size, dtype=np.float64)
    r = lib().oracle_corr_index(_p(F), _dt(F), S, ns, P, Df, Df, K, mode, _p(rows), rows.size,
                                _p(out), _p(tau), _p(nxt))
    if r < 0:
        raise ValueError(f"oracle_corr_index failed ({r})")
    return out, tau, nxt


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------
def attention_sets(q: np.ndarray, k: np.ndarray, v: np.ndarray, rows, row_set, sets) -> np.ndarray:
    """Softmax attention of the listed query rows over their key sets.

    sets: list of int arrays; row r uses sets[row_set[r]].  q, k, v: [N, d]."""
    q, k, v = (np.ascontiguousarray(a) for a in (q, k, v))
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    d = q.shape[1]
    rows, row_set = _i64(rows), _i64(row_set)
    lens = np.array([len(s) for s in sets], dtype=np.int64)
    set_ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    keys = _i64(np.concatenate([np.asarray(s, dtype=np.int64) for s in sets]) if sets else [])
    out = np.empty((rows.size, d), dtype=np.float64)
    rc = lib().oracle_attention(_p(q), _p(k), _p(v), _dt(q), d, d, d, rows.size, _p(rows),
                                _p(row_set), _p(set_ptr), _p(keys), _p(out))
    if rc != 0:
        raise ValueError("empty key set")
    return out


def attention(q, k, v, rows, keys) -> np.ndarray:
    """All listed rows attend to one shared key set."""
    rows = _i64(rows)
    return attention_sets(q, k, v, rows, np.zeros(rows.size, dtype=np.int64), [keys])


def _as_f64(a: np.ndarray) -> np.ndarray:
    """float32 values, or bfloat16 bits (uint16) decoded exactly, as float64."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if a.dtype == np.float32:
        return a.astype(np.float64)
    raise TypeError("oracle inputs are float32 or bfloat16 bits (uint16)")


def qk_index(q: np.ndarray, k: np.ndarray, S: int, ns: int, P: int, K: int, rows: Sequence[int],
             mode: int = MODE_TOTAL):
    """Correspondence key rows taken from one head's own attention logits
    instead of DINO features (SAF3R Sec. 5, first direction named for the
    DINO Top-K kernel): for patch u (token i) the patch tokens j of other
    frames ranked by (q_i . k_j desc, token asc) -- the 1/sqrt(d) scale
    does not change the order -- first min(K, (S-1)P) of them (total) or
    min(K, P) of every other frame (per frame).  q, k: one head's [N, d].
    Returns (idx [nrows, kc] ascending, kth score per row)."""
    T = ns + P
    Q, Kf = _as_f64(q), _as_f64(k)
    patch_tok = np.array([(v // P) * T + ns + v % P for v in range(S * P)], dtype=np.int64)
    rows = _i64(rows)
    out, kth = [], []
    for u in rows:
        fu = u // P
        s = Kf[patch_tok] @ Q[patch_tok[u]]
        if mode == MODE_TOTAL:
            ok = np.arange(S * P) // P != fu
            ids, kv, _ = topk(s[ok], K, patch_tok[ok])
        else:
            parts, kv = [], []
            for f in range(S):
                if f == fu:
                    continue
                ids_f, k_f, _ = topk(s[f * P:(f + 1) * P], K, patch_tok[f * P:(f + 1) * P])
                parts.append(ids_f)
                kv.append(k_f)
            ids = np.concatenate(parts)
        out.append(ids)
        kth.append(kv)
    return np.array(out, dtype=np.int64), kth


# ---------------------------------------------------------------------------
# Block-wise correspondence (Sec. 4.3)
def block_scores(F: np.ndarray, S: int, P: int, b: int, qblocks: Sequence[int]) -> np.ndarray:
    """Block-wise DINO similarity (Sec. 4.3, block-wise implementation).

    Blocks are b consecutive patches of one frame (b divides P); block B =
    patches B*b .. B*b+b-1.  The similarity of two blocks is the token-level
    cosine averaged over their b x b patch pairs, computed here literally
    from the cosine rows.  Returns [len(qblocks), S*P/b]; NaN for the blocks
    of the query block's own frame."""
    if P % b:
        raise ValueError("block size must divide P")
    nb = S * (P // b)
    qblocks = _i64(qblocks)
    out = np.empty((qblocks.size, nb), dtype=np.float64)
    for i, A in enumerate(qblocks):
        c = corr_scores(F, S, P, np.arange(A * b, (A + 1) * b))   # [b, S*P]
        out[i] = c.reshape(b, nb, b).mean(axis=(0, 2))
    return out


def block_corr_index(F: np.ndarray, S: int, ns: int, P: int, b: int, K: int, rows: Sequence[int],
                     mode: int = MODE_TOTAL):
    """Correspondence key rows under block-wise similarity.

    Every patch of query block A gets the patches of A's selected blocks: the
    first min(K, (S-1)P/b) blocks of other frames by (similarity desc, block
    asc) (total mode), or the first min(K, P/b) of every other frame
    (per-frame mode).  Returns (idx [nrows, kb*b] global tokens ascending,
    {query block: (selected blocks, kth score, best dropped score)})."""
    if P % b:
        raise ValueError("block size must divide P")
    T, per = ns + P, P // b
    rows = _i64(rows)
    qb = np.unique(rows // b)
    sc = block_scores(F, S, P, b, qb)
    blk = np.arange(S * per)
    sel = {}
    for i, A in enumerate(qb):
        fa = A // per
        if mode == MODE_TOTAL:
            ok = blk // per != fa
            ids, kth, nxt = topk(sc[i][ok], K, blk[ok])
        else:
            parts, kth, nxt = [], [], []
            for f in range(S):
                if f == fa:
                    continue
                g = blk[f * per:(f + 1) * per]
                ids_f, k_f, n_f = topk(sc[i][g], K, g)
                parts.append(ids_f)
                kth.append(k_f)
                nxt.append(n_f)
            ids = np.concatenate(parts)
        sel[int(A)] = (ids, kth, nxt)
    kb = len(next(iter(sel.values()))[0]) if sel else 0
    out = np.empty((rows.size, kb * b), dtype=np.int64)
    for r, u in enumerate(rows):
        patches = (sel[int(u // b)][0][:, None] * b + np.arange(b)[None, :]).reshape(-1)
        out[r] = (patches // P) * T + ns + patches % P
    return out, sel


# ---------------------------------------------------------------------------
# One layer: every head by its role, on a subset of query rows.
def layer_sets(geom, plan, q, k, v, dino=None, corr_K: int = 0, corr_mode: int = MODE_TOTAL,
               rows: Optional[np.ndarray] = None, corr_rows: Optional[Dict[int, np.ndarray]] = None,
               vert_sets: Optional[Dict[int, np.ndarray]] = None):
    """Key sets per head for the given query rows, from the oracle's own selection.

    corr_rows / vert_sets supply index rows (patch number -> token ids) and
    vertical key sets (head -> token ids) selected elsewhere, e.g. sets that a
    test has already checked against the oracle's scores; whatever is not
    supplied is selected here.

    Returns (per-head (row_set, sets), corr rows dict, vertical info dict)."""
    S, ns, P, N, T = geom.S, geom.ns, geom.P, geom.N, geom.T
    rows = np.arange(N, dtype=np.int64) if rows is None else _i64(rows)
    frame = rows // T
    is_special = (rows % T) < ns
    out = {}
    vert = {}
    corr = dict(corr_rows or {})
    if any(p[0] in (ROLE_CORRESPONDENCE, ROLE_CORR_STRIDE) for p in plan):
        need = [int((i // T) * P + (i % T) - ns) for i in rows[~is_special]]
        missing = sorted(set(need) - set(corr))
        if missing:
            idx, _, _ = corr_index(dino, S, ns, P, corr_K, missing, corr_mode)
            for u, r in zip(missing, idx):
                corr[u] = r
    for h, (role, budget, anchor, _flags) in enumerate(plan):
        if role == ROLE_POSITION:
            frames = np.unique(frame)
            sets = [position_set(S, ns, P, anchor, int(f)) for f in frames]
            row_set = np.searchsorted(frames, frame)
        elif role == ROLE_SCANNING:
            sets = [scan_set(S, ns, P, budget)]
            row_set = np.zeros(rows.size, dtype=np.int64)
        elif role == ROLE_VERTICAL:
            if vert_sets is not None and h in vert_sets:
                ids = np.asarray(vert_sets[h], dtype=np.int64)
                vert[h] = dict(ids=ids)
            else:
                ids, r, kth, nxt = vertical_index(q[h], k[h], budget)
                vert[h] = dict(ids=ids, scores=r, kth=kth, next=nxt)
            sets = [ids]
            row_set = np.zeros(rows.size, dtype=np.int64)
        elif role == ROLE_CORR_STRIDE:
            scan = scan_set(S, ns, P, budget)
            sets = [np.arange(N, dtype=np.int64)]
            row_set = np.zeros(rows.size, dtype=np.int64)
            for r_i, i in enumerate(rows):
                if not is_special[r_i]:
                    u = int((i // T) * P + (i % T) - ns)
                    row_set[r_i] = len(sets)
                    sets.append(np.union1d(scan, corr[u]))
        elif role == ROLE_CORRESPONDENCE:
            sets = [np.arange(N, dtype=np.int64)]
            row_set = np.zeros(rows.size, dtype=np.int64)
            for r_i, i in enumerate(rows):
                if not is_special[r_i]:
                    u = int((i // T) * P + (i % T) - ns)
                    row_set[r_i] = len(sets)
                    sets.append(corr[u])
        elif role == ROLE_DENSE:
            sets = [np.arange(N, dtype=np.int64)]
            row_set = np.zeros(rows.size, dtype=np.int64)
        elif role == ROLE_BROADCAST:
            # special queries have no grid position: every key
            sets = [np.arange(N, dtype=np.int64)]
            row_set = np.zeros(rows.size, dtype=np.int64)
            pos = rows % T - ns
            seen = {}
            for r_i in np.nonzero(~is_special)[0]:
                p_ = int(pos[r_i])
                if p_ not in seen:
                    seen[p_] = len(sets)
                    sets.append(broadcast_set(S, ns, P, budget, anchor, p_))
                row_set[r_i] = seen[p_]
        else:
            raise ValueError(f"unknown role {role}")
        out[h] = (row_set, sets)
    return out, corr, vert


def layer(geom, plan, q, k, v, dino=None, corr_K: int = 0, corr_mode: int = MODE_TOTAL,
          rows: Optional[np.ndarray] = None, corr_rows: Optional[Dict[int, np.ndarray]] = None,
          heads: Optional[Iterable[int]] = None, vert_sets: Optional[Dict[int, np.ndarray]] = None):
    """Oracle outputs [H][nrows, d] (float64) for the listed query rows."""
    rows = np.arange(geom.N, dtype=np.int64) if rows is None else _i64(rows)
    sets, corr, vert = layer_sets(geom, plan, q, k, v, dino, corr_K, corr_mode, rows, corr_rows, vert_sets)
    heads = range(geom.H) if heads is None else heads
    outs = {}
    for h in heads:
        row_set, s = sets[h]
        outs[h] = attention_sets(q[h], k[h], v[h], rows, row_set, s)
    return outs, corr, vert
