"""Seeded synthetic workloads for head-wise sparse global attention.

The pages ("SAF3R: Dynamic Sparse Attention for Feed-Forward 3D Reconstruction
Transformers", Sec. 5.1) measure on 7Scenes / ScanNet sequences with VGGT-like
token grids.  Those datasets are not available, so these seeded generators stand
in for them with the same shapes: S frames, each holding ns special tokens
(one camera + four register tokens, placed first) followed by P patch tokens in
row-major order; H = 16 heads of width d = 64.

What is drawn (one numpy PCG64 SeedSequence per workload, spawned into seven
sub-streams in this order: latents, frame sampling, DINO noise, per-head
projections W_h, Q/K/V, salient keys, probe directions):

* M latent scene points z ~ N(0, I_Df).  Normal draws are float32.
* Frame 0's patches take P distinct latents.  In every other frame,
  round(0.7 P) randomly placed patches take latents drawn without replacement
  from frame 0's set; the remaining patches take distinct latents from the
  complement.
* DINO-like patch features f_u = z_lat(u) + N(0, 0.3^2) (patches only).
* Q, K, V ~ N(0, 1) everywhere, then per role:
  - correspondence heads: patch rows of Q and K become z_lat W_h + 0.1 eps,
    with W_h ~ N(0, 1/Df) of shape Df x d, eps the row's own N(0,1) draw;
  - vertical-line heads: a unit direction u per head; 24 patch keys drawn
    uniformly get K += 4u and every query gets Q += u.
* bf16 workloads are rounded to bfloat16 with round-to-nearest-even.
* Each head draws from its own sub-streams (projection, Q/K/V, salient keys,
  direction), spawned from the four per-layer streams.

Nothing here computes key sets, scores or attention: this module only draws
and lays out numbers, so it may feed both the oracle and the GPU path.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

ROLE_POSITION = 0
ROLE_VERTICAL = 1
ROLE_CORRESPONDENCE = 2
ROLE_SCANNING = 3
ROLE_DENSE = 4
ROLE_CORR_STRIDE = 5
ROLE_BROADCAST = 6
ROLE_NAMES = {0: "position", 1: "vertical", 2: "correspondence", 3: "scanning", 4: "dense", 5: "corr_stride",
              6: "broadcast"}

N_SALIENT = 24


@dataclass(frozen=True)
class Geometry:
    S: int            # frames
    ns: int           # special tokens per frame (first in the frame)
    P: int            # patch tokens per frame
    H: int = 16       # heads
    d: int = 64       # head width

    @property
    def T(self) -> int:
        return self.ns + self.P

    @property
    def N(self) -> int:
        return self.S * self.T

    @property
    def Np(self) -> int:
        return self.S * self.P

    def patch_token(self, u):
        """Global token index of patch number u (u = frame * P + p)."""
        u = np.asarray(u, dtype=np.int64)
        return (u // self.P) * self.T + self.ns + (u % self.P)


@dataclass
class Workload:
    name: str
    geom: Geometry
    dtype: str                              # "f32" or "bf16"
    plan: List[Tuple[int, int, int, int]]   # per head: (role, budget, anchor_frame, flags)
    q: np.ndarray                           # [H, N, d] float32, or uint16 bf16 bits
    k: np.ndarray
    v: np.ndarray
    dino: np.ndarray                        # [S*P, Df] float32 or uint16 bf16 bits
    Df: int
    corr_K: int
    lat: np.ndarray = field(repr=False, default=None)       # [S*P] latent id per patch
    salient: Dict[int, np.ndarray] = field(default_factory=dict)  # head -> salient token ids
    seed: int = 0

    @property
    def roles(self) -> List[int]:
        return [p[0] for p in self.plan]

    def heads(self, role: int) -> List[int]:
        return [h for h, p in enumerate(self.plan) if p[0] == role]


# ---------------------------------------------------------------------------
# Workload table.  Sizes follow the measured configurations: a tiny fp32 case,
# VGGT-scale layers at S = 32 and S = 100 (518 px -> 37 x 37 patches), a
# 24-layer stack at S = 100, and S = 500 at 504 px (36 x 36 patches).
# ---------------------------------------------------------------------------
def _mix(n_pos, n_vert, n_corr, n_scan):
    return ([ROLE_POSITION] * n_pos + [ROLE_VERTICAL] * n_vert +
            [ROLE_CORRESPONDENCE] * n_corr + [ROLE_SCANNING] * n_scan)


CONFIGS: Dict[int, dict] = {
    1: dict(name="tiny_fp32_S4", S=4, ns=5, P=256, dtype="f32", M=600, Df=384,
            roles=_mix(4, 4, 4, 4), vert_K=64, corr_K=32, scan_s=8),
    2: dict(name="vggt_S32_bf16", S=32, ns=5, P=1369, dtype="bf16", M=20000, Df=1024,
            roles=_mix(4, 3, 3, 6), vert_K=2048, corr_K=256, scan_s=16),
    3: dict(name="vggt_S100_bf16", S=100, ns=5, P=1369, dtype="bf16", M=20000, Df=1024,
            roles=_mix(4, 3, 3, 6), vert_K=2048, corr_K=256, scan_s=16),
    4: dict(name="vggt_stack24_S100_bf16", S=100, ns=5, P=1369, dtype="bf16", M=20000,
            Df=1024, roles=_mix(4, 3, 3, 6), corr_roles=_mix(4, 3, 6, 3), corr_layers=range(10, 17),
            layers=24, vert_K=2048, corr_K=256, scan_s=16),
    5: dict(name="long_S500_bf16", S=500, ns=5, P=1296, dtype="bf16", M=150000, Df=1024,
            roles=_mix(4, 3, 3, 6), vert_K=4096, corr_K=128, scan_s=32),
}


def config(cid: int) -> dict:
    return CONFIGS[cid]


def _budget(role: int, vert_K: int, corr_K: int, scan_s: int) -> int:
    if role == ROLE_VERTICAL:
        return vert_K
    if role == ROLE_CORRESPONDENCE:
        return corr_K
    if role == ROLE_SCANNING:
        return scan_s
    return 0


# ---------------------------------------------------------------------------
# bfloat16 encoding (round to nearest even) -- input encoding only.
# ---------------------------------------------------------------------------
def bf16_round(x) -> np.ndarray:
    """float array -> uint16 bfloat16 bits, round-to-nearest-even via float32."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bf16_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def _encode(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_round(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


# ---------------------------------------------------------------------------
# Generator
# ---------------------------------------------------------------------------
def _frame_latents(rng, S: int, P: int, M: int) -> np.ndarray:
    if M < 2 * P:
        raise ValueError("need at least 2P latent points")
    lat = np.empty((S, P), dtype=np.int64)
    lat[0] = rng.choice(M, size=P, replace=False)
    f0 = lat[0].copy()
    comp = np.setdiff1d(np.arange(M, dtype=np.int64), f0)
    n_ov = int(round(0.7 * P))
    for f in range(1, S):
        pos = rng.choice(P, size=n_ov, replace=False)
        src = rng.permutation(f0)[:n_ov]
        rest = rng.choice(comp, size=P - n_ov, replace=False)
        take = np.zeros(P, dtype=bool)
        take[pos] = True
        lat[f, pos] = src
        lat[f, ~take] = rest
    return lat.reshape(-1)


def make_geometry_inputs(geom: Geometry, dtype: str, roles: Sequence[int],
                         budgets: Sequence[int], M: int, Df: int, seed: int,
                         qkv_seed: Optional[int] = None, corr_K: int = 0,
                         name: str = "custom", anchors: Optional[Sequence[int]] = None,
                         dino: bool = True, heads: Optional[Sequence[int]] = None) -> Workload:
    """Draw one layer's Q/K/V (+ DINO-like features) for any geometry.

    Every head draws from its own sub-stream, so `heads` (default: all) can
    restrict the draw to a subset; the other heads' Q/K/V are left zero."""
    if len(roles) != geom.H or len(budgets) != geom.H:
        raise ValueError("roles/budgets must have one entry per head")
    S, P, N, H, d, T, ns = geom.S, geom.P, geom.N, geom.H, geom.d, geom.T, geom.ns
    streams = np.random.SeedSequence(seed).spawn(7)
    s_lat, s_frames, s_dino = streams[0], streams[1], streams[2]
    if qkv_seed is None:
        s_w, s_qkv, s_sal, s_probe = streams[3:]
    else:
        s_w, s_qkv, s_sal, s_probe = np.random.SeedSequence(qkv_seed).spawn(7)[3:]

    z = np.random.default_rng(s_lat).standard_normal((M, Df), dtype=np.float32)
    lat = _frame_latents(np.random.default_rng(s_frames), S, P, M)
    patch_tok = geom.patch_token(np.arange(S * P))

    dino_arr = None
    if dino:
        rng_d = np.random.default_rng(s_dino)
        dino_arr = np.empty((S * P, Df), dtype=np.uint16 if dtype == "bf16" else np.float32)
        for f in range(S):
            sl = slice(f * P, (f + 1) * P)
            dino_arr[sl] = _encode(z[lat[sl]] + np.float32(0.3) * rng_d.standard_normal((P, Df), dtype=np.float32),
                                   dtype)

    per_head = list(zip(s_w.spawn(H), s_qkv.spawn(H), s_sal.spawn(H), s_probe.spawn(H)))
    store = np.uint16 if dtype == "bf16" else np.float32
    qo = np.zeros((H, N, d), dtype=store)
    ko = np.zeros((H, N, d), dtype=store)
    vo = np.zeros((H, N, d), dtype=store)
    salient: Dict[int, np.ndarray] = {}
    for h in (range(H) if heads is None else heads):
        sw, sq, ss, sp = per_head[h]
        rng_qkv = np.random.default_rng(sq)
        q = rng_qkv.standard_normal((N, d), dtype=np.float32)
        k = rng_qkv.standard_normal((N, d), dtype=np.float32)
        v = rng_qkv.standard_normal((N, d), dtype=np.float32)
        if roles[h] == ROLE_CORRESPONDENCE:
            W = (np.random.default_rng(sw).standard_normal((Df, d)) / math.sqrt(Df)).astype(np.float32)
            zw = z @ W
            q[patch_tok] = zw[lat] + np.float32(0.1) * q[patch_tok]
            k[patch_tok] = zw[lat] + np.float32(0.1) * k[patch_tok]
        elif roles[h] == ROLE_VERTICAL:
            u = np.random.default_rng(sp).standard_normal(d)
            u = (u / np.linalg.norm(u)).astype(np.float32)
            rs = np.random.default_rng(ss)
            sal = np.sort(patch_tok[rs.choice(S * P, size=min(N_SALIENT, S * P), replace=False)])
            k[sal] += np.float32(4.0) * u
            q += u
            salient[h] = sal
        qo[h] = _encode(q, dtype)
        ko[h] = _encode(k, dtype)
        vo[h] = _encode(v, dtype)
    if anchors is None:
        anchors = [0] * H
    plan = [(int(roles[h]), int(budgets[h]), int(anchors[h]), 0) for h in range(H)]
    return Workload(name=name, geom=geom, dtype=dtype, plan=plan, q=qo, k=ko, v=vo,
                    dino=dino_arr, Df=Df, corr_K=corr_K, lat=lat, salient=salient, seed=seed)


def layer_roles(cid: int, layer: int = 0) -> Tuple[List[int], List[int]]:
    """(roles, budgets) of the 16 heads of one measured configuration (one
    layer of config 4's stack: roles permuted by rng(4000 + layer))."""
    c = CONFIGS[cid]
    roles = list(c["roles"])
    if cid == 4:
        if layer in c["corr_layers"]:
            roles = list(c["corr_roles"])
        roles = [roles[i] for i in np.random.default_rng(4000 + layer).permutation(len(roles))]
    budgets = [_budget(r, c["vert_K"], c["corr_K"], c["scan_s"]) for r in roles]
    return roles, budgets


def make_layer(cid: int, layer: int = 0, dino: bool = True,
               heads: Optional[Sequence[int]] = None) -> Workload:
    """Inputs of one measured configuration (one layer of config 4's stack)."""
    c = CONFIGS[cid]
    geom = Geometry(S=c["S"], ns=c["ns"], P=c["P"])
    roles, budgets = layer_roles(cid, layer)
    qkv_seed = None
    name = c["name"]
    if cid == 4:
        qkv_seed = 100 + layer
        name = f"{name}_L{layer}"
    return make_geometry_inputs(geom, c["dtype"], roles, budgets, c["M"], c["Df"], seed=cid,
                                qkv_seed=qkv_seed, corr_K=c["corr_K"], name=name, dino=dino, heads=heads)


def make_inputs(cid: int, layer: int = 0, dino: bool = True,
                heads: Optional[Sequence[int]] = None) -> Workload:
    return make_layer(cid, layer, dino, heads)


def sample_rows(geom: Geometry, n_target: int, seed: int = 12345) -> np.ndarray:
    """Deterministic query-row sample for checks at full size.

    Always includes every special-token row, every row of frame 0, the first
    and last rows of every frame, and the last token; the rest is a seeded
    uniform draw, sorted ascending.
    """
    N, T, ns = geom.N, geom.T, geom.ns
    must = [np.arange(geom.S, dtype=np.int64)[:, None] * T + np.arange(ns)[None, :]]
    must.append(np.arange(min(T, N), dtype=np.int64))
    must.append(np.arange(geom.S, dtype=np.int64) * T + T - 1)
    must.append(np.array([N - 1], dtype=np.int64))
    base = np.unique(np.concatenate([m.reshape(-1) for m in must]))
    extra = max(0, n_target - base.size)
    rng = np.random.default_rng(seed)
    if extra:
        pick = rng.choice(N, size=min(extra, N), replace=False)
        base = np.unique(np.concatenate([base, pick.astype(np.int64)]))
    return base


def make_front_loaded_dino(S: int, P: int, Df: int, first_frames: int, n_rows: int, copies: int,
                           seed: int) -> Tuple[np.ndarray, np.ndarray]:
    """bf16 features [S*P, Df] of i.i.d. N(0, 1) draws, except that n_rows
    patches of frames >= first_frames each get `copies` near-copies (the
    patch plus N(0, 0.05^2) noise) among the patches of frames
    [0, first_frames).  Returns (features as bf16 bits, the n_rows patches).
    Such rows have their best matches concentrated in the first frames."""
    rng = np.random.default_rng(seed)
    F = rng.standard_normal((S * P, Df), dtype=np.float32)
    front = first_frames * P
    if n_rows * copies > front:
        raise ValueError("not enough patches in the first frames for the copies")
    rows = np.sort(rng.choice(np.arange(front, S * P), n_rows, replace=False))
    slots = rng.permutation(front)[:n_rows * copies].reshape(n_rows, copies)
    for r, sl in zip(rows, slots):
        F[sl] = F[r] + np.float32(0.05) * rng.standard_normal((copies, Df), dtype=np.float32)
    return bf16_round(F), rows


def make_grouped_front_dino(S: int, P: int, Df: int, first_frames: int, groups: int, group_size: int,
                            copies: int, seed: int) -> Tuple[np.ndarray, np.ndarray]:
    """bf16 features [S*P, Df] of i.i.d. N(0, 1) draws, except for `groups`
    latent directions z_g ~ N(0, I): group g puts `group_size` noisy copies
    (z_g + N(0, 0.05^2)) at random patches of frames >= first_frames and
    `copies` more at random patches of frames [0, first_frames).  Returns
    (features as bf16 bits, the late patches of every group, sorted)."""
    rng = np.random.default_rng(seed)
    F = rng.standard_normal((S * P, Df), dtype=np.float32)
    front = first_frames * P
    if groups * copies > front or groups * group_size > S * P - front:
        raise ValueError("not enough patches for the groups")
    early = rng.permutation(front)[:groups * copies].reshape(groups, copies)
    late = (front + rng.permutation(S * P - front)[:groups * group_size]).reshape(groups, group_size)
    for gi in range(groups):
        z = rng.standard_normal(Df, dtype=np.float32)
        for idx in (early[gi], late[gi]):
            F[idx] = z + np.float32(0.05) * rng.standard_normal((idx.size, Df), dtype=np.float32)
    return bf16_round(F), np.sort(late.reshape(-1))
