"""Head-wise dynamic sparse global attention on MI355X (gfx950).

Thin ctypes binding of ``libsaf3r.so`` (declared in ``include/saf3r.h``).
The raw C entry points are exposed under their C names (``saf_create``,
``saf_sparse_attention`` ...); ``Context`` marshals torch tensors (device
pointers, strides, the current HIP stream) into those calls.  Every step of
the computation runs in the library's HIP kernels; there is no CPU or
PyTorch fallback: if the library is missing, loading fails with an error.

torch is imported before the library is loaded so that both resolve the same
HIP runtime (libamdhip64.so.7).
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsaf3r.so")

SAF_OK, SAF_EINVAL, SAF_ENOMEM, SAF_EHIP, SAF_EUNSUPPORTED, SAF_ESTATE = 0, -1, -2, -3, -4, -5
SAF_F32, SAF_BF16 = 0, 1
SAF_POSITION, SAF_VERTICAL, SAF_CORRESPONDENCE, SAF_SCANNING, SAF_DENSE = 0, 1, 2, 3, 4
SAF_CORR_STRIDE = 5
SAF_BROADCAST = 6
SAF_CORR_TOTAL, SAF_CORR_PER_FRAME, SAF_CORR_PER_FRAME_STORED = 0, 1, 2

_STATUS_NAMES = {0: "SAF_OK", -1: "SAF_EINVAL", -2: "SAF_ENOMEM", -3: "SAF_EHIP",
                 -4: "SAF_EUNSUPPORTED", -5: "SAF_ESTATE"}


class saf_geometry_t(C.Structure):
    _fields_ = [("num_frames", C.c_int32), ("specials_per_frame", C.c_int32),
                ("patches_per_frame", C.c_int32), ("num_heads", C.c_int32),
                ("head_dim", C.c_int32), ("dtype", C.c_int32)]


class saf_layout_t(C.Structure):
    _fields_ = [("head_stride", C.c_int64), ("token_stride", C.c_int64)]


class saf_head_plan_t(C.Structure):
    _fields_ = [("role", C.c_int32), ("budget", C.c_int32), ("anchor_frame", C.c_int32),
                ("flags", C.c_int32)]


class SafError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


_lib = None
_VP, _I32, _I64, _SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
_PROTOS = {
    "saf_create": (C.c_int, [C.POINTER(saf_geometry_t), C.POINTER(_VP)]),
    "saf_destroy": (None, [_VP]),
    "saf_last_error": (C.c_char_p, [_VP]),
    "saf_workspace_size": (C.c_int, [_VP, _VP, C.POINTER(_SZ)]),
    "saf_build_corr_index": (C.c_int, [_VP, _VP, _I32, _I32, _I64, _I32, _I32, _VP]),
    "saf_build_corr_index_blocks": (C.c_int, [_VP, _VP, _I32, _I32, _I64, _I32, _I32, _I32, _VP]),
    "saf_build_corr_index_qk": (C.c_int, [_VP, _VP, _VP, saf_layout_t, _I32, _I32, _I32, _VP]),
    "saf_head_nmse": (C.c_int, [_VP, _VP, _VP, saf_layout_t, _VP, _VP]),
    "saf_head_nmse_accumulate": (C.c_int, [_VP, _VP, _VP, saf_layout_t, C.c_double, _VP, _I64, _VP]),
    "saf_head_pairs": (C.c_int, [_VP, C.POINTER(saf_head_plan_t), _I32, C.POINTER(C.c_int64)]),
    "saf_head_cost": (C.c_int, [_VP, C.POINTER(saf_head_plan_t), _I32, C.POINTER(C.c_double)]),
    "saf_profile_select": (C.c_int32, [C.POINTER(C.c_double), C.POINTER(C.c_double), _I32]),
    "saf_baseline_stride": (C.c_int32, [C.c_double]),
    "saf_set_corr_index": (C.c_int, [_VP, _VP, _I32, _VP]),
    "saf_get_corr_index": (C.c_int, [_VP, _VP, C.POINTER(_I32), _VP]),
    "saf_corr_recomputed_rows": (C.c_int, [_VP, _VP, _I32, C.POINTER(_I32), _VP]),
    "saf_build_vertical_index": (C.c_int, [_VP, _VP, _VP, saf_layout_t, _I32, _I32, _VP, _VP, _SZ, _VP]),
    "saf_sparse_attention": (C.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, saf_layout_t, _VP, _I64, _VP, _SZ, _VP]),
    "saf_dense_attention": (C.c_int, [_VP, _VP, _VP, _VP, _VP, saf_layout_t, _VP, _SZ, _VP]),
    "saf_sparse_attention_noalloc": (C.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, saf_layout_t, _VP, _I64, _VP]),
    "saf_debug_fail_alloc": (C.c_int, [_I32]),
    "saf_set_kernel_timing": (C.c_int, [_VP, _I32]),
    "saf_read_kernel_timing": (C.c_int, [_VP, _I32, C.POINTER(C.c_char_p), C.POINTER(C.c_float),
                                         C.POINTER(_I32)]),
}


def lib() -> C.CDLL:
    """Load libsaf3r.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with head_wise_dynamic_amd._build "
                               "(or __graft_entry__.build()); there is no fallback path")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _PROTOS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def exported_symbols() -> Sequence[str]:
    return tuple(_PROTOS)


# Raw C entry points under their C names (argument marshalling is the caller's).
def saf_create(geometry: saf_geometry_t, out: C.c_void_p) -> int:
    return lib().saf_create(C.byref(geometry), C.byref(out))


def saf_destroy(ctx) -> None:
    lib().saf_destroy(ctx)


def saf_last_error(ctx) -> str:
    return (lib().saf_last_error(ctx) or b"").decode()


def saf_workspace_size(ctx, plan, nbytes: C.c_size_t) -> int:
    return lib().saf_workspace_size(ctx, plan, C.byref(nbytes))


def saf_build_corr_index(ctx, dino, dino_dtype, Df, row_stride, K, mode, stream) -> int:
    return lib().saf_build_corr_index(ctx, dino, dino_dtype, Df, row_stride, K, mode, stream)


def saf_build_corr_index_blocks(ctx, dino, dino_dtype, Df, row_stride, block, K, mode, stream) -> int:
    return lib().saf_build_corr_index_blocks(ctx, dino, dino_dtype, Df, row_stride, block, K, mode, stream)


def saf_build_corr_index_qk(ctx, q, k, layout, head, K, mode, stream) -> int:
    return lib().saf_build_corr_index_qk(ctx, q, k, layout, head, K, mode, stream)


def saf_head_nmse(ctx, o_full, o_sparse, layout, dev_out, stream) -> int:
    return lib().saf_head_nmse(ctx, o_full, o_sparse, layout, dev_out, stream)


def saf_head_nmse_accumulate(ctx, o_full, o_sparse, layout, weight, dev_err, err_stride, stream) -> int:
    return lib().saf_head_nmse_accumulate(ctx, o_full, o_sparse, layout, weight, dev_err, err_stride, stream)


def saf_head_pairs(ctx, head, corr_kc, pairs) -> int:
    return lib().saf_head_pairs(ctx, head, corr_kc, pairs)


def saf_head_cost(ctx, head, corr_kc, flops) -> int:
    return lib().saf_head_cost(ctx, head, corr_kc, flops)


def saf_profile_select(errors, costs, n) -> int:
    return lib().saf_profile_select(errors, costs, n)


def saf_baseline_stride(sigma) -> int:
    return lib().saf_baseline_stride(sigma)


def saf_set_corr_index(ctx, dev_idx, Kc, stream) -> int:
    return lib().saf_set_corr_index(ctx, dev_idx, Kc, stream)


def saf_get_corr_index(ctx, dev_out, Kc: C.c_int32, stream) -> int:
    return lib().saf_get_corr_index(ctx, dev_out, C.byref(Kc), stream)


def saf_corr_recomputed_rows(ctx, host_rows, max_rows, count: C.c_int32, stream) -> int:
    return lib().saf_corr_recomputed_rows(ctx, host_rows, max_rows, C.byref(count), stream)


def saf_build_vertical_index(ctx, q, k, layout, head, K, dev_idx_out, ws, ws_bytes, stream) -> int:
    return lib().saf_build_vertical_index(ctx, q, k, layout, head, K, dev_idx_out, ws, ws_bytes, stream)


def saf_sparse_attention(ctx, plan, q, k, v, o, layout, vert_idx, vert_ld, ws, ws_bytes, stream) -> int:
    return lib().saf_sparse_attention(ctx, plan, q, k, v, o, layout, vert_idx, vert_ld, ws, ws_bytes, stream)


def saf_sparse_attention_noalloc(ctx, plan, q, k, v, o, layout, vert_idx, vert_ld, stream) -> int:
    return lib().saf_sparse_attention_noalloc(ctx, plan, q, k, v, o, layout, vert_idx, vert_ld, stream)


def saf_dense_attention(ctx, q, k, v, o, layout, ws, ws_bytes, stream) -> int:
    return lib().saf_dense_attention(ctx, q, k, v, o, layout, ws, ws_bytes, stream)


def saf_debug_fail_alloc(allowed) -> int:
    return lib().saf_debug_fail_alloc(allowed)


def saf_set_kernel_timing(ctx, enable) -> int:
    return lib().saf_set_kernel_timing(ctx, enable)


def saf_read_kernel_timing(ctx, max_entries, names, ms, count: C.c_int32) -> int:
    return lib().saf_read_kernel_timing(ctx, max_entries, names, ms, C.byref(count))


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------
_DT = {torch.float32: SAF_F32, torch.bfloat16: SAF_BF16}


def make_plan(plan: Sequence[Tuple[int, int, int, int]]):
    arr = (saf_head_plan_t * len(plan))()
    for i, p in enumerate(plan):
        role, budget, anchor, flags = (tuple(p) + (0, 0, 0, 0))[:4]
        arr[i] = saf_head_plan_t(int(role), int(budget), int(anchor), int(flags))
    return arr


def _stream(stream: Optional[torch.cuda.Stream]):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


class Context:
    """One geometry (S frames of ns special + P patch tokens, H heads of 64)."""

    def __init__(self, S: int, ns: int, P: int, H: int = 16, d: int = 64,
                 dtype: torch.dtype = torch.bfloat16):
        self.S, self.ns, self.P, self.H, self.d = S, ns, P, H, d
        self.T = ns + P
        self.N = S * self.T
        self.Np = S * P
        self.dtype = dtype
        self._ctx = C.c_void_p()
        geom = saf_geometry_t(S, ns, P, H, d, _DT.get(dtype, 99))
        self._check(saf_create(geom, self._ctx), None)
        self._ws = None

    def close(self):
        if self._ctx:
            saf_destroy(self._ctx)
            self._ctx = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, st: int, ctx=...):
        if st != SAF_OK:
            raise SafError(st, saf_last_error(self._ctx if ctx is ... else ctx))

    # -- tensors ------------------------------------------------------------
    def layout_of(self, t: torch.Tensor) -> saf_layout_t:
        if t.dim() != 3 or t.stride(2) != 1:
            raise ValueError("expected a 3-D tensor with contiguous channels")
        if t.shape == (self.H, self.N, self.d):
            return saf_layout_t(t.stride(0), t.stride(1))
        if t.shape == (self.N, self.H, self.d):
            return saf_layout_t(t.stride(1), t.stride(0))
        raise ValueError(f"tensor shape {tuple(t.shape)} is neither [H,N,d] nor [N,H,d]")

    def _tensors(self, q: torch.Tensor, *others) -> saf_layout_t:
        """Layout of q after checking q and every (name, tensor) in others.

        The library takes one layout and one dtype for q, k, v and o, so every
        tensor must match q's shape and strides, carry the context's dtype and
        live on q's GPU; any mismatch would read or write out of bounds.
        Checked in that order (shapes, dtypes, devices), for all tensors."""
        if not isinstance(q, torch.Tensor) or not all(isinstance(t, torch.Tensor) for _, t in others):
            raise TypeError("q, k, v and o must be torch tensors")
        lay = self.layout_of(q)
        named = [("q", q)] + list(others)
        for name, t in named[1:]:
            if tuple(t.shape) != tuple(q.shape) or tuple(t.stride()) != tuple(q.stride()):
                raise ValueError(f"{name} has shape {tuple(t.shape)} / strides {tuple(t.stride())}; expected "
                                 f"{tuple(q.shape)} / {tuple(q.stride())} like q")
        for name, t in named:
            if t.dtype != self.dtype:
                raise ValueError(f"{name} has dtype {t.dtype}, the context computes in {self.dtype}")
        for name, t in named:
            if t.device != q.device or t.device.type != "cuda":
                raise ValueError(f"{name} is on {t.device}; expected q's GPU (q is on {q.device})")
        return lay

    def _rows_of(self, t: torch.Tensor, name: str, rows: int, device=None) -> None:
        if t.shape[0] != rows:
            raise ValueError(f"{name} has {t.shape[0]} rows; expected {rows}")
        if t.device.type != "cuda" or (device is not None and t.device != device):
            raise ValueError(f"{name} must be a GPU tensor" + (f" on {device}" if device is not None else ""))

    def workspace(self, nbytes: int, device) -> torch.Tensor:
        if self._ws is None or self._ws.numel() < nbytes or self._ws.device != device:
            self._ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        return self._ws

    def workspace_size(self, plan) -> int:
        n = C.c_size_t()
        self._check(saf_workspace_size(self._ctx, make_plan(plan) if plan is not None else None, n))
        return n.value

    # -- index builders -----------------------------------------------------
    def build_corr_index(self, dino: torch.Tensor, K: int, mode: int = SAF_CORR_TOTAL, stream=None):
        if dino.dim() != 2 or dino.stride(1) != 1:
            raise ValueError("dino must be [S*P, Df] with contiguous channels")
        self._rows_of(dino, "dino", self.Np)
        self._check(saf_build_corr_index(self._ctx, C.c_void_p(dino.data_ptr()), _DT.get(dino.dtype, 99),
                                         dino.shape[1], dino.stride(0), K, mode, _stream(stream)))

    def build_corr_index_blocks(self, dino: torch.Tensor, block: int, K: int, mode: int = SAF_CORR_TOTAL,
                                stream=None):
        if dino.dim() != 2 or dino.stride(1) != 1:
            raise ValueError("dino must be [S*P, Df] with contiguous channels")
        self._rows_of(dino, "dino", self.Np)
        self._check(saf_build_corr_index_blocks(self._ctx, C.c_void_p(dino.data_ptr()), _DT.get(dino.dtype, 99),
                                                dino.shape[1], dino.stride(0), block, K, mode, _stream(stream)))

    def build_corr_index_qk(self, q: torch.Tensor, k: torch.Tensor, head: int, K: int, mode: int = SAF_CORR_TOTAL,
                            stream=None):
        lay = self._tensors(q, ("k", k))
        self._check(saf_build_corr_index_qk(self._ctx, C.c_void_p(q.data_ptr()), C.c_void_p(k.data_ptr()), lay, head,
                                            K, mode, _stream(stream)))

    def set_corr_index(self, idx: torch.Tensor, stream=None):
        if idx.dtype != torch.int32 or idx.dim() != 2 or not idx.is_contiguous():
            raise ValueError("index must be a contiguous int32 [S*P, Kc] tensor")
        self._rows_of(idx, "index", self.Np)
        self._check(saf_set_corr_index(self._ctx, C.c_void_p(idx.data_ptr()), idx.shape[1], _stream(stream)))

    def corr_k(self) -> int:
        kc = C.c_int32()
        self._check(saf_get_corr_index(self._ctx, None, kc, None))
        return kc.value

    def get_corr_index(self, device="cuda", stream=None) -> torch.Tensor:
        kc = self.corr_k()
        out = torch.empty((self.Np, kc), dtype=torch.int32, device=device)
        self._check(saf_get_corr_index(self._ctx, C.c_void_p(out.data_ptr()), C.c_int32(), _stream(stream)))
        return out

    def recomputed_rows(self, stream=None):
        """Patch numbers the last index build recomputed exactly (sorted): total
        mode on the matrix-core engine, or the fused per-frame build."""
        cnt = C.c_int32()
        self._check(saf_corr_recomputed_rows(self._ctx, None, 0, cnt, _stream(stream)))
        n = cnt.value
        buf = (C.c_int32 * max(n, 1))()
        self._check(saf_corr_recomputed_rows(self._ctx, buf, n, cnt, _stream(stream)))
        return sorted(buf[i] for i in range(min(n, cnt.value)))

    def build_vertical_index(self, q: torch.Tensor, k: torch.Tensor, head: int, K: int, stream=None):
        lay = self._tensors(q, ("k", k))
        plan = [(SAF_VERTICAL, K, 0, 0)] + [(SAF_DENSE, 0, 0, 0)] * (self.H - 1)
        ws = self.workspace(self.workspace_size(plan), q.device)
        out = torch.empty(min(K, self.N), dtype=torch.int32, device=q.device)
        self._check(saf_build_vertical_index(self._ctx, C.c_void_p(q.data_ptr()), C.c_void_p(k.data_ptr()),
                                             lay, head, K, C.c_void_p(out.data_ptr()),
                                             C.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream)))
        return out

    # -- attention ----------------------------------------------------------
    def sparse_attention(self, plan, q, k, v, o=None, vert_idx: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
        if len(plan) != self.H:
            raise ValueError(f"plan has {len(plan)} entries; the context has {self.H} heads")
        if o is None:
            o = torch.empty_like(q)
        lay = self._tensors(q, ("k", k), ("v", v), ("o", o))
        cplan = make_plan(plan)
        need = self.workspace_size(plan)
        ws = self.workspace(need, q.device)
        vptr, vld = None, 0
        if vert_idx is not None:
            if vert_idx.dtype != torch.int32 or vert_idx.dim() != 2 or not vert_idx.is_contiguous():
                raise ValueError("vert_idx must be a contiguous int32 [H, ld] tensor")
            self._rows_of(vert_idx, "vert_idx", self.H, q.device)
            vptr, vld = C.c_void_p(vert_idx.data_ptr()), vert_idx.shape[1]
        self._check(saf_sparse_attention(self._ctx, cplan, C.c_void_p(q.data_ptr()), C.c_void_p(k.data_ptr()),
                                         C.c_void_p(v.data_ptr()), C.c_void_p(o.data_ptr()), lay, vptr, vld,
                                         C.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream)))
        return o

    def set_kernel_timing(self, enable: bool = True):
        self._check(saf_set_kernel_timing(self._ctx, 1 if enable else 0))

    def read_kernel_timing(self, max_entries: int = 4096):
        """[(launch group name, ms)] recorded since the last read (after a sync)."""
        names = (C.c_char_p * max_entries)()
        ms = (C.c_float * max_entries)()
        cnt = C.c_int32()
        self._check(saf_read_kernel_timing(self._ctx, max_entries, names, ms, cnt))
        return [(names[i].decode(), float(ms[i])) for i in range(min(cnt.value, max_entries))]

    def head_nmse(self, o_full: torch.Tensor, o_sparse: torch.Tensor, out: torch.Tensor = None, stream=None):
        """[H, 2] float64 (device): per head sum (o_full - o_sparse)^2 and sum o_full^2."""
        lay = self._tensors(o_full, ("o_sparse", o_sparse))
        if out is None:
            out = torch.empty((self.H, 2), dtype=torch.float64, device=o_full.device)
        if out.dtype != torch.float64 or out.numel() < 2 * self.H or not out.is_contiguous() or \
                out.device != o_full.device:
            raise ValueError("out must be a contiguous float64 GPU tensor of at least 2H elements")
        self._check(saf_head_nmse(self._ctx, C.c_void_p(o_full.data_ptr()), C.c_void_p(o_sparse.data_ptr()), lay,
                                  C.c_void_p(out.data_ptr()), _stream(stream)))
        return out

    def head_nmse_accumulate(self, o_full: torch.Tensor, o_sparse: torch.Tensor, err: torch.Tensor,
                             weight: float, stream=None) -> torch.Tensor:
        """err[h] += weight * ||o_full[h] - o_sparse[h]||^2 / ||o_full[h]||^2 (Eq. 1,
        in the library).  err: float64 GPU tensor of H elements (any stride, e.g.
        a column of an [H, configurations] table)."""
        lay = self._tensors(o_full, ("o_sparse", o_sparse))
        if err.dtype != torch.float64 or err.dim() != 1 or err.shape[0] != self.H or err.stride(0) < 1 or \
                err.device != o_full.device:
            raise ValueError("err must be a float64 GPU vector of H elements")
        self._check(saf_head_nmse_accumulate(self._ctx, C.c_void_p(o_full.data_ptr()),
                                             C.c_void_p(o_sparse.data_ptr()), lay, float(weight),
                                             C.c_void_p(err.data_ptr()), err.stride(0), _stream(stream)))
        return err

    def head_pairs(self, role: int, budget: int = 0, anchor: int = 0, corr_kc: int = 0) -> int:
        n = C.c_int64()
        h = saf_head_plan_t(role, budget, anchor, 0)
        self._check(saf_head_pairs(self._ctx, C.byref(h), corr_kc, C.byref(n)))
        return n.value

    def head_cost(self, role: int, budget: int = 0, anchor: int = 0, corr_kc: int = 0) -> float:
        """Eq. 2's cost of one head under (role, budget, anchor): FLOPs."""
        f = C.c_double()
        h = saf_head_plan_t(role, budget, anchor, 0)
        self._check(saf_head_cost(self._ctx, C.byref(h), corr_kc, C.byref(f)))
        return f.value

    def dense_attention(self, q, k, v, o=None, stream=None) -> torch.Tensor:
        if o is None:
            o = torch.empty_like(q)
        lay = self._tensors(q, ("k", k), ("v", v), ("o", o))
        need = self.workspace_size(None)
        ws = self.workspace(need, q.device) if need else None
        self._check(saf_dense_attention(self._ctx, C.c_void_p(q.data_ptr()), C.c_void_p(k.data_ptr()),
                                        C.c_void_p(v.data_ptr()), C.c_void_p(o.data_ptr()), lay,
                                        C.c_void_p(ws.data_ptr()) if ws is not None else None,
                                        ws.numel() if ws is not None else 0, _stream(stream)))
        return o
