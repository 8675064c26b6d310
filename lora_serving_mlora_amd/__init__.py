"""Python binding of libmlora.so, the MI355X heterogeneous multi-LoRA linear.

Argument marshalling only: every step of the layer runs in the HIP kernels
behind include/mlora.h.  torch is used for device memory (tensors give
pointers) and streams (the current stream is passed to every call).  There
is no CPU fallback: if the library is missing, every call raises.

Typical use::

    pool = Pool(din, dout, n_proj, max_adapters, max_rank, n_pages)
    pool.load(adapter_id, rank, scale, down_bits, up_bits)   # host bf16 bits
    seg = build_segments(pool, row_adapter)                  # device int32 [n]
    Y = apply(pool, proj, X, W0, seg)                        # device bf16
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

__all__ = [
    "MloraError", "lib", "Pool", "build_segments", "segments_header", "segments_status", "read_segments",
    "base_gemm", "shrink", "shrink_max_chunks", "expand", "fused", "shrink_rows", "gemm_lora", "new_work", "rows_t", "apply", "forward", "plan", "work_bytes",
    "forward_static", "STATIC_SCRATCH_BYTES", "merge", "hbm_copy", "hbm_read", "hbm_read_lds", "timing_arm", "timing_read", "VARIANTS", "ITEM_ROWS", "TILE_ROWS", "MAX_ROWS", "MAX_RANK", "SEG", "EXPORTS", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmlora.so")

OK, EINVAL, ENOSPC, EEXIST, ENOENT, EHIP = range(6)
VARIANTS = {"auto": 0, "split": 1, "fused": 2, "rows": 3}
ITEM_ROWS = 4
TILE_ROWS = 64
MAX_ROWS = 16384
MAX_RANK = 128
SEG = dict(nseg=0, n_act=1, n_none=2, n_bad=3, status=4, n_items=5, n_rows=6, max_adapters=7, n_tiles=8)
SEG_HEADER = 16
SEG_BAD_ID, SEG_NOT_RESIDENT = 1, 2  # bits of the status word

_c_void_p, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_pi32, _pi64, _pf32 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_float)


class _PoolDesc(ctypes.Structure):
    _fields_ = [("din", _i32), ("dout", _i32), ("n_proj", _i32), ("max_adapters", _i32), ("max_rank", _i32),
                ("reserved", _i32), ("n_down_pages", _i64), ("n_up_pages", _i64), ("down_pages", _c_void_p),
                ("up_pages", _c_void_p), ("meta", _c_void_p)]


# name -> (restype, argtypes); every symbol include/mlora.h declares
EXPORTS = {
    "mlora_version": (ctypes.c_char_p, []),
    "mlora_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "mlora_last_error": (ctypes.c_char_p, []),
    "mlora_pool_meta_bytes": (_sz, [_i32, _i32, _i32]),
    "mlora_pool_create": (ctypes.c_int, [ctypes.POINTER(_PoolDesc), _c_void_p, ctypes.POINTER(_c_void_p)]),
    "mlora_pool_destroy": (ctypes.c_int, [_c_void_p]),
    "mlora_pool_load": (ctypes.c_int, [_c_void_p, _i32, _i32, _f32, _c_void_p, _c_void_p, _c_void_p]),
    "mlora_pool_unload": (ctypes.c_int, [_c_void_p, _i32, _c_void_p]),
    "mlora_pool_ready": (ctypes.c_int, [_c_void_p, _i32, _c_void_p]),
    "mlora_pool_query": (ctypes.c_int, [_c_void_p, _i32, _pi32, _pf32]),
    "mlora_pool_free_pages": (ctypes.c_int, [_c_void_p, _pi64, _pi64, _pi32]),
    "mlora_pool_fail_next_load": (ctypes.c_int, [_c_void_p, _i32]),
    "mlora_segments_bytes": (_sz, [_i32]),
    "mlora_build_segments": (ctypes.c_int, [_c_void_p, _c_void_p, _i32, _c_void_p, _c_void_p]),
    "mlora_segments_header": (ctypes.c_int, [_c_void_p, _pi32, _c_void_p]),
    "mlora_segments_status": (ctypes.c_int, [_c_void_p, _pi32, _c_void_p]),
    "mlora_base_gemm": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32, _c_void_p]),
    "mlora_shrink_max_chunks": (_i32, [_i32]),
    "mlora_shrink": (ctypes.c_int, [_c_void_p, _i32, _c_void_p, _c_void_p, _i32, _c_void_p, _i32, _c_void_p]),
    "mlora_expand": (ctypes.c_int, [_c_void_p, _i32, _c_void_p, _i32, _c_void_p, _c_void_p, _i32, _c_void_p]),
    "mlora_fused": (ctypes.c_int, [_c_void_p, _i32, _c_void_p, _c_void_p, _c_void_p, _i32, _c_void_p]),
    "mlora_work_bytes": (_sz, [_c_void_p, _i32]),
    "mlora_shrink_rows": (ctypes.c_int, [_c_void_p, _i32, _c_void_p, _c_void_p, _i32, _c_void_p, _sz, _c_void_p]),
    "mlora_gemm_lora": (ctypes.c_int, [_c_void_p, _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _sz, _c_void_p,
                                       _i32, _c_void_p]),
    "mlora_plan": (ctypes.c_int, [_c_void_p, _i32, _i32, _pi32, _pi32]),
    "mlora_apply": (ctypes.c_int, [_c_void_p, _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _c_void_p,
                                   _sz, _i32, _c_void_p]),
    "mlora_forward": (ctypes.c_int, [_c_void_p, _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32,
                                     _c_void_p, _sz, _i32, _c_void_p]),
    "mlora_forward_static": (ctypes.c_int, [_c_void_p, _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                            _i32, _i32, _c_void_p]),
    "mlora_merge": (ctypes.c_int, [_c_void_p, _i32, _i32, _c_void_p, _f32, _c_void_p]),
    "mlora_hbm_copy": (ctypes.c_int, [_c_void_p, _c_void_p, _sz, _c_void_p]),
    "mlora_hbm_read": (ctypes.c_int, [_c_void_p, _sz, _c_void_p, _c_void_p]),
    "mlora_hbm_read_lds": (ctypes.c_int, [_c_void_p, _sz, _c_void_p, _c_void_p]),
    "mlora_timing_arm": (ctypes.c_int, [ctypes.c_int32]),
    "mlora_timing_read": (ctypes.c_int, [ctypes.POINTER(ctypes.c_float), ctypes.c_int32,
                                         ctypes.POINTER(ctypes.c_int32)]),
    "mlora_timing_name": (ctypes.c_char_p, [ctypes.c_int32]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use).  Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m lora_serving_mlora_amd.build` "
                               "(the multi-LoRA path has no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


class MloraError(RuntimeError):
    def __init__(self, status: int, where: str):
        L = lib()
        self.status = status
        msg = L.mlora_status_string(status).decode()
        detail = L.mlora_last_error().decode()
        super().__init__(f"{where}: {msg}" + (f" ({detail})" if detail else ""))


def _check(status: int, where: str) -> None:
    if status != OK:
        raise MloraError(status, where)


def _torch():
    import torch
    return torch


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def _bf16_dev(t, name: str):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous bfloat16 CUDA tensor")
    return t


def _host_bits(a, shape, name: str) -> np.ndarray:
    """bf16 data on the host as a C-contiguous uint16 array of `shape`."""
    torch = _torch()
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu()
        if a.dtype == torch.bfloat16:
            a = a.view(torch.int16)
        a = a.numpy()
    a = np.asarray(a)
    if a.dtype not in (np.int16, np.uint16):
        raise TypeError(f"{name} must hold bf16 bit patterns (uint16/int16 array or bfloat16 tensor)")
    a = np.ascontiguousarray(a).view(np.uint16)
    if tuple(a.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(a.shape)}, expected {tuple(shape)}")
    return a


class Pool:
    """A rank-stacked paged adapter pool on the current device.

    One page is one rank row of one adapter for one projection (Down rows of
    din, Up^T rows of dout).  n_pages pages are allocated in each arena."""

    def __init__(self, din: int, dout: int, n_proj: int, max_adapters: int, max_rank: int,
                 n_pages: int, n_up_pages: Optional[int] = None):
        torch = _torch()
        L = lib()
        self.din, self.dout, self.n_proj = din, dout, n_proj
        self.max_adapters, self.max_rank = max_adapters, max_rank
        n_up = n_pages if n_up_pages is None else n_up_pages
        dev = torch.device("cuda", torch.cuda.current_device())
        self.down_pages = torch.zeros((max(n_pages, 1), din), dtype=torch.bfloat16, device=dev)
        self.up_pages = torch.zeros((max(n_up, 1), dout), dtype=torch.bfloat16, device=dev)
        mb = L.mlora_pool_meta_bytes(max_adapters, n_proj, max_rank)
        self.meta = torch.empty(max(mb, 256), dtype=torch.uint8, device=dev)
        d = _PoolDesc(din, dout, n_proj, max_adapters, max_rank, 0, n_pages, n_up,
                      self.down_pages.data_ptr(), self.up_pages.data_ptr(), self.meta.data_ptr())
        h = ctypes.c_void_p()
        _check(L.mlora_pool_create(ctypes.byref(d), _stream(), ctypes.byref(h)), "mlora_pool_create")
        self._h = h

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._h is None:
            raise RuntimeError("pool is closed")
        return self._h

    def load(self, adapter_id: int, rank: int, scale: float, down, up) -> None:
        """down: bf16 bits [n_proj][rank][din]; up: bf16 bits [n_proj][dout][rank]."""
        d = _host_bits(down, (self.n_proj, rank, self.din), "down")
        u = _host_bits(up, (self.n_proj, self.dout, rank), "up")
        _check(lib().mlora_pool_load(self.handle, adapter_id, rank, ctypes.c_float(scale),
                                     d.ctypes.data_as(ctypes.c_void_p), u.ctypes.data_as(ctypes.c_void_p), _stream()),
               f"mlora_pool_load({adapter_id})")

    def unload(self, adapter_id: int) -> None:
        _check(lib().mlora_pool_unload(self.handle, adapter_id, _stream()), f"mlora_pool_unload({adapter_id})")

    def ready(self, adapter_id: int) -> None:
        """Makes the current stream wait (on the device) for the adapter's
        latest load, which may have been issued on another stream."""
        _check(lib().mlora_pool_ready(self.handle, adapter_id, _stream()), f"mlora_pool_ready({adapter_id})")

    def query(self, adapter_id: int):
        r, s = ctypes.c_int32(), ctypes.c_float()
        st = lib().mlora_pool_query(self.handle, adapter_id, ctypes.byref(r), ctypes.byref(s))
        if st == ENOENT:
            return None
        _check(st, "mlora_pool_query")
        return r.value, s.value

    def free_pages(self):
        fd, fu, nr = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
        _check(lib().mlora_pool_free_pages(self.handle, ctypes.byref(fd), ctypes.byref(fu), ctypes.byref(nr)),
               "mlora_pool_free_pages")
        return fd.value, fu.value, nr.value

    def fail_next_load(self, step: int) -> None:
        """Testing aid: the next load on this pool fails at `step` (1: before
        its last staging flush, 2: after its metadata copies; 0: off)."""
        _check(lib().mlora_pool_fail_next_load(self.handle, step), "mlora_pool_fail_next_load")

    def close(self) -> None:
        if getattr(self, "_h", None) is not None:
            _check(lib().mlora_pool_destroy(self._h), "mlora_pool_destroy")
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def segments_bytes(n: int) -> int:
    return int(lib().mlora_segments_bytes(n))


def build_segments(pool: Pool, row_adapter, seg_ws=None):
    """row_adapter: int32 CUDA tensor [n].  Returns the seg_ws tensor."""
    torch = _torch()
    if row_adapter.dtype != torch.int32 or not row_adapter.is_cuda or not row_adapter.is_contiguous():
        raise TypeError("row_adapter must be a contiguous int32 CUDA tensor")
    n = row_adapter.shape[0]
    nb = segments_bytes(n)
    if seg_ws is None:
        seg_ws = torch.empty(nb // 4, dtype=torch.int32, device=row_adapter.device)
    elif seg_ws.numel() * seg_ws.element_size() < nb:
        raise ValueError("seg_ws too small")
    _check(lib().mlora_build_segments(pool.handle, _ptr(row_adapter), n, _ptr(seg_ws), _stream()),
           "mlora_build_segments")
    return seg_ws


def segments_header(seg_ws) -> dict:
    """The header words of seg_ws (synchronises the stream)."""
    h = (ctypes.c_int32 * SEG_HEADER)()
    _check(lib().mlora_segments_header(_ptr(seg_ws), h, _stream()), "mlora_segments_header")
    return {k: int(h[i]) for k, i in SEG.items()}


def segments_status(seg_ws) -> int:
    """The batch's status word (SEG_BAD_ID | SEG_NOT_RESIDENT bits; synchronises the stream)."""
    st = ctypes.c_int32(0)
    _check(lib().mlora_segments_status(_ptr(seg_ws), ctypes.byref(st), _stream()), "mlora_segments_status")
    return int(st.value)


def read_segments(seg_ws, n: int) -> dict:
    """Copies seg_ws to the host and splits it by the documented layout."""
    w = seg_ws.cpu().numpy()
    hdr = {k: int(w[i]) for k, i in SEG.items()}
    nseg = hdr["nseg"]
    perm0, inv0, ad0, off0 = SEG_HEADER, SEG_HEADER + n, SEG_HEADER + 2 * n, SEG_HEADER + 3 * n
    items0 = (SEG_HEADER + 4 * n + 2) & ~1
    out = dict(hdr)
    max_items = n + (n + ITEM_ROWS - 1) // ITEM_ROWS + 1
    rk0 = items0 + 2 * max_items
    out["row_key"] = w[rk0:rk0 + n].copy()
    tl0 = rk0 + n
    out["tiles"] = w[tl0:tl0 + 2 * hdr["n_tiles"]].reshape(-1, 2).copy()
    out.update(perm=w[perm0:perm0 + n].copy(), inv=w[inv0:inv0 + n].copy(),
               seg_adapter=w[ad0:ad0 + nseg].copy(), seg_off=w[off0:off0 + nseg + 1].copy(),
               items=w[items0:items0 + 2 * hdr["n_items"]].reshape(-1, 2).copy())
    return out


def base_gemm(X, W0, Y=None):
    torch = _torch()
    _bf16_dev(X, "X"), _bf16_dev(W0, "W0")
    n, din = X.shape
    dout = W0.shape[0]
    if W0.shape[1] != din:
        raise ValueError("X and W0 disagree on din")
    if Y is None:
        Y = torch.empty((n, dout), dtype=torch.bfloat16, device=X.device)
    _bf16_dev(Y, "Y")
    if tuple(Y.shape) != (n, dout):
        raise ValueError("Y has the wrong shape")
    _check(lib().mlora_base_gemm(_ptr(X), _ptr(W0), _ptr(Y), n, din, dout, _stream()), "mlora_base_gemm")
    return Y


def shrink_max_chunks(din: int) -> int:
    return int(lib().mlora_shrink_max_chunks(din))


def _rows_check(pool: Pool, X, n: int):
    _bf16_dev(X, "X")
    if tuple(X.shape) != (n, pool.din):
        raise ValueError(f"X must be [{n}][{pool.din}]")


def shrink(pool: Pool, proj: int, X, seg_ws, n_chunks: int = 1, T=None):
    """Returns T, fp32 [n_chunks][n][max_rank] partial t in sorted-row order."""
    torch = _torch()
    n = X.shape[0]
    _rows_check(pool, X, n)
    if T is None:
        T = torch.zeros((n_chunks, n, pool.max_rank), dtype=torch.float32, device=X.device)
    _check(lib().mlora_shrink(pool.handle, proj, _ptr(X), _ptr(seg_ws), n, _ptr(T), n_chunks, _stream()),
           "mlora_shrink")
    return T


def expand(pool: Pool, proj: int, T, seg_ws, Y):
    """Y[perm[j]] += s * Up t_j (in place), t_j summed over T's chunks."""
    torch = _torch()
    _bf16_dev(Y, "Y")
    n = Y.shape[0]
    if T.dtype != torch.float32 or T.dim() != 3 or tuple(T.shape[1:]) != (n, pool.max_rank) or not T.is_contiguous():
        raise ValueError(f"T must be contiguous fp32 [chunks][{n}][{pool.max_rank}]")
    _check(lib().mlora_expand(pool.handle, proj, _ptr(T), T.shape[0], _ptr(seg_ws), _ptr(Y), n, _stream()),
           "mlora_expand")
    return Y


def fused(pool: Pool, proj: int, X, seg_ws, Y):
    n = X.shape[0]
    _rows_check(pool, X, n)
    _bf16_dev(Y, "Y")
    _check(lib().mlora_fused(pool.handle, proj, _ptr(X), _ptr(seg_ws), _ptr(Y), n, _stream()), "mlora_fused")
    return Y


def new_work(pool: Pool, n: int, device=None):
    """A zeroed work buffer for apply / the per-row path (mlora_work_bytes)."""
    torch = _torch()
    return torch.zeros(max(work_bytes(pool, n), 256), dtype=torch.uint8,
                       device=device if device is not None else torch.device("cuda", torch.cuda.current_device()))


def rows_t(pool: Pool, work, n: int):
    """The T region of a per-row work buffer: fp32 [n][max_rank] view."""
    torch = _torch()
    return work[: n * pool.max_rank * 4].view(torch.float32).view(n, pool.max_rank)


def shrink_rows(pool: Pool, proj: int, X, seg_ws, work=None):
    """Per-row shrink; returns the work buffer (T = rows_t(pool, work, n))."""
    n = X.shape[0]
    _rows_check(pool, X, n)
    if work is None:
        work = new_work(pool, n, X.device)
    _check(lib().mlora_shrink_rows(pool.handle, proj, _ptr(X), _ptr(seg_ws), n, _ptr(work),
                                   work.numel() * work.element_size(), _stream()), "mlora_shrink_rows")
    return work


def gemm_lora(pool: Pool, proj: int, X, W0, seg_ws, work, Y=None):
    """Y = X W0^T + per-row s * Up t, t from shrink_rows in `work`."""
    torch = _torch()
    n = X.shape[0]
    _rows_check(pool, X, n)
    _bf16_dev(W0, "W0")
    if Y is None:
        Y = torch.empty((n, pool.dout), dtype=torch.bfloat16, device=X.device)
    _bf16_dev(Y, "Y")
    _check(lib().mlora_gemm_lora(pool.handle, proj, _ptr(X), _ptr(W0), _ptr(seg_ws), _ptr(work),
                                 work.numel() * work.element_size(), _ptr(Y), n, _stream()), "mlora_gemm_lora")
    return Y


def work_bytes(pool: Pool, n: int) -> int:
    return int(lib().mlora_work_bytes(pool.handle, n))


def plan(pool: Pool, n: int, variant: str = "auto"):
    """(variant name, shrink slices) that apply() runs for a batch of n rows."""
    v, c = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().mlora_plan(pool.handle, n, VARIANTS[variant], ctypes.byref(v), ctypes.byref(c)), "mlora_plan")
    return {0: "auto", 1: "split", 2: "fused", 3: "rows"}[v.value], c.value


def apply(pool: Pool, proj: int, X, W0, seg_ws, Y=None, work=None, variant: str = "auto"):
    """The whole layer for one projection: Y = X W0^T + each row's delta."""
    torch = _torch()
    n = X.shape[0]
    _rows_check(pool, X, n)
    _bf16_dev(W0, "W0")
    if tuple(W0.shape) != (pool.dout, pool.din):
        raise ValueError(f"W0 must be [{pool.dout}][{pool.din}]")
    if Y is None:
        Y = torch.empty((n, pool.dout), dtype=torch.bfloat16, device=X.device)
    _bf16_dev(Y, "Y")
    if work is None:
        work = new_work(pool, n, X.device)
    _check(lib().mlora_apply(pool.handle, proj, _ptr(X), _ptr(W0), _ptr(seg_ws), _ptr(Y), n, _ptr(work),
                             work.numel() * work.element_size(), VARIANTS[variant], _stream()), "mlora_apply")
    return Y


def forward(pool: Pool, proj: int, X, W0, row_adapter, seg_ws=None, Y=None, work=None, variant: str = "auto"):
    """Segment build and the layer for one projection in one call (the
    results of build_segments followed by apply).  Returns (Y, seg_ws); seg_ws
    serves apply on the batch's other projections."""
    torch = _torch()
    n = X.shape[0]
    _rows_check(pool, X, n)
    _bf16_dev(W0, "W0")
    if tuple(W0.shape) != (pool.dout, pool.din):
        raise ValueError(f"W0 must be [{pool.dout}][{pool.din}]")
    if row_adapter.dtype != torch.int32 or not row_adapter.is_cuda or not row_adapter.is_contiguous():
        raise TypeError("row_adapter must be a contiguous int32 CUDA tensor")
    if row_adapter.shape[0] != n:
        raise ValueError("row_adapter must have one id per row of X")
    nb = segments_bytes(n)
    if seg_ws is None:
        seg_ws = torch.empty(nb // 4, dtype=torch.int32, device=X.device)
    elif seg_ws.numel() * seg_ws.element_size() < nb:
        raise ValueError("seg_ws too small")
    if Y is None:
        Y = torch.empty((n, pool.dout), dtype=torch.bfloat16, device=X.device)
    _bf16_dev(Y, "Y")
    if work is None:
        work = new_work(pool, n, X.device)
    _check(lib().mlora_forward(pool.handle, proj, _ptr(X), _ptr(W0), _ptr(row_adapter), _ptr(seg_ws), _ptr(Y), n,
                               _ptr(work), work.numel() * work.element_size(), VARIANTS[variant], _stream()),
           "mlora_forward")
    return Y, seg_ws


def forward_static(pool: Pool, proj: int, X, W0, row_adapter, seg_ws=None, Y=None, variant: str = "auto"):
    """forward() with the library's static scratch in place of a work buffer
    (the call allocates no device memory).  Returns (Y, seg_ws)."""
    torch = _torch()
    n = X.shape[0]
    _rows_check(pool, X, n)
    _bf16_dev(W0, "W0")
    if tuple(W0.shape) != (pool.dout, pool.din):
        raise ValueError(f"W0 must be [{pool.dout}][{pool.din}]")
    if row_adapter.dtype != torch.int32 or not row_adapter.is_cuda or not row_adapter.is_contiguous():
        raise TypeError("row_adapter must be a contiguous int32 CUDA tensor")
    if row_adapter.shape[0] != n:
        raise ValueError("row_adapter must have one id per row of X")
    nb = segments_bytes(n)
    if seg_ws is None:
        seg_ws = torch.empty(nb // 4, dtype=torch.int32, device=X.device)
    elif seg_ws.numel() * seg_ws.element_size() < nb:
        raise ValueError("seg_ws too small")
    if Y is None:
        Y = torch.empty((n, pool.dout), dtype=torch.bfloat16, device=X.device)
    _bf16_dev(Y, "Y")
    _check(lib().mlora_forward_static(pool.handle, proj, _ptr(X), _ptr(W0), _ptr(row_adapter), _ptr(seg_ws), _ptr(Y),
                                      n, VARIANTS[variant], _stream()), "mlora_forward_static")
    return Y, seg_ws


STATIC_SCRATCH_BYTES = 20 << 20


def merge(pool: Pool, adapter_id: int, proj: int, W0, sign: float = 1.0):
    """W0 (device bf16 [dout][din], in place) += sign * s_a * Up_a Down_a."""
    torch = _torch()
    if W0.dtype != torch.bfloat16 or not W0.is_cuda or not W0.is_contiguous() or W0.dim() != 2:
        raise ValueError("W0 must be a contiguous CUDA bfloat16 matrix")
    if tuple(W0.shape) != (pool.dout, pool.din):
        raise ValueError(f"W0 must be [{pool.dout}][{pool.din}], got {tuple(W0.shape)}")
    _check(lib().mlora_merge(pool.handle, adapter_id, proj, _ptr(W0), ctypes.c_float(sign), _stream()),
           f"mlora_merge({adapter_id})")
    return W0


def hbm_copy(dst, src, nbytes: Optional[int] = None):
    nb = src.numel() * src.element_size() if nbytes is None else nbytes
    _check(lib().mlora_hbm_copy(_ptr(dst), _ptr(src), nb, _stream()), "mlora_hbm_copy")
    return dst


def hbm_read(src, out, nbytes: Optional[int] = None):
    """Streams src and XORs its 32-bit words into out[0] (device int32)."""
    nb = src.numel() * src.element_size() if nbytes is None else nbytes
    _check(lib().mlora_hbm_read(_ptr(src), nb, _ptr(out), _stream()), "mlora_hbm_read")
    return out


def hbm_read_lds(src, out, nbytes: Optional[int] = None):
    """Streams src through LDS DMA in 1 KiB pieces (mlora_hbm_read_lds)."""
    nb = src.numel() * src.element_size() if nbytes is None else nbytes
    _check(lib().mlora_hbm_read_lds(_ptr(src), nb, _ptr(out), _stream()), "mlora_hbm_read_lds")
    return out


_timing_armed = [0]


def timing_arm(n_launches: int):
    """Arms kernel start/end events on the library's next n_launches kernel
    launches (a measurement aid)."""
    _check(lib().mlora_timing_arm(n_launches), "mlora_timing_arm")
    _timing_armed[0] = n_launches


def timing_read() -> list:
    """Waits for the armed events: [(kernel name, milliseconds)] per marked
    launch, in launch order."""
    cap = max(_timing_armed[0], 1)
    ms = (ctypes.c_float * cap)()
    n = ctypes.c_int32(0)
    _check(lib().mlora_timing_read(ms, cap, ctypes.byref(n)), "mlora_timing_read")
    return [(lib().mlora_timing_name(i).decode(), float(ms[i])) for i in range(n.value)]
