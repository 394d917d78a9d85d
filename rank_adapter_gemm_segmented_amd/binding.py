"""Thin ctypes binding of ``libmlora.so`` (the C ABI in ``include/mlora.h``).

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the HIP stream, status codes become exceptions. Every step of
the layer runs in the library's HIP kernels; there is no Python or CPU
fallback, and importing this module fails loudly when the library is not
built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmlora.so")

MLORA_F32, MLORA_BF16 = 0, 1
STATUS = {
    0: "MLORA_OK", 1: "MLORA_ERR_INVALID_ARG", 2: "MLORA_ERR_SHAPE", 3: "MLORA_ERR_DTYPE",
    4: "MLORA_ERR_RANK", 5: "MLORA_ERR_ADAPTER", 6: "MLORA_ERR_EXISTS",
    7: "MLORA_ERR_WORKSPACE", 8: "MLORA_ERR_METADATA", 9: "MLORA_ERR_HIP",
}
STATUS_CODE = {v: k for k, v in STATUS.items()}


class MloraError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        self.name = STATUS.get(code, f"status {code}")
        super().__init__(f"{what}: {self.name} ({_lib.mlora_status_string(code).decode()})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built: run `python rank_adapter_gemm_segmented_amd/build.py` "
            "(or __graft_entry__.build()) first. There is no fallback path.")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    sig = {
        "mlora_status_string": ([I], ctypes.c_char_p),
        "mlora_pool_bytes": ([I, I, I, I, I], SZ),
        "mlora_pool_create": ([P, SZ, I, I, I, I, I, P, ctypes.POINTER(P)], I),
        "mlora_pool_destroy": ([P], I),
        "mlora_register_adapter": ([P, I, I, P, P, P], I),
        "mlora_unregister_adapter": ([P, I, P], I),
        "mlora_adapter_rank": ([P, I], I),
        "mlora_workspace_bytes": ([P, I], SZ),
        "mlora_workspace_init": ([P, SZ, P], I),
        "mlora_linear": ([P, P, P, P, P, P, P, P, I, I, I, P, P, SZ, P], I),
        "mlora_build_segments": ([P, P, I, P, P, P, P, P, P, P, P], I),
        "mlora_linear_tokens": ([P, P, P, P, P, I, I, P, P, SZ, P], I),
        "mlora_token_map": ([P, P, I, I, P, P, P], I),
        "mlora_validate": ([P, P, P, P, P, I, I, P, SZ, P], I),
        "mlora_merge_adapter": ([P, P, P, I, ctypes.c_float, P], I),
        "mlora_register_adapter_fused": ([P, I, I, P, P, P, P, P], I),
        "mlora_linear_fp8w": ([P, P, P, P, P, P, P, P, P, I, I, I, P, P, SZ, P], I),
        "mlora_linear_noalloc": ([P, P, P, P, P, P, P, P, I, I, I, P, P], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()


def library() -> ctypes.CDLL:
    return _lib


def _check(code: int, what: str):
    if code != 0:
        raise MloraError(code, what)


def _ptr(t: Optional[torch.Tensor]):
    # plain ints (ctypes passes them as void*): no wrapper object per argument
    return None if t is None else t.data_ptr()


_raw_stream = torch._C._cuda_getCurrentRawStream


def _stream():
    """The current torch stream of the current device as a raw HIP stream
    handle (also the capture stream inside torch.cuda.graph)."""
    return _raw_stream(torch.cuda.current_device())


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return MLORA_BF16
    if dt == torch.float32:
        return MLORA_F32
    raise TypeError(f"unsupported dtype {dt}")


def _i32(t, name):
    if t is None:
        return None
    if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous int32 device tensor")
    return t


class Pool:
    """Fixed-slot device adapter pool (``mlora_pool_create``). The arena is a
    torch uint8 tensor, so torch's allocator owns every device byte."""

    def __init__(self, d_in: int, d_out: int, dtype: torch.dtype, max_rank: int, capacity: int,
                 device="cuda"):
        self.d_in, self.d_out, self.dtype = d_in, d_out, dtype
        self.max_rank, self.capacity = max_rank, capacity
        code = _dtype_code(dtype)
        nbytes = _lib.mlora_pool_bytes(d_in, d_out, code, max_rank, capacity)
        if nbytes == 0:
            raise MloraError(STATUS_CODE["MLORA_ERR_SHAPE"], "mlora_pool_bytes")
        self.arena = torch.empty(nbytes, dtype=torch.uint8, device=device)
        h = ctypes.c_void_p()
        _check(_lib.mlora_pool_create(_ptr(self.arena), nbytes, d_in, d_out, code, max_rank,
                                      capacity, _stream(), ctypes.byref(h)), "mlora_pool_create")
        self.handle = h

    def register(self, adapter_id: int, A: torch.Tensor, B: torch.Tensor):
        """Copy A [rank, d_in] and B [d_out, rank] into slot ``adapter_id``."""
        rank = int(A.shape[0])
        if A.dtype != self.dtype or B.dtype != self.dtype:
            raise TypeError("adapter dtype differs from the pool dtype")
        if tuple(A.shape) != (rank, self.d_in) or tuple(B.shape) != (self.d_out, rank):
            raise ValueError("adapter shapes must be A [rank, d_in], B [d_out, rank]")
        A = A.contiguous()
        B = B.contiguous()
        _check(_lib.mlora_register_adapter(self.handle, adapter_id, rank, _ptr(A), _ptr(B),
                                           _stream()), "mlora_register_adapter")
        # the copy is stream-ordered: keep the sources alive until it has run
        torch.cuda.current_stream().synchronize()

    def register_fused(self, adapter_id: int, slices):
        """``mlora_register_adapter_fused``: one adapter over stacked projections.
        ``slices`` is a list of (A_m [r_m, d_in], B_m [rows_m, r_m]) in the
        order the projections are stacked in W. A pool holds either plain or
        fused adapters, and all fused ones stack W the same way; segments
        name the adapter with the stacked rank sum(r_m)."""
        n = len(slices)
        rows = (ctypes.c_int * n)(*[int(B.shape[0]) for _, B in slices])
        ranks = (ctypes.c_int * n)(*[int(A.shape[0]) for A, _ in slices])
        keep = []
        for A, B in slices:
            if A.dtype != self.dtype or B.dtype != self.dtype:
                raise TypeError("adapter dtype differs from the pool dtype")
            if A.dim() != 2 or A.shape[1] != self.d_in or B.dim() != 2 or B.shape[1] != A.shape[0]:
                raise ValueError("slice shapes must be A [r, d_in], B [rows, r]")
            keep.append((A.contiguous(), B.contiguous()))
        pa = (ctypes.c_void_p * n)(*[A.data_ptr() for A, _ in keep])
        pb = (ctypes.c_void_p * n)(*[B.data_ptr() for _, B in keep])
        _check(_lib.mlora_register_adapter_fused(self.handle, adapter_id, n, rows, ranks, pa, pb,
                                                 _stream()), "mlora_register_adapter_fused")
        torch.cuda.current_stream().synchronize()

    def unregister(self, adapter_id: int):
        _check(_lib.mlora_unregister_adapter(self.handle, adapter_id, _stream()),
               "mlora_unregister_adapter")

    def rank(self, adapter_id: int) -> int:
        return int(_lib.mlora_adapter_rank(self.handle, adapter_id))

    def workspace_bytes(self, max_tokens: int) -> int:
        return int(_lib.mlora_workspace_bytes(self.handle, max_tokens))

    def workspace(self, max_tokens: int) -> torch.Tensor:
        n = self.workspace_bytes(max_tokens)
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=self.arena.device)
        _check(_lib.mlora_workspace_init(_ptr(ws), ws.numel(), _stream()), "mlora_workspace_init")
        return ws

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            _lib.mlora_pool_destroy(h)
            self.handle = None


def _check_xw(x, W, pool: Pool):
    if x.dtype != pool.dtype or W.dtype != pool.dtype:
        raise TypeError("x and W must have the pool's dtype")
    if x.dim() != 2 or x.shape[1] != pool.d_in or tuple(W.shape) != (pool.d_out, pool.d_in):
        raise ValueError("x must be [T, d_in] and W [d_out, d_in]")
    if not (x.is_contiguous() and W.is_contiguous()):
        raise ValueError("x and W must be contiguous")


def linear(x, W, pool: Pool, seg_start=None, seg_adapter=None, seg_rank=None, seg_scale=None,
           lora_on: int = 1, token_index=None, out=None, workspace=None):
    """``mlora_linear``: y = W x + per-segment adapter term (sorted metadata)."""
    _check_xw(x, W, pool)
    T = int(x.shape[0])
    y = out if out is not None else torch.empty((T, pool.d_out), dtype=pool.dtype, device=x.device)
    ws = workspace if workspace is not None else pool.workspace(T)
    n_seg = int(seg_adapter.numel()) if seg_adapter is not None else 0
    if seg_scale is not None and (seg_scale.dtype != torch.float32 or not seg_scale.is_contiguous()):
        raise TypeError("seg_scale must be contiguous float32")
    _check(_lib.mlora_linear(_ptr(x), _ptr(W), pool.handle, _ptr(_i32(seg_start, "seg_start")),
                             _ptr(_i32(seg_adapter, "seg_adapter")), _ptr(_i32(seg_rank, "seg_rank")),
                             _ptr(seg_scale), _ptr(_i32(token_index, "token_index")), T, n_seg,
                             int(lora_on), _ptr(y), _ptr(ws), ws.numel(), _stream()),
           "mlora_linear")
    return y


def linear_noalloc(x, W, pool: Pool, seg_start=None, seg_adapter=None, seg_rank=None, seg_scale=None,
                   lora_on: int = 1, token_index=None, out=None):
    """``mlora_linear_noalloc``: ``linear`` with the library's own device
    scratch as the workspace (the call allocates nothing; ``out`` should be
    given by callers that cannot allocate either)."""
    _check_xw(x, W, pool)
    T = int(x.shape[0])
    y = out if out is not None else torch.empty((T, pool.d_out), dtype=pool.dtype, device=x.device)
    n_seg = int(seg_adapter.numel()) if seg_adapter is not None else 0
    if seg_scale is not None and (seg_scale.dtype != torch.float32 or not seg_scale.is_contiguous()):
        raise TypeError("seg_scale must be contiguous float32")
    _check(_lib.mlora_linear_noalloc(_ptr(x), _ptr(W), pool.handle, _ptr(_i32(seg_start, "seg_start")),
                                     _ptr(_i32(seg_adapter, "seg_adapter")), _ptr(_i32(seg_rank, "seg_rank")),
                                     _ptr(seg_scale), _ptr(_i32(token_index, "token_index")), T, n_seg,
                                     int(lora_on), _ptr(y), _stream()), "mlora_linear_noalloc")
    return y


def linear_fp8w(x, W_fp8, w_scale, pool: Pool, seg_start=None, seg_adapter=None, seg_rank=None,
                seg_scale=None, lora_on: int = 1, token_index=None, out=None, workspace=None):
    """``mlora_linear_fp8w``: the layer with an FP8 (e4m3 codes, uint8 [d_out, d_in])
    base weight and float32 per-row scales; x, y and the pool in bf16."""
    if x.dtype != torch.bfloat16 or pool.dtype != torch.bfloat16:
        raise TypeError("x and the pool must be bf16")
    if W_fp8.dtype != torch.uint8 or tuple(W_fp8.shape) != (pool.d_out, pool.d_in) or not W_fp8.is_contiguous():
        raise ValueError("W_fp8 must be contiguous uint8 [d_out, d_in]")
    if w_scale.dtype != torch.float32 or w_scale.numel() != pool.d_out or not w_scale.is_contiguous():
        raise ValueError("w_scale must be contiguous float32 [d_out]")
    if x.dim() != 2 or x.shape[1] != pool.d_in or not x.is_contiguous():
        raise ValueError("x must be contiguous [T, d_in]")
    T = int(x.shape[0])
    y = out if out is not None else torch.empty((T, pool.d_out), dtype=pool.dtype, device=x.device)
    ws = workspace if workspace is not None else pool.workspace(T)
    n_seg = int(seg_adapter.numel()) if seg_adapter is not None else 0
    _check(_lib.mlora_linear_fp8w(_ptr(x), _ptr(W_fp8), _ptr(w_scale), pool.handle,
                                  _ptr(_i32(seg_start, "seg_start")), _ptr(_i32(seg_adapter, "seg_adapter")),
                                  _ptr(_i32(seg_rank, "seg_rank")), _ptr(seg_scale),
                                  _ptr(_i32(token_index, "token_index")), T, n_seg, int(lora_on), _ptr(y),
                                  _ptr(ws), ws.numel(), _stream()), "mlora_linear_fp8w")
    return y


def linear_tokens(x, W, pool: Pool, token_adapter, adapter_scale, lora_on: int = 1, out=None,
                  workspace=None):
    """``mlora_linear_tokens``: the layer on an unsorted batch (library segments it)."""
    _check_xw(x, W, pool)
    T = int(x.shape[0])
    y = out if out is not None else torch.empty((T, pool.d_out), dtype=pool.dtype, device=x.device)
    ws = workspace if workspace is not None else pool.workspace(T)
    _check(_lib.mlora_linear_tokens(_ptr(x), _ptr(W), pool.handle,
                                    _ptr(_i32(token_adapter, "token_adapter")), _ptr(adapter_scale),
                                    T, int(lora_on), _ptr(y), _ptr(ws), ws.numel(), _stream()),
           "mlora_linear_tokens")
    return y


def build_segments(token_adapter, adapter_scale, pool: Pool):
    """``mlora_build_segments``: canonical segments of an unsorted batch.
    Returns (token_index, seg_start, seg_adapter, seg_rank, seg_scale, n_seg) as
    device tensors sized for the worst case; n_seg is a 1-element tensor."""
    T = int(token_adapter.numel())
    dev = token_adapter.device
    ti = torch.empty(max(T, 1), dtype=torch.int32, device=dev)
    ss = torch.empty(T + 2, dtype=torch.int32, device=dev)
    sa = torch.empty(T + 1, dtype=torch.int32, device=dev)
    sr = torch.empty(T + 1, dtype=torch.int32, device=dev)
    sc = torch.empty(T + 1, dtype=torch.float32, device=dev)
    ns = torch.empty(1, dtype=torch.int32, device=dev)
    _check(_lib.mlora_build_segments(_ptr(_i32(token_adapter, "token_adapter")), _ptr(adapter_scale),
                                     T, pool.handle, _ptr(ti), _ptr(ss), _ptr(sa), _ptr(sr),
                                     _ptr(sc), _ptr(ns), _stream()), "mlora_build_segments")
    return ti[:T], ss, sa, sr, sc, ns


def token_map(seg_start, seg_adapter, n_tokens: int):
    """``mlora_token_map``: per sorted position, its segment and adapter id."""
    dev = seg_start.device
    ts = torch.empty(max(n_tokens, 1), dtype=torch.int32, device=dev)
    ta = torch.empty(max(n_tokens, 1), dtype=torch.int32, device=dev)
    n_seg = int(seg_adapter.numel())
    _check(_lib.mlora_token_map(_ptr(_i32(seg_start, "seg_start")), _ptr(_i32(seg_adapter, "seg_adapter")),
                                n_tokens, n_seg, _ptr(ts), _ptr(ta), _stream()), "mlora_token_map")
    return ts[:n_tokens], ta[:n_tokens]


def validate(pool: Pool, seg_start, seg_adapter, seg_rank=None, token_index=None, n_tokens=None,
             workspace=None) -> int:
    """``mlora_validate``: returns the status code (0 = valid); synchronizes."""
    T = int(n_tokens) if n_tokens is not None else int(seg_start[-1].item())
    ws = workspace if workspace is not None else pool.workspace(T)
    return int(_lib.mlora_validate(pool.handle, _ptr(_i32(seg_start, "seg_start")),
                                   _ptr(_i32(seg_adapter, "seg_adapter")),
                                   _ptr(_i32(seg_rank, "seg_rank")),
                                   _ptr(_i32(token_index, "token_index")), T,
                                   int(seg_adapter.numel()), _ptr(ws), ws.numel(), _stream()))


def merge_adapter(W, pool: Pool, adapter_id: int, scale: float, out=None):
    """``mlora_merge_adapter``: W + scale * B_a A_a into ``out`` (a new tensor
    if None; pass ``out=W`` to merge in place). A negative scale unmerges."""
    if W.dtype != pool.dtype or tuple(W.shape) != (pool.d_out, pool.d_in) or not W.is_contiguous():
        raise ValueError("W must be a contiguous [d_out, d_in] tensor of the pool's dtype")
    o = out if out is not None else torch.empty_like(W)
    if o.dtype != W.dtype or o.shape != W.shape or not o.is_contiguous():
        raise ValueError("out must match W")
    _check(_lib.mlora_merge_adapter(_ptr(W), _ptr(o), pool.handle, int(adapter_id), float(scale),
                                    _stream()), "mlora_merge_adapter")
    return o
