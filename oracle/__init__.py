"""ctypes front end of the fp64 CPU oracle (``mlora_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module; the product library never
does. It shares no code with the GPU path; the only thing both sides see is the
seeded input generator in ``mlora_inputs``.

The C source computes the plain per-token definition of the multi-LoRA linear
layer in double precision (see the header comment of ``mlora_oracle.c``), and
the merged weight W + scale * B A of one adapter.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mlora_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmlora_oracle.so")
_lock = threading.Lock()
_lib = None

MLO_OK, MLO_ERR_ARG, MLO_ERR_META, MLO_ERR_ADAPTER, MLO_ERR_RANK = 0, -1, -2, -3, -4

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
          "-std=c99", "-Wall", "-Wextra"]


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"oracle {what} failed with code {code}")
        self.code = code


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc (fp64, no FMA contraction, OpenMP)."""
    cmd = ["gcc", *CFLAGS, src, "-o", out + ".tmp"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(out + ".tmp", out)
    return out


def _i32p(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _f32p(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _f64p(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _i64p(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def load(path: Optional[str] = None):
    """Load the compiled oracle, compiling it first only if it is missing."""
    global _lib
    with _lock:
        if path is None and _lib is not None:
            return _lib
        p = path or _LIB_PATH
        if not os.path.exists(p):
            build(out=p)
        lib = ctypes.CDLL(p)
        P = ctypes.c_void_p
        i32 = ctypes.c_int
        lib.mlo_segment.argtypes = [i32, P, i32, P, P, P]
        lib.mlo_segment.restype = i32
        lib.mlo_check_meta.argtypes = [i32, i32, P, P, P, P, i32, P]
        lib.mlo_check_meta.restype = i32
        lib.mlo_token_map.argtypes = [i32, i32, P, P, P, P]
        lib.mlo_token_map.restype = i32
        lib.mlo_linear.argtypes = [i32, i32, i32, P, P, i32, P, P, P, P, P, i32, P, P, P, P, P,
                                   i32, i32, P, P, P, i32]
        lib.mlo_linear.restype = i32
        lib.mlo_merge.argtypes = [i32, i32, i32, P, P, P, ctypes.c_double, P, i32]
        lib.mlo_merge.restype = i32
        if path is None:
            _lib = lib
        return lib


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------------------
# Python wrappers
# ---------------------------------------------------------------------------

def segment(token_adapter: Sequence[int], capacity: int, lib=None):
    """Canonical stable grouping of unsorted ids: returns
    (token_index[T], seg_start[S+1], seg_adapter[S])."""
    lib = lib or load()
    ids = _c(token_adapter, np.int32)
    T = int(ids.shape[0])
    ti = np.zeros(max(T, 1), np.int32)
    ss = np.zeros(T + 2, np.int32)
    sa = np.zeros(T + 1, np.int32)
    S = lib.mlo_segment(T, _i32p(ids), int(capacity), _i32p(ti), _i32p(ss), _i32p(sa))
    if S < 0:
        raise OracleError(S, "segment")
    return ti[:T].copy(), ss[:S + 1].copy(), sa[:S].copy()


def token_map(seg_start, seg_adapter, n_tokens: int, lib=None):
    """Per sorted position: (token_seg[T], token_adapter[T])."""
    lib = lib or load()
    ss = _c(seg_start, np.int32)
    sa = _c(seg_adapter, np.int32)
    S = int(sa.shape[0])
    ts = np.zeros(max(n_tokens, 1), np.int32)
    ta = np.zeros(max(n_tokens, 1), np.int32)
    rc = lib.mlo_token_map(int(n_tokens), S, _i32p(ss), _i32p(sa), _i32p(ts), _i32p(ta))
    if rc != MLO_OK:
        raise OracleError(rc, "token_map")
    return ts[:n_tokens].copy(), ta[:n_tokens].copy()


class PackedPool:
    """Adapters of a case packed into two flat float32 arrays plus offsets."""

    def __init__(self, adapters: dict, capacity: int, d_in: int, d_out: int):
        self.capacity = capacity
        self.rank = np.zeros(max(capacity, 1), np.int32)
        self.a_off = np.zeros(max(capacity, 1), np.int64)
        self.b_off = np.zeros(max(capacity, 1), np.int64)
        a_parts, b_parts = [], []
        ao = bo = 0
        for aid in sorted(adapters):
            ad = adapters[aid]
            self.rank[aid] = ad.rank
            self.a_off[aid] = ao
            self.b_off[aid] = bo
            a_parts.append(np.ascontiguousarray(ad.A, np.float32).reshape(-1))
            b_parts.append(np.ascontiguousarray(ad.B, np.float32).reshape(-1))
            ao += ad.rank * d_in
            bo += d_out * ad.rank
        self.A = np.concatenate(a_parts) if a_parts else np.zeros(1, np.float32)
        self.B = np.concatenate(b_parts) if b_parts else np.zeros(1, np.float32)


def linear(x, W, pool: PackedPool, seg_start, seg_adapter, seg_rank, seg_scale,
           token_index=None, lora_on: int = 1, rows=None, threads: int = 0,
           with_base: bool = False, lib=None):
    """fp64 y for the requested batch rows (all rows if ``rows`` is None)."""
    lib = lib or load()
    x = _c(x, np.float32)
    W = _c(W, np.float32)
    T, d_in = x.shape
    d_out = W.shape[0]
    assert W.shape[1] == d_in
    ss = _c(seg_start, np.int32) if seg_start is not None else np.zeros(1, np.int32)
    sa = _c(seg_adapter, np.int32) if seg_adapter is not None else np.zeros(0, np.int32)
    sr = _c(seg_rank, np.int32) if seg_rank is not None else None
    sc = _c(seg_scale, np.float32) if seg_scale is not None else np.zeros(max(sa.shape[0], 1), np.float32)
    ti = _c(token_index, np.int32)
    rws = _c(rows, np.int32)
    n_rows = T if rws is None else int(rws.shape[0])
    y = np.zeros((max(n_rows, 1), d_out), np.float64)
    yb = np.zeros((max(n_rows, 1), d_out), np.float64) if with_base else None
    rc = lib.mlo_linear(T, d_in, d_out, _f32p(x), _f32p(W), pool.capacity, _i32p(pool.rank),
                        _i64p(pool.a_off), _i64p(pool.b_off), _f32p(pool.A), _f32p(pool.B),
                        int(sa.shape[0]), _i32p(ss), _i32p(sa), _i32p(sr), _f32p(sc), _i32p(ti),
                        int(lora_on), n_rows, _i32p(rws), _f64p(y), _f64p(yb), int(threads))
    if rc != MLO_OK:
        raise OracleError(rc, "linear")
    if with_base:
        return y[:n_rows], yb[:n_rows]
    return y[:n_rows]


def case_metadata(case) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray, Optional[np.ndarray]]:
    """Segment metadata for a generated case. Unsorted cases are segmented
    here by the oracle's own canonical grouping."""
    if case.sorted_input:
        return case.seg_start, case.seg_adapter, case.seg_rank, case.seg_scale, case.token_index
    ti, ss, sa = segment(case.token_adapter, case.capacity)
    sr = np.array([case.adapters[a].rank if a >= 0 else 0 for a in sa], np.int32)
    sc = np.array([case.adapter_scale[a] if a >= 0 else 0.0 for a in sa], np.float32)
    return ss, sa, sr, sc, ti


def case_linear(case, lora_on: int = 1, rows=None, threads: int = 0, with_base: bool = False,
                pool: Optional[PackedPool] = None):
    """Oracle output for a ``mlora_inputs.Case``."""
    pool = pool or PackedPool(case.adapters, case.capacity, case.d_in, case.d_out)
    ss, sa, sr, sc, ti = case_metadata(case)
    return linear(case.x, case.W, pool, ss, sa, sr, sc, ti, lora_on, rows, threads, with_base)


def merge(W, A, B, scale: float, threads: int = 0, lib=None) -> np.ndarray:
    """fp64 merged weight W + scale * B A of one adapter (A [r, d_in],
    B [d_out, r]); a negative scale unmerges. ``scale`` is taken as the
    float32 value the library receives."""
    lib = lib or load()
    W = _c(W, np.float32)
    d_out, d_in = W.shape
    A = _c(A, np.float32).reshape(-1, d_in)
    r = int(A.shape[0])
    B = _c(B, np.float32).reshape(d_out, r)
    out = np.zeros((d_out, d_in), np.float64)
    rc = lib.mlo_merge(d_in, d_out, r, _f32p(W), _f32p(A), _f32p(B),
                       float(np.float32(scale)), _f64p(out), int(threads))
    if rc != MLO_OK:
        raise OracleError(rc, "merge")
    return out


def fused_case_linear(slice_cases, lora_on: int = 1, rows=None, threads: int = 0):
    """Oracle output of several projections stacked into one weight: each
    slice is the plain layer over its own W_m and adapters (A_m, B_m) with the
    batch's shared segments and scales, and the slices' outputs sit side by
    side in the order given."""
    return np.concatenate([case_linear(c, lora_on, rows=rows, threads=threads) for c in slice_cases],
                          axis=1)


def e4m3_decode(codes) -> np.ndarray:
    """Values of FP8 e4m3 codes (OCP 8-bit floating point, E4M3: sign bit,
    4 exponent bits with bias 7, 3 mantissa bits, no infinities; exponent 0 is
    subnormal, m/8 * 2^-6; code S.1111.111 is NaN), as float32 (exact)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return (sign * mag).astype(np.float32)


def fp8w_case_linear(case, codes, w_scale, lora_on: int = 1, rows=None, threads: int = 0):
    """Oracle output of the layer whose base weight is stored as FP8: the
    dequantized weight W[n, k] = w_scale[n] * e4m3(codes[n, k]), i.e.
        y_i = diag(w_scale) (Q x_i) + scale_s B_a (A_a x_i)
    with Q the decoded codes (the row scale taken out of the sum over k)."""
    import dataclasses
    Q = e4m3_decode(codes)
    qcase = dataclasses.replace(case, W=Q)
    base = case_linear(qcase, 0, rows=rows, threads=threads)
    y = base * np.asarray(w_scale, np.float64)[None, :]
    if lora_on:
        zcase = dataclasses.replace(case, W=np.zeros_like(Q))
        y = y + case_linear(zcase, 1, rows=rows, threads=threads)
    return y
