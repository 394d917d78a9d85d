"""Host-only checks of the C-ABI library (no GPU needed, no kernel launched).

* libmlora.so loads and exports every function include/mlora.h declares.
* Pure host entry points: status strings, pool geometry, argument checks that
  return before any HIP call.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mlora.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mlora_[a-z_]+)\s*\(", src)))


def test_header_declares_the_layer_calls():
    names = _declared()
    for required in ("mlora_linear", "mlora_register_adapter", "mlora_pool_create",
                     "mlora_build_segments", "mlora_linear_tokens", "mlora_token_map",
                     "mlora_validate", "mlora_workspace_bytes"):
        assert required in names


def test_library_exports_every_declared_symbol():
    import rank_adapter_gemm_segmented_amd as ml
    lib = ctypes.CDLL(ml.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings():
    import rank_adapter_gemm_segmented_amd as ml
    lib = ml.library()
    for code, name in ml.STATUS.items():
        s = lib.mlora_status_string(code).decode()
        assert s and s != "unknown status", name
    assert lib.mlora_status_string(12345).decode() == "unknown status"


def _geometry(d_in, d_out, elem, max_rank, capacity):
    # slot: A [max_rank, d_in], then B: bf16 pools in blocks of 16 rank
    # columns (d_out x max_rank rounded up to 16), fp32 pools in rows of the
    # rank rounded up to 8
    a = max_rank * d_in
    b_off = (a + 127) // 128 * 128
    b = d_out * ((max_rank + 15) // 16 * 16 if elem == 2 else (max_rank + 7) // 8 * 8)
    slot = (b_off + b + 127) // 128 * 128
    slots = (capacity * slot * elem + 255) // 256 * 256
    return slots + (capacity * 4 + 255) // 256 * 256 + 4096


@pytest.mark.parametrize("shape", [(4096, 4096, 1, 16, 32), (5120, 5120, 1, 64, 512),
                                   (256, 256, 0, 8, 4), (4104, 1000, 1, 7, 3), (8, 1, 1, 1, 1)])
def test_pool_bytes_geometry(shape):
    import rank_adapter_gemm_segmented_amd as ml
    d_in, d_out, dt, r, cap = shape
    got = ml.library().mlora_pool_bytes(d_in, d_out, dt, r, cap)
    assert got == _geometry(d_in, d_out, 4 if dt == 0 else 2, r, cap)


@pytest.mark.parametrize("shape", [(4100, 64, 1, 8, 4),     # d_in not a multiple of 8 (bf16)
                                   (0, 64, 1, 8, 4), (64, 0, 1, 8, 4), (64, 64, 7, 8, 4),
                                   (64, 64, 1, 0, 4), (64, 64, 1, 257, 4), (64, 64, 1, 8, 0)])
def test_pool_bytes_rejects_bad_shapes(shape):
    import rank_adapter_gemm_segmented_amd as ml
    assert ml.library().mlora_pool_bytes(*shape) == 0


def test_host_argument_checks_return_before_any_device_call():
    import rank_adapter_gemm_segmented_amd as ml
    lib = ml.library()
    E = ml.STATUS_CODE
    out = ctypes.c_void_p()
    assert lib.mlora_pool_create(None, 0, 64, 64, 1, 8, 4, None, ctypes.byref(out)) == E["MLORA_ERR_INVALID_ARG"]
    fake = ctypes.c_void_p(256)  # aligned, never dereferenced: the shape check fails first
    assert lib.mlora_pool_create(fake, 1 << 20, 64, 64, 9, 8, 4, None, ctypes.byref(out)) == E["MLORA_ERR_DTYPE"]
    assert lib.mlora_pool_create(fake, 1 << 20, 63, 64, 1, 8, 4, None, ctypes.byref(out)) == E["MLORA_ERR_SHAPE"]
    assert lib.mlora_pool_create(fake, 16, 64, 64, 1, 8, 4, None, ctypes.byref(out)) == E["MLORA_ERR_WORKSPACE"]
    assert lib.mlora_linear(None, None, None, None, None, None, None, None, 4, 1, 1, None, None, 0,
                            None) == E["MLORA_ERR_INVALID_ARG"]
    assert lib.mlora_adapter_rank(None, 0) == -1
    assert lib.mlora_workspace_bytes(None, 16) == 0
    assert lib.mlora_pool_destroy(None) == 0
    assert lib.mlora_token_map(None, None, 0, 0, None, None, None) == 0      # zero tokens: no-op
    assert lib.mlora_token_map(None, None, 4, 1, None, None, None) == E["MLORA_ERR_INVALID_ARG"]


def test_bench_refuses_more_than_one_gpu():
    # the layer is built and measured on one GPU: bench.py says so and exits
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
