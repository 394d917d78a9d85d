"""GPU parity of the adapter merge (``mlora_merge_adapter``) against the fp64 oracle.

W_out = W_in + scale * B_a A_a: the merged weight W = W0 + dW of the "LoRA
Inference" glossary (first paragraph), dW the scaled low-rank term of the
"Multi-LoRA Serving in Practice" LoRA forward. A negative scale unmerges.

Tolerance, derived from the arithmetic: the bf16 kernel forms dW on MFMA
(exact bf16 products, fp32 sums), scales and adds W in fp32, and rounds once to
bf16 by round-to-nearest-even. RNE to bf16 errs by at most 2^-8 |v|; the fp32
steps add at most (r + 3) 2^-24 M with M = |W| + |c| (|B| @ |A|). So
    |W_gpu - W_ref| <= 2^-8 |W_ref| + (r + 4) 2^-24 M      (bf16)
    |W_gpu - W_ref| <= (r + 4) 2^-24 M                       (fp32)
and, since the fp32 error is far below a bf16 ulp, W_gpu equals the
correctly rounded W_ref except where W_ref sits next to a rounding midpoint
(expected about 1e-5 of the elements; the test allows 1e-3).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import compare, f32, i32, log, oracle_threads, to_dev, y_host
from mlora_inputs import bf16_round, make_custom_case, make_merge_inputs

pytestmark = pytest.mark.gpu


def _ml():
    import rank_adapter_gemm_segmented_amd as ml
    return ml


def _pool_with(dtype, d_in, d_out, W, ad, aid=2, max_rank=None):
    """A pool of capacity 3 holding the adapter at slot ``aid`` and a decoy of
    another rank at slot 0 (a wrong slot offset shows up as wrong values)."""
    ml = _ml()
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    mr = max_rank or max(ad.rank, 9)
    pool = ml.Pool(d_in, d_out, tdt, mr, 3)
    _, decoy = make_merge_inputs(999, dtype, d_in, d_out, 9 if ad.rank != 9 else 7)
    pool.register(0, to_dev(decoy.A, dtype), to_dev(decoy.B, dtype))
    pool.register(aid, to_dev(ad.A, dtype), to_dev(ad.B, dtype))
    return pool, to_dev(W, dtype)


def _check_merge(W_gpu, W, ad, scale, dtype, what):
    ref = oracle.merge(W, ad.A, ad.B, scale, threads=oracle_threads())
    c = float(np.float32(scale))
    M = np.abs(W.astype(np.float64)) + abs(c) * (np.abs(ad.B.astype(np.float64)) @ np.abs(ad.A.astype(np.float64)))
    fp = (ad.rank + 4) * 2.0 ** -24 * M
    bound = (2.0 ** -8 * np.abs(ref) + fp) if dtype == "bf16" else fp
    assert np.all(np.isfinite(W_gpu)), what
    err = np.abs(W_gpu - ref)
    worst = float(np.max(err / bound))
    assert worst <= 1.0, f"{what}: max err/bound {worst:.3f}"
    if dtype == "bf16":
        rounded = bf16_round(ref.astype(np.float32)).astype(np.float64)
        frac = float(np.mean(W_gpu != rounded))
        assert frac <= 1e-3, f"{what}: {frac:.2e} of the elements differ from the rounded oracle"
        log(f"  {what}: err/bound {worst:.3f}, {frac:.1e} off the rounded oracle")
    else:
        log(f"  {what}: err/bound {worst:.3f}")


CASES = [
    # dtype, d_in, d_out, rank, scale, in_place
    ("bf16", 4096, 4096, 16, 2.0, False),      # decode q projection at its real size
    ("bf16", 4096, 1024, 64, 2.0, True),       # prefill k projection, rank 64, in place
    ("bf16", 14336, 4096, 64, -2.0, True),     # prefill down projection (unmerge sign)
    ("bf16", 328, 200, 24, -0.75, False),      # ragged tiles both ways, rank not a multiple of 16
    ("bf16", 136, 70, 72, 1.5, True),          # two rank chunks
    ("bf16", 264, 33, 256, 0.5, False),        # the largest rank, four chunks
    ("bf16", 8, 1, 1, 3.0, False),             # smallest shape
    ("bf16", 1 << 17, 8, 16, 2.0, True),       # the largest d_in (MLORA_MAX_DIM)
    ("bf16", 64, 1 << 17, 64, -1.0, False),    # the largest d_out
    ("f32", 256, 256, 8, 2.0, False),          # the fp32 tiny shape
    ("f32", 100, 37, 5, -1.0, True),           # ragged fp32
]


@pytest.mark.parametrize("dtype,d_in,d_out,rank,scale,in_place", CASES)
def test_merge_parity(dtype, d_in, d_out, rank, scale, in_place):
    what = f"merge {dtype} {d_out}x{d_in} r{rank} c={scale} {'in place' if in_place else 'out of place'}"
    log(f"[merge] {what}")
    W, ad = make_merge_inputs(500 + rank + d_in % 97, dtype, d_in, d_out, rank)
    pool, Wd = _pool_with(dtype, d_in, d_out, W, ad)
    keep = Wd.clone()
    out = _ml().merge_adapter(Wd, pool, 2, scale, out=Wd if in_place else None)
    torch.cuda.synchronize()
    if not in_place:
        assert torch.equal(Wd, keep), "out-of-place merge wrote its input"
    _check_merge(y_host(out), W, ad, scale, dtype, what)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_merge_zero_scale_is_identity(dtype):
    log(f"[merge] scale 0 ({dtype})")
    W, ad = make_merge_inputs(71, dtype, 520, 130, 16)
    pool, Wd = _pool_with(dtype, 520, 130, W, ad)
    out = _ml().merge_adapter(Wd, pool, 2, 0.0)
    torch.cuda.synchronize()
    assert np.array_equal(y_host(out), W.astype(np.float64))


def test_merge_unmerge_roundtrip():
    # bf16: each call rounds once, so unmerging returns W within two roundings
    log("[merge] merge then unmerge")
    W, ad = make_merge_inputs(72, "bf16", 1024, 512, 32)
    pool, Wd = _pool_with("bf16", 1024, 512, W, ad)
    ml = _ml()
    ml.merge_adapter(Wd, pool, 2, 2.0, out=Wd)
    ml.merge_adapter(Wd, pool, 2, -2.0, out=Wd)
    torch.cuda.synchronize()
    back = y_host(Wd)
    dW = 2.0 * np.abs(ad.B.astype(np.float64) @ ad.A.astype(np.float64))
    bound = 2.0 ** -7 * (np.abs(W) + dW) + 1e-12
    assert np.all(np.abs(back - W) <= bound)


def test_merged_weight_serves_like_the_adapter():
    # the glossary's merged model: a LoRA-off pass over W + c B A gives the
    # oracle's LoRA-on output for a batch whose tokens all use that adapter
    log("[merge] LoRA-off over merged W vs oracle LoRA-on")
    T, d_in, d_out, r, c = 64, 4096, 4096, 16, 2.0
    case = make_custom_case(73, "bf16", d_in, d_out, [3] * T, {a: r for a in range(4)},
                            scales={a: c for a in range(4)})
    ml = _ml()
    pool = ml.Pool(d_in, d_out, torch.bfloat16, r, case.capacity)
    for aid, ad in sorted(case.adapters.items()):
        pool.register(aid, to_dev(ad.A, "bf16"), to_dev(ad.B, "bf16"))
    Wm = ml.merge_adapter(to_dev(case.W, "bf16"), pool, 3, c)
    y = ml.linear(to_dev(case.x, "bf16"), Wm, pool, lora_on=0, workspace=pool.workspace(T))
    torch.cuda.synchronize()
    y_ref = oracle.case_linear(case, 1, threads=oracle_threads())
    compare(y_host(y), y_ref, 2e-2, "merged LoRA-off vs oracle LoRA-on")


def test_merge_errors():
    log("[merge] error paths")
    ml = _ml()
    E = ml.STATUS_CODE
    W, ad = make_merge_inputs(74, "bf16", 64, 48, 8)
    pool, Wd = _pool_with("bf16", 64, 48, W, ad)
    for aid, code in [(1, "MLORA_ERR_ADAPTER"), (3, "MLORA_ERR_ADAPTER"), (-1, "MLORA_ERR_ADAPTER")]:
        with pytest.raises(ml.MloraError) as e:
            ml.merge_adapter(Wd, pool, aid, 1.0)
        assert e.value.code == E[code], aid
    lib = ml.library()
    import ctypes
    base = Wd.data_ptr()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # partial overlap of W_in and W_out, and a misaligned pointer
    big = torch.empty(2 * 64 * 48, dtype=torch.bfloat16, device="cuda")
    assert lib.mlora_merge_adapter(ctypes.c_void_p(big.data_ptr()), ctypes.c_void_p(big.data_ptr() + 256),
                                   pool.handle, 2, ctypes.c_float(1.0), st) == E["MLORA_ERR_INVALID_ARG"]
    assert lib.mlora_merge_adapter(ctypes.c_void_p(base + 2), ctypes.c_void_p(big.data_ptr()),
                                   pool.handle, 2, ctypes.c_float(1.0), st) == E["MLORA_ERR_INVALID_ARG"]
    assert lib.mlora_merge_adapter(None, ctypes.c_void_p(base), pool.handle, 2, ctypes.c_float(1.0),
                                   st) == E["MLORA_ERR_INVALID_ARG"]
    torch.cuda.synchronize()
    assert torch.equal(Wd, to_dev(W, "bf16")), "a rejected call wrote W"
