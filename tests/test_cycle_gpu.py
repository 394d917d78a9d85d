"""GPU parity of the InvisibleLoRA cycle's two passes at one layer.

The *InvisibleLoRA* abstract drafts with the base model alone (a LoRA-off
pass, one token per request) and verifies every draft in one LoRA-on pass.
At the gate/up shape (4096 -> 14336, one rank-16 adapter per request, scale
2) and b = 16, 32, 64 and 128 requests, the draft pass (T = b, lora_on = 0)
and the verification pass (T = 2 b, lora_on = 1: each request's last
committed token and its draft, request-major) both run through the C ABI and
are compared with the fp64 oracle on every row.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
from gpu_util import BF16_TOL, compare, f32, i32, log, oracle_threads, to_dev, y_host
from mlora_inputs import make_custom_case

pytestmark = pytest.mark.gpu

B_MAX, D_IN, D_OUT, RANK = 128, 4096, 14336, 16


@functools.lru_cache(maxsize=1)
def _setup():
    import rank_adapter_gemm_segmented_amd as ml
    log(f"[cycle] building the gate/up case: {D_IN}->{D_OUT}, {B_MAX} rank-{RANK} adapters")
    # request q owns adapter q and rows 2q (last committed token), 2q + 1 (draft)
    case = make_custom_case(4000, "bf16", D_IN, D_OUT, np.repeat(np.arange(B_MAX), 2),
                            {a: RANK for a in range(B_MAX)}, scales={a: 2.0 for a in range(B_MAX)})
    pool = ml.Pool(D_IN, D_OUT, torch.bfloat16, RANK, B_MAX)
    for a in range(B_MAX):
        pool.register(a, to_dev(case.adapters[a].A, "bf16"), to_dev(case.adapters[a].B, "bf16"))
    opool = oracle.PackedPool(case.adapters, B_MAX, D_IN, D_OUT)
    return case, to_dev(case.x, "bf16"), to_dev(case.W, "bf16"), pool, opool, pool.workspace(2 * B_MAX)


@pytest.mark.parametrize("b", [16, 32, 64, 128])
def test_cycle_draft_and_verify_passes(b):
    import rank_adapter_gemm_segmented_amd as ml
    from rank_adapter_gemm_segmented_amd.cycle import cycle_passes, verify_segments
    case, x, W, pool, opool, ws = _setup()
    log(f"[cycle] b={b}: draft T={b} lora_on=0, verify T={2 * b} lora_on=1")
    ss = np.arange(b + 1, dtype=np.int32)
    sa = np.arange(b, dtype=np.int32)
    sr = np.full(b, RANK, np.int32)
    sc = np.full(b, 2.0, np.float32)
    x_draft = x[0:2 * b:2].contiguous()   # each request's last committed token
    x_verify = x[:2 * b].contiguous()     # that token and its draft
    y_d, y_v = cycle_passes(ml.linear, x_draft, x_verify, W, pool, i32(ss), i32(sa), i32(sr), f32(sc),
                            workspace=ws)
    torch.cuda.synchronize()
    xd_h = case.x[0:2 * b:2]
    ref_d = oracle.linear(xd_h, case.W, opool, ss, sa, sr, sc, None, 0, threads=oracle_threads())
    ref_v = oracle.linear(case.x[:2 * b], case.W, opool, verify_segments(ss), sa, sr, sc, None, 1,
                          threads=oracle_threads())
    compare(y_host(y_d), ref_d, BF16_TOL, f"cycle b={b} draft pass")
    compare(y_host(y_v), ref_v, BF16_TOL, f"cycle b={b} verify pass")
