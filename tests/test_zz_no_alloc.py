"""The entry point that allocates nothing (mlora_linear_noalloc) against
mlora_linear, through the C ABI.

mlora_linear_noalloc runs the same kernels with the library's own device
scratch as the workspace, so its output must equal mlora_linear's bit for
bit (stronger than the oracle tolerance both meet). Two calls in a row on the
shared scratch, the second with a smaller input, on the tiled-GEMM path and
on the split-K decode path; both are also checked against the fp64 oracle.
A call whose workspace exceeds the scratch is refused before anything runs.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import BF16_TOL, DeviceCase, compare, f32, i32, log, oracle_threads, y_host
from mlora_inputs import make_custom_case

pytestmark = pytest.mark.gpu


def _run_both(dc, lora_on):
    import rank_adapter_gemm_segmented_amd as ml
    c = dc.case
    meta = (dc.seg_start, dc.seg_adapter, dc.seg_rank, dc.seg_scale)
    y_ref = ml.linear(dc.x, dc.W, dc.pool, *meta, lora_on=lora_on, token_index=dc.token_index,
                      workspace=dc.ws)
    y_na = torch.full_like(y_ref, 3.0)
    ml.linear_noalloc(dc.x, dc.W, dc.pool, *meta, lora_on=lora_on, token_index=dc.token_index, out=y_na)
    torch.cuda.synchronize()
    return y_ref, y_na


@pytest.mark.parametrize("lora_on", [1, 0])
def test_noalloc_equals_linear_two_calls(lora_on):
    # call 1: 200 tokens on the tiled GEMM path (mixed ranks, a d_in tail);
    # call 2: 40 tokens on the split-K decode path, a smaller input that
    # finds the first call's contents in the scratch
    shapes = [(501, 1000, 700, 200, {a: [8, 16, 32, 64][a % 4] for a in range(12)}),
              (502, 512, 320, 40, {a: [16, 8][a % 2] for a in range(6)})]
    for seed, d_in, d_out, T, ranks in shapes:
        ids = sorted(np.random.default_rng(seed).integers(-1, len(ranks), size=T).tolist())
        log(f"[noalloc] lora_on={lora_on}: {d_in}->{d_out}, T={T}")
        c = make_custom_case(seed, "bf16", d_in, d_out, ids, ranks)
        dc = DeviceCase(c)
        y_ref, y_na = _run_both(dc, lora_on)
        assert torch.equal(y_na.view(torch.int16), y_ref.view(torch.int16)), f"T={T}: outputs differ"
        compare(y_host(y_na), oracle.case_linear(c, lora_on, threads=oracle_threads()), BF16_TOL,
                f"noalloc T={T} lora_on={lora_on}")


def test_noalloc_refuses_a_call_beyond_the_scratch():
    # 65536 tokens at max rank 256: the v tables alone need far more than the
    # scratch; the call returns MLORA_ERR_WORKSPACE and writes nothing
    import rank_adapter_gemm_segmented_amd as ml
    T, d = 65536, 64
    pool = ml.Pool(d, d, torch.bfloat16, 256, 1)
    assert pool.workspace_bytes(T) > (64 << 20)
    x = torch.zeros((T, d), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((d, d), dtype=torch.bfloat16, device="cuda")
    y = torch.full((T, d), 5.0, dtype=torch.bfloat16, device="cuda")
    ss = i32(np.array([0, T], np.int32))
    with pytest.raises(ml.MloraError) as e:
        ml.linear_noalloc(x, W, pool, ss, i32(np.array([-1], np.int32)), i32(np.array([0], np.int32)),
                          f32(np.array([0.0], np.float32)), lora_on=1, out=y)
    assert e.value.code == ml.STATUS_CODE["MLORA_ERR_WORKSPACE"]
    torch.cuda.synchronize()
    assert bool((y == 5.0).all())
