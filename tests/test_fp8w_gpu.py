"""GPU parity of the layer with an FP8 (e4m3) base weight (``mlora_linear_fp8w``).

The dequantized weight is W[n, k] = w_scale[n] * e4m3(codes[n, k]); x, the
adapters and y are bf16 ("LoRA Inference" glossary: FP8 quantization of the
served weights). Every e4m3 value is exact in bf16, so the kernels multiply
exactly as the bf16 layer does, and the bf16 layer's tolerance applies:
|y - y_ref| <= 2e-2 (1 + |y_ref|) against the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import BF16_TOL, compare, f32, i32, log, oracle_threads, to_dev, y_host
from mlora_inputs import e4m3_quantize_rows, make_custom_case, make_fp8w_case

pytestmark = pytest.mark.gpu


def _ml():
    import rank_adapter_gemm_segmented_amd as ml
    return ml


class Fp8Case:
    def __init__(self, case, codes, w_scale):
        ml = _ml()
        self.case, self.codes, self.w_scale = case, codes, w_scale
        self.x = to_dev(case.x, "bf16")
        self.W8 = torch.from_numpy(np.ascontiguousarray(codes)).cuda()
        self.ws = f32(w_scale)
        self.pool = ml.Pool(case.d_in, case.d_out, torch.bfloat16, case.max_rank, case.capacity)
        for aid, ad in sorted(case.adapters.items()):
            self.pool.register(aid, to_dev(ad.A, "bf16"), to_dev(ad.B, "bf16"))
        self.work = self.pool.workspace(case.n_tokens)
        self.meta = (i32(case.seg_start), i32(case.seg_adapter), i32(case.seg_rank), f32(case.seg_scale))
        self.token_index = None if case.token_index is None else i32(case.token_index)

    def run(self, lora_on):
        y = _ml().linear_fp8w(self.x, self.W8, self.ws, self.pool, *self.meta, lora_on=lora_on,
                              token_index=self.token_index, workspace=self.work)
        torch.cuda.synchronize()
        return y

    def check(self, lora_on, what):
        y = y_host(self.run(lora_on))
        y_ref = oracle.fp8w_case_linear(self.case, self.codes, self.w_scale, lora_on, threads=oracle_threads())
        worst = compare(y, y_ref, BF16_TOL, what)
        log(f"  {what}: max err/bound {worst:.3f}")


def _custom(seed, d_in, d_out, ids, ranks):
    c = make_custom_case(seed, "bf16", d_in, d_out, ids, ranks)
    codes, scale = e4m3_quantize_rows(c.W)
    return c, codes, scale


def test_fp8w_decode_batch():
    log("[fp8w] decode batch: 64 tokens, 4096->4096, 32 rank-16 adapters")
    fc = Fp8Case(*make_fp8w_case("decode_bf16"))
    fc.check(1, "decode fp8w lora_on=1")
    fc.check(0, "decode fp8w lora_on=0")


SHAPES = [
    # (seed, d_in, d_out, ids, ranks): a d_in tail chunk (2064 = 2 * 1024 + 16), ragged d_out,
    # base-only tokens, one token, mixed ranks up to 64
    (601, 2064, 520, sorted(np.random.default_rng(601).integers(-1, 6, size=40).tolist()), {a: [8, 16, 32, 64, 16, 8][a] for a in range(6)}),
    (602, 4096, 1024, [3], {3: 16}),
    (603, 1040, 4100, sorted(np.random.default_rng(603).integers(0, 20, size=33).tolist()), {a: 16 for a in range(20)}),
    (604, 14336, 256, sorted(np.random.default_rng(604).integers(-1, 4, size=17).tolist()), {a: 64 for a in range(4)}),
    # the largest d_in (MLORA_MAX_DIM): 256 chunks of 512 columns
    (607, 1 << 17, 8, sorted(np.random.default_rng(607).integers(-1, 3, size=24).tolist()), {a: 16 for a in range(3)}),
]


@pytest.mark.parametrize("idx", range(len(SHAPES)))
def test_fp8w_shapes(idx):
    seed, d_in, d_out, ids, ranks = SHAPES[idx]
    log(f"[fp8w] {d_in}->{d_out}, T={len(ids)}")
    fc = Fp8Case(*_custom(seed, d_in, d_out, ids, ranks))
    fc.check(1, f"fp8w {d_in}->{d_out} lora_on=1")
    fc.check(0, f"fp8w {d_in}->{d_out} lora_on=0")


def test_fp8w_zero_B_equals_lora_off():
    log("[fp8w] B = 0 equals LoRA-off bitwise")
    c, codes, scale = _custom(605, 2048, 768, sorted(np.random.default_rng(605).integers(0, 8, size=48).tolist()),
                              {a: 16 for a in range(8)})
    for ad in c.adapters.values():
        ad.B[:] = 0
    fc = Fp8Case(c, codes, scale)
    y_on, y_off = fc.run(1).clone(), fc.run(0).clone()
    assert torch.equal(y_on.view(torch.int16), y_off.view(torch.int16))


def test_fp8w_errors():
    log("[fp8w] shape and dtype errors")
    ml = _ml()
    E = ml.STATUS_CODE
    c, codes, scale = _custom(606, 1024, 256, [0] * 65, {0: 8})
    fc = Fp8Case(c, codes, scale)
    with pytest.raises(ml.MloraError) as e:        # 65 tokens: beyond the decode path
        fc.run(1)
    assert e.value.code == E["MLORA_ERR_SHAPE"]
    pool = ml.Pool(1000, 64, torch.bfloat16, 8, 2)  # d_in not a multiple of 16
    x = torch.zeros(4, 1000, dtype=torch.bfloat16, device="cuda")
    W8 = torch.zeros(64, 1000, dtype=torch.uint8, device="cuda")
    with pytest.raises(ml.MloraError) as e:
        ml.linear_fp8w(x, W8, torch.ones(64, device="cuda"), pool, lora_on=0)
    assert e.value.code == E["MLORA_ERR_SHAPE"]
    pool32 = ml.Pool(1024, 64, torch.float32, 8, 2)
    lib = ml.library()
    import ctypes
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    y = torch.empty(4, 64, dtype=torch.bfloat16, device="cuda")
    ws = pool32.workspace(4)
    x2 = torch.zeros(4, 1024, dtype=torch.bfloat16, device="cuda")
    W82 = torch.zeros(64, 1024, dtype=torch.uint8, device="cuda")
    sc = torch.ones(64, device="cuda")
    rc = lib.mlora_linear_fp8w(ctypes.c_void_p(x2.data_ptr()), ctypes.c_void_p(W82.data_ptr()),
                               ctypes.c_void_p(sc.data_ptr()), pool32.handle, None, None, None, None, None,
                               4, 0, 0, ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                               ws.numel(), st)
    assert rc == E["MLORA_ERR_DTYPE"]
