"""The layer captured in a HIP graph: every replay equals the eager call bit for bit.

Serving loops capture decode steps in graphs, and bench.py times its calls
as graph replays. The calls allocate nothing and record no memset, so a
graph holds only their kernels. Each test captures one call, then replays it
three times with eager work of the program (another layer call, a torch op)
and a synchronization between replays, clearing the output before each
replay, and compares every replay with the eager result.
"""
import numpy as np
import pytest
import torch

from gpu_util import DeviceCase, f32, i32, log, to_dev
from mlora_inputs import make_case, make_fp8w_case

pytestmark = pytest.mark.gpu


def _replays_match(call, eager_other):
    y_eager = call().clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        y_graph = call()
    for r in range(3):
        y_graph.zero_()
        eager_other()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_graph.view(torch.int16), y_eager.view(torch.int16)), f"replay {r}"
        assert float(y_graph.float().abs().sum()) > 0


@pytest.mark.parametrize("name", ["decode_bf16", "verify_bf16", "hetero_bf16"])
@pytest.mark.parametrize("lora_on", [1, 0])
def test_graph_replays_equal_eager(name, lora_on):
    log(f"[graph] {name} lora_on={lora_on}")
    c = make_case(name)
    dc = DeviceCase(c)
    y = torch.empty((c.n_tokens, c.d_out), dtype=torch.bfloat16, device="cuda")
    other = torch.empty_like(y)
    ws2 = dc.pool.workspace(c.n_tokens)
    ml = dc.ml

    def call(out=y, ws=dc.ws, lo=lora_on):
        if c.sorted_input:
            return ml.linear(dc.x, dc.W, dc.pool, dc.seg_start, dc.seg_adapter, dc.seg_rank, dc.seg_scale,
                             lora_on=lo, token_index=dc.token_index, out=out, workspace=ws)
        return ml.linear_tokens(dc.x, dc.W, dc.pool, dc.token_adapter, dc.adapter_scale, lora_on=lo,
                                out=out, workspace=ws)

    def eager_other():
        call(out=other, ws=ws2, lo=1 - lora_on)
        other.mul_(2)

    _replays_match(call, eager_other)


def test_graph_replays_equal_eager_fp8w():
    log("[graph] decode fp8w")
    import rank_adapter_gemm_segmented_amd as ml
    case, codes, wsc = make_fp8w_case("decode_bf16")
    pool = ml.Pool(case.d_in, case.d_out, torch.bfloat16, case.max_rank, case.capacity)
    for aid, ad in sorted(case.adapters.items()):
        pool.register(aid, to_dev(ad.A, "bf16"), to_dev(ad.B, "bf16"))
    x = to_dev(case.x, "bf16")
    W8 = torch.from_numpy(codes).cuda()
    sc = f32(wsc)
    meta = (i32(case.seg_start), i32(case.seg_adapter), i32(case.seg_rank), f32(case.seg_scale))
    y = torch.empty((case.n_tokens, case.d_out), dtype=torch.bfloat16, device="cuda")
    other = torch.empty_like(y)
    ws, ws2 = pool.workspace(case.n_tokens), pool.workspace(case.n_tokens)

    def call():
        return ml.linear_fp8w(x, W8, sc, pool, *meta, lora_on=1, out=y, workspace=ws)

    def eager_other():
        ml.linear_fp8w(x, W8, sc, pool, lora_on=0, out=other, workspace=ws2)

    _replays_match(call, eager_other)
