"""The adapter term as a dense fp32 tile (k_expand_delta, added by the tiled
GEMM before its rounding) against the fp64 oracle, beside the GEMM
epilogue's MFMA expand on the same inputs.

The formula is the LoRA forward of *Multi-LoRA Serving in Practice*, section
"Core Principle: Shared Base Model, Per-Request Adapter Selection": y = W x +
scale * B (A x) per token, with each token's adapter chosen by its segment
(*InvisibleLoRA* abstract). Both expands compute the same term; the dense
one sums each output row's rank products in fp32 with the full fp32 v, the
MFMA one with v split into two bf16 parts. Each is checked on its own
against the oracle at the bf16 tolerance, on sorted and unsorted batches,
ragged token counts, mixed ranks (8 to 64, including ranks whose B rows are
not a power of two of 16-byte chunks), and segments without an adapter.
"""
import os

import numpy as np
import pytest
import torch

from gpu_util import DeviceCase, check_case, log, sample_rows
from mlora_inputs import make_custom_case

pytestmark = pytest.mark.gpu

# (seed, d_in, d_out, T, ranks by adapter id, sorted input)
SHAPES = [
    (201, 512, 640, 65, {a: [8, 16, 32, 64][a % 4] for a in range(12)}, True),
    (202, 768, 1032, 200, {a: [24, 40, 56, 8, 64][a % 5] for a in range(30)}, False),
    (203, 256, 2048, 512, {a: [64, 32][a % 2] for a in range(90)}, True),
    (204, 1024, 512, 130, {a: [8, 64][a % 2] for a in range(6)}, False),
    # sorted, mean segment over 16 positions: the shrink's 64-position items
    (206, 1024, 512, 130, {a: [8, 64][a % 2] for a in range(6)}, True),
]


class _Expand:
    """MLORA_EXPAND for the calls inside the block (read at every call)."""

    def __init__(self, mode):
        self.mode = mode

    def __enter__(self):
        self.old = os.environ.get("MLORA_EXPAND")
        os.environ["MLORA_EXPAND"] = self.mode

    def __exit__(self, *exc):
        if self.old is None:
            os.environ.pop("MLORA_EXPAND", None)
        else:
            os.environ["MLORA_EXPAND"] = self.old


def _case(seed, d_in, d_out, T, ranks, sorted_input):
    rng = np.random.default_rng(seed)
    # Zipf-like popularity over the pool plus base-only tokens (id -1)
    ids = rng.choice(np.arange(-1, len(ranks)), size=T,
                     p=np.r_[0.05, 0.95 * (1.0 / np.arange(1, len(ranks) + 1)) /
                             np.sum(1.0 / np.arange(1, len(ranks) + 1))])
    if sorted_input:
        ids = np.sort(ids, kind="stable")
    return make_custom_case(seed, "bf16", d_in, d_out, ids.tolist(), ranks, sorted_input=sorted_input)


@pytest.mark.parametrize("shape", SHAPES, ids=[f"T{s[3]}_{s[2]}_{'sorted' if s[5] else 'unsorted'}" for s in SHAPES])
@pytest.mark.parametrize("mode", ["dense", "mfma"])
def test_expand_against_oracle(shape, mode, capfd):
    seed, d_in, d_out, T, ranks, sorted_input = shape
    log(f"[dense-expand] {mode}: {d_in}->{d_out}, T={T}, sorted={sorted_input}")
    c = _case(*shape)
    dc = DeviceCase(c)
    os.environ["MLORA_LOG"] = "1"
    try:
        with _Expand(mode):
            check_case(dc, 1, sample_rows(c, 48), what=f"{mode} expand T={T} d_out={d_out}")
    finally:
        os.environ.pop("MLORA_LOG", None)
    err = capfd.readouterr().err
    want = "path=gemm-dense-expand" if mode == "dense" else "path=gemm "
    assert want in err, err[-400:]


def test_dense_expand_zero_B_equals_lora_off():
    log("[dense-expand] B = 0 gives the LoRA-off bits")
    c = _case(*SHAPES[1])
    for ad in c.adapters.values():
        ad.B[:] = 0
    dc = DeviceCase(c)
    with _Expand("dense"):
        y_on = dc.run(1).clone()
    y_off = dc.run(0).clone()
    assert torch.equal(y_on.view(torch.int16), y_off.view(torch.int16))


@pytest.mark.parametrize("max_rank,want", [(64, "path=gemm-dense-expand"), (16, "path=gemm ")])
def test_dense_expand_default_rule(max_rank, want, capfd):
    # the choice depends on the pool and T only: a pool whose largest rank is
    # at least 32 takes the dense term at T <= 512, a rank-16 pool keeps the
    # MFMA expand (sorted and unsorted forms of one batch then agree bit for
    # bit, which test_invariants_gpu checks on a rank-32 pool)
    log(f"[dense-expand] default rule, max rank {max_rank}")
    ranks = {a: min(max_rank, [8, 16, 32, 64][a % 4]) for a in range(16)}
    c = _case(205, 512, 768, 150, ranks, False)
    dc = DeviceCase(c)
    os.environ["MLORA_LOG"] = "1"
    try:
        os.environ.pop("MLORA_EXPAND", None)
        check_case(dc, 1, sample_rows(c, 32), what=f"default rule, max rank {max_rank}")
    finally:
        os.environ.pop("MLORA_LOG", None)
    assert want in capfd.readouterr().err
