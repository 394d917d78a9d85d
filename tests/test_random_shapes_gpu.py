"""Seeded random small layers through the C ABI against the fp64 oracle.

Each case draws a shape (d_in a multiple of 8 for bf16 and of 4 for fp32, up
to 640; d_out up to 600, not a tile multiple), a token count on both sides of
the decode/GEMM boundary (1..300), a pool of adapters with mixed ranks (1..80)
and per-token adapter ids with base-only tokens (-1), given either grouped
(sorted metadata) or unsorted (the library segments them). Every row of y is
compared, LoRA-on and LoRA-off, at the layer's tolerance. Every fourth bf16
case is verify-shaped: many rank <= 16 adapters with one or two positions
each, grouped. The draw is fixed
by the seed, so a failure names a reproducible case.
"""
import numpy as np
import pytest

from gpu_util import DeviceCase, check_case, log
from mlora_inputs import make_custom_case

pytestmark = pytest.mark.gpu

N_CASES = 64


def _draw(i):
    rng = np.random.default_rng(7000 + i)
    dtype = "f32" if i % 6 == 5 else "bf16"
    step = 4 if dtype == "f32" else 8
    d_in = int(rng.integers(1, 81)) * step
    d_out = int(rng.integers(1, 601))
    T = int(rng.choice([int(rng.integers(1, 65)), int(rng.integers(65, 301))]))
    n_ad = int(rng.integers(1, 40))
    ranks = {a: int(rng.choice([1, 3, 8, 16, 24, 32, 64, 80])) for a in range(n_ad)}
    ids = rng.integers(-1, n_ad, size=T)
    if rng.random() < 0.5:   # long runs: fewer, longer segments
        ids = np.repeat(ids[: max(1, T // 8)], 8)[:T]
        if ids.size < T:
            ids = np.concatenate([ids, np.full(T - ids.size, ids[-1])])
    sorted_input = bool(rng.random() < 0.5)
    if i % 4 == 3 and dtype == "bf16":
        # verify-like: many adapters of rank <= 16, segments of one or two
        # positions, grouped, T > 64 (the short-segment shrink's regime)
        n_ad = int(rng.integers(48, 160))
        ranks = {a: int(rng.choice([1, 4, 8, 12, 16])) for a in range(n_ad)}
        seg_ids = rng.permutation(np.arange(-1, n_ad))[: int(rng.integers(40, n_ad))]
        ids = np.repeat(seg_ids, rng.integers(1, 3, size=seg_ids.size))
        sorted_input = True
        T = int(ids.size)
    elif sorted_input:
        ids = np.sort(ids)
    scales = {a: float(rng.choice([-1.0, 0.5, 2.0])) for a in range(n_ad)}
    return (dtype, d_in, d_out, ids.tolist(), ranks, scales, sorted_input)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_layer(i):
    dtype, d_in, d_out, ids, ranks, scales, srt = _draw(i)
    log(f"[random] case {i}: {dtype} {d_in}->{d_out} T={len(ids)} adapters={len(ranks)} sorted={srt}")
    c = make_custom_case(7000 + i, dtype, d_in, d_out, ids, ranks, scales=scales, sorted_input=srt)
    dc = DeviceCase(c)
    check_case(dc, 1, what=f"random case {i} lora_on=1")
    check_case(dc, 0, what=f"random case {i} lora_on=0")
