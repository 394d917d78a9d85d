"""Host-side checks of the InvisibleLoRA cycle model (rank_adapter_gemm_segmented_amd.cycle).

The cycle (a LoRA-off draft pass over b tokens, one LoRA-on verification pass
over 2 b tokens, 1 + alpha tokens committed per request) and the run-time gate
follow the "InvisibleLoRA" abstract; the gate's rule is a reading (the abstract
names the gate but gives no rule): draft when the cycle's time per committed
token is below a plain LoRA-on step's.
"""
import pytest

import numpy as np

from rank_adapter_gemm_segmented_amd.cycle import break_even_alpha, cycle_estimate, verify_segments


def test_break_even_is_the_gate_boundary():
    t_on_b, t_off_b, t_on_2b = 100.0, 60.0, 120.0
    a = break_even_alpha(t_on_b, t_off_b, t_on_2b)
    assert a == pytest.approx(0.8)
    assert not cycle_estimate(t_on_b, t_off_b, t_on_2b, a).draft        # equal cost: no draft
    assert cycle_estimate(t_on_b, t_off_b, t_on_2b, 0.81).draft
    assert not cycle_estimate(t_on_b, t_off_b, t_on_2b, 0.79).draft


def test_unit_bytes_example_at_the_verify_shape():
    # the layer's algorithmic bytes as time (HBM-bound passes) at gate/up
    # 4096->14336, 128 requests, one rank-16 adapter each:
    #   plain step  = W + 128 adapters' A,B + x + y over 128 tokens
    #   draft pass  = W + x + y over 128 tokens; verify = W + adapters + x + y over 256 tokens
    W = 14336 * 4096 * 2
    ad = 128 * 16 * (4096 + 14336) * 2
    xy = lambda T: T * (4096 + 14336) * 2
    t_on_b, t_off_b, t_on_2b = W + ad + xy(128), W + xy(128), W + ad + xy(256)
    assert t_on_b == 197_656_576 and t_off_b + t_on_2b == 324_534_272
    est = cycle_estimate(t_on_b, t_off_b, t_on_2b, 0.95)
    assert est.speedup == pytest.approx(197_656_576 * 1.95 / 324_534_272)
    assert est.draft and 1.18 < est.speedup < 1.19


def test_never_drafts_when_a_cycle_costs_two_steps_or_more():
    # with t_off(b) + t_on(2b) >= 2 t_on(b) no acceptance rate can pay
    assert break_even_alpha(10.0, 10.0, 10.0) == pytest.approx(1.0)
    assert not cycle_estimate(10.0, 10.0, 10.0, 1.0).draft
    with pytest.raises(ValueError):
        cycle_estimate(10.0, 10.0, 10.0, 1.5)


def test_verify_segments_keep_each_request_in_its_segment():
    # draft: 5 requests, adapters grouped as [0, 0 | 3 | 7, 7]; verify: two
    # positions per request, request-major, so every position 2q, 2q + 1
    # falls in request q's segment
    ss = np.array([0, 2, 3, 5], np.int32)
    vs = verify_segments(ss)
    assert vs.tolist() == [0, 4, 6, 10] and vs.dtype == np.int32
    seg_of = lambda starts, p: int(np.searchsorted(starts, p, side="right") - 1)
    for q in range(5):
        for j in range(2):
            assert seg_of(vs, 2 * q + j) == seg_of(ss, q)
    assert verify_segments(ss, 3).tolist() == [0, 6, 9, 15]
    with pytest.raises(ValueError):
        verify_segments(np.array([1, 2], np.int32))
    with pytest.raises(ValueError):
        verify_segments(ss, 0)
