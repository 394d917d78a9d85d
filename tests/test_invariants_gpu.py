"""GPU invariants that hold bit for bit, and the library's error paths.

* lora_on = 1 with every B = 0 equals lora_on = 0 (the adapter term vanishes;
  the base accumulation order does not depend on lora_on).
* Permuting the batch (rows with their adapter ids) permutes y exactly: no
  token's arithmetic depends on where it sits in a tile.
* Two runs give identical bits (no atomics in any reduction).
* Metadata checks on the device agree with the oracle's error semantics.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import DeviceCase, compare, f32, i32, log, to_dev, y_host
from mlora_inputs import Adapter, make_case, make_custom_case

pytestmark = pytest.mark.gpu


def _ml():
    import rank_adapter_gemm_segmented_amd as ml
    return ml


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_B_equals_lora_off(dtype):
    log(f"[invariant] B=0 equals lora_off ({dtype})")
    ids = sorted(np.random.default_rng(1).integers(0, 6, size=70).tolist())
    c = make_custom_case(31, dtype, 512, 384, ids, {a: [8, 16, 32, 64, 4, 12][a] for a in range(6)})
    for ad in c.adapters.values():
        ad.B[:] = 0
    dc = DeviceCase(c)
    y_on = dc.run(1).clone()
    y_off = dc.run(0).clone()
    assert torch.equal(y_on.view(torch.int16) if dtype == "bf16" else y_on.view(torch.int32),
                       y_off.view(torch.int16) if dtype == "bf16" else y_off.view(torch.int32))


def test_permutation_bitwise():
    log("[invariant] permutation")
    rng = np.random.default_rng(2)
    T = 150
    ids = rng.integers(-1, 20, size=T).tolist()
    ranks = {a: [8, 16, 32, 64][a % 4] for a in range(20)}
    c = make_custom_case(41, "bf16", 1024, 640, ids, ranks, sorted_input=False)
    dc = DeviceCase(c)
    ml = _ml()
    y = dc.run(1).clone()
    perm = rng.permutation(T)
    xp = dc.x[torch.from_numpy(perm).cuda()].contiguous()
    tp = i32(np.asarray(ids, np.int32)[perm])
    yp = ml.linear_tokens(xp, dc.W, dc.pool, tp, dc.adapter_scale, lora_on=1, workspace=dc.ws)
    torch.cuda.synchronize()
    assert torch.equal(yp.view(torch.int16), y[torch.from_numpy(perm).cuda()].view(torch.int16))


@pytest.mark.parametrize("name", ["decode_bf16", "hetero_bf16"])
def test_run_to_run_determinism(name):
    log(f"[invariant] determinism {name}")
    dc = DeviceCase(make_case(name))
    y1 = dc.run(1).clone()
    y2 = dc.run(1).clone()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_sorted_and_unsorted_paths_agree():
    # the same batch given pre-grouped (sorted metadata) or unsorted (library
    # segments it) yields the same bits
    log("[invariant] sorted vs unsorted")
    rng = np.random.default_rng(3)
    ids = rng.integers(-1, 10, size=90)
    ranks = {a: [8, 16, 32][a % 3] for a in range(10)}
    cu = make_custom_case(51, "bf16", 768, 512, ids.tolist(), ranks, sorted_input=False)
    dc = DeviceCase(cu)
    y_u = y_host(dc.run(1))
    ti, ss, sa = oracle.segment(cu.token_adapter, cu.capacity)
    sr = np.array([ranks[a] if a >= 0 else 0 for a in sa], np.int32)
    sc = np.array([cu.adapter_scale[a] if a >= 0 else 0 for a in sa], np.float32)
    ml = _ml()
    y_s = ml.linear(dc.x, dc.W, dc.pool, i32(ss), i32(sa), i32(sr), f32(sc), lora_on=1,
                    token_index=i32(ti), workspace=dc.ws)
    torch.cuda.synchronize()
    assert np.array_equal(y_host(y_s), y_u)


def test_validate_matches_oracle_errors():
    log("[invariant] validate")
    ml = _ml()
    c = make_custom_case(61, "bf16", 64, 64, [0, 0, 1, 1], {0: 8, 1: 16}, capacity=4)
    dc = DeviceCase(c)
    pool = oracle.PackedPool(c.adapters, c.capacity, 64, 64)

    def both(ss, sa, sr, ti=None):
        g = ml.validate(dc.pool, i32(ss), i32(sa), i32(sr), None if ti is None else i32(ti),
                        n_tokens=4, workspace=dc.ws)
        try:
            oracle.linear(c.x, c.W, pool, np.array(ss, np.int32), np.array(sa, np.int32),
                          np.array(sr, np.int32), np.ones(len(sa), np.float32),
                          None if ti is None else np.array(ti, np.int32), 1)
            o = 0
        except oracle.OracleError as e:
            o = {oracle.MLO_ERR_META: 8, oracle.MLO_ERR_ADAPTER: 5, oracle.MLO_ERR_RANK: 4}[e.code]
        return g, o

    for args in [([0, 2, 4], [0, 1], [8, 16]),
                 ([0, 2, 3], [0, 1], [8, 16]),
                 ([0, 3, 2, 4], [0, 1, 1], [8, 16, 16]),
                 ([0, 2, 4], [0, 3], [8, 16]),          # slot 3 not registered
                 ([0, 2, 4], [0, 9], [8, 16]),          # beyond capacity
                 ([0, 2, 4], [0, 1], [8, 8]),           # rank mismatch
                 ([0, 2, 4], [-1, 1], [0, 16]),
                 ([0, 2, 4], [0, 1], [8, 16], [1, 0, 3, 2]),
                 ([0, 2, 4], [0, 1], [8, 16], [1, 1, 3, 2])]:
        g, o = both(*args)
        assert g == o, (args, g, o)


def test_host_validation_errors():
    ml = _ml()
    c = make_custom_case(71, "bf16", 64, 64, [0, 0], {0: 8})
    dc = DeviceCase(c)
    E = ml.STATUS_CODE
    with pytest.raises(ml.MloraError) as e:
        ml.linear(dc.x, dc.W, dc.pool, dc.seg_start, dc.seg_adapter, dc.seg_rank, dc.seg_scale,
                  lora_on=2, workspace=dc.ws)
    assert e.value.code == E["MLORA_ERR_INVALID_ARG"]
    with pytest.raises(ml.MloraError) as e:
        ml.linear(dc.x, dc.W, dc.pool, None, None, None, None, lora_on=1, workspace=dc.ws)
    assert e.value.code == E["MLORA_ERR_INVALID_ARG"]
    with pytest.raises(ml.MloraError) as e:
        ml.linear(dc.x, dc.W, dc.pool, dc.seg_start, dc.seg_adapter, dc.seg_rank, dc.seg_scale,
                  lora_on=1, workspace=dc.ws[:64])
    assert e.value.code == E["MLORA_ERR_WORKSPACE"]
    # registration errors
    A = to_dev(c.adapters[0].A, "bf16")
    B = to_dev(c.adapters[0].B, "bf16")
    with pytest.raises(ml.MloraError) as e:
        dc.pool.register(0, A, B)
    assert e.value.code == E["MLORA_ERR_EXISTS"]
    with pytest.raises(ml.MloraError) as e:
        dc.pool.register(5, A, B)
    assert e.value.code == E["MLORA_ERR_ADAPTER"]
    assert dc.pool.rank(0) == 8
    dc.pool.unregister(0)
    assert dc.pool.rank(0) == 0
    with pytest.raises(ml.MloraError) as e:
        dc.pool.unregister(0)
    assert e.value.code == E["MLORA_ERR_ADAPTER"]
    # an unregistered adapter is reported by validate and contributes no term
    assert ml.validate(dc.pool, dc.seg_start, dc.seg_adapter, dc.seg_rank, n_tokens=2,
                       workspace=dc.ws) == E["MLORA_ERR_ADAPTER"]
    y_on = dc.run(1).clone()
    y_off = dc.run(0).clone()
    assert torch.equal(y_on.view(torch.int16), y_off.view(torch.int16))
    # re-register after unregister (hot swap)
    dc.pool.register(0, A, B)
    assert dc.pool.rank(0) == 8


@pytest.mark.gpu
def test_build_segments_at_the_token_limit():
    # the largest unsorted batch the library accepts (the segmentation kernel
    # keeps four ints per token in LDS): integer outputs bit for bit
    import rank_adapter_gemm_segmented_amd as ml
    T = 8192   # MLORA_MAX_UNSORTED_TOKENS
    rng = np.random.default_rng(61)
    ids = rng.integers(-1, 300, size=T).tolist()
    ranks = {a: [8, 16, 32][a % 3] for a in range(300)}
    log(f"[parity] build_segments at T={T}")
    c = make_custom_case(61, "bf16", 64, 64, ids, ranks, sorted_input=False)
    dc = DeviceCase(c)
    ti, ss, sa, sr, sc, ns = ml.build_segments(dc.token_adapter, dc.adapter_scale, dc.pool)
    torch.cuda.synchronize()
    o_ti, o_ss, o_sa = oracle.segment(c.token_adapter, c.capacity)
    S = int(ns.item())
    assert S == len(o_sa)
    assert np.array_equal(ti.cpu().numpy(), o_ti)
    assert np.array_equal(ss[:S + 1].cpu().numpy(), o_ss)
    assert np.array_equal(sa[:S].cpu().numpy(), o_sa)
    assert np.array_equal(sr[:S].cpu().numpy(), np.array([c.adapters[a].rank if a >= 0 else 0 for a in o_sa]))


@pytest.mark.parametrize("T", [0, 1, 3, 64, 65, 130, 256, 511, 513, 1024, 1100, 3000])
def test_build_segments_stable_grouping(T):
    # Canonical segmentation is a stable sort of the rows by id: ids ascending,
    # rows of one id in batch order, one segment per distinct id. Ids outside
    # [-1, capacity) (down to INT32_MIN, up to INT32_MAX) stay segments of
    # their own value with rank 0 and scale 0. Sizes span one to several
    # 64-token groups, split and unsplit count ranges, and ragged tails.
    ml = _ml()
    log(f"[parity] build_segments stable grouping T={T}")
    rng = np.random.default_rng(900 + T)
    cap = 40
    extreme = np.array([-2**31, -7, -2, cap, 99999, 2**31 - 2, 2**31 - 1], np.int64)
    ids = np.where(rng.random(T) < 0.15, rng.choice(extreme, size=T),
                   rng.integers(-1, cap, size=T)).astype(np.int32)
    pool = ml.Pool(64, 64, torch.bfloat16, 16, cap)
    ranks = {a: [8, 16][a % 2] for a in range(0, cap, 3)}
    for a, r in ranks.items():
        pool.register(a, torch.zeros(r, 64, dtype=torch.bfloat16, device="cuda"),
                      torch.zeros(64, r, dtype=torch.bfloat16, device="cuda"))
    scale = (np.arange(cap, dtype=np.float32) + 1) / 8
    ti, ss, sa, sr, sc, ns = ml.build_segments(i32(ids), f32(scale), pool)
    torch.cuda.synchronize()
    if T == 0:   # an empty batch: no segments, seg_start = [0]
        assert int(ns.item()) == 0 and int(ss[0].item()) == 0
        return
    order = np.argsort(ids, kind="stable")
    sid = ids[order]
    starts = np.flatnonzero(np.r_[True, sid[1:] != sid[:-1]])
    S = int(ns.item())
    assert S == len(starts)
    assert np.array_equal(ti.cpu().numpy(), order)
    assert np.array_equal(ss[:S + 1].cpu().numpy(), np.r_[starts, T])
    assert np.array_equal(sa[:S].cpu().numpy(), sid[starts])
    valid = [0 <= a < cap for a in sid[starts]]
    assert np.array_equal(sr[:S].cpu().numpy(),
                          [ranks.get(int(a), 0) if v else 0 for a, v in zip(sid[starts], valid)])
    assert np.array_equal(sc[:S].cpu().numpy(),
                          np.array([scale[a] if v else 0 for a, v in zip(sid[starts], valid)], np.float32))


def test_debug_validate_mode(monkeypatch):
    # MLORA_DEBUG_VALIDATE=1: bad metadata is reported by the layer call itself
    # (and nothing is written); good metadata gives the ordinary result
    log("[invariant] MLORA_DEBUG_VALIDATE")
    ml = _ml()
    E = ml.STATUS_CODE
    ids = sorted(np.random.default_rng(9).integers(0, 4, size=24).tolist())
    c = make_custom_case(91, "bf16", 256, 192, ids, {a: 8 for a in range(4)})
    dc = DeviceCase(c)
    y_plain = dc.run(1).clone()
    monkeypatch.setenv("MLORA_DEBUG_VALIDATE", "1")
    assert torch.equal(dc.run(1).view(torch.int16), y_plain.view(torch.int16))
    bad = [
        ("seg_start ends short", dict(seg_start=np.r_[c.seg_start[:-1], c.seg_start[-1] - 1]), "MLORA_ERR_METADATA"),
        ("unregistered adapter", dict(seg_adapter=np.where(c.seg_adapter == 2, 7, c.seg_adapter)), "MLORA_ERR_ADAPTER"),
        ("rank mismatch", dict(seg_rank=c.seg_rank + 8), "MLORA_ERR_RANK"),
    ]
    for what, change, code in bad:
        meta = dict(seg_start=c.seg_start, seg_adapter=c.seg_adapter, seg_rank=c.seg_rank)
        meta.update(change)
        y = torch.full_like(y_plain, 7.0)
        with pytest.raises(ml.MloraError) as e:
            ml.linear(dc.x, dc.W, dc.pool, i32(meta["seg_start"]), i32(meta["seg_adapter"]),
                      i32(meta["seg_rank"]), f32(c.seg_scale), lora_on=1, out=y, workspace=dc.ws)
        assert e.value.code == E[code], what
        torch.cuda.synchronize()
        assert bool((y == 7.0).all()), f"{what}: the layer ran"
    monkeypatch.delenv("MLORA_DEBUG_VALIDATE")


def test_log_mode(monkeypatch, capfd):
    # MLORA_LOG=1: one stderr line per call naming the path taken
    log("[invariant] MLORA_LOG")
    ml = _ml()
    monkeypatch.setenv("MLORA_LOG", "1")
    for T, path in ((16, "path=decode "), (200, "path=gemm ")):
        ids = sorted(np.random.default_rng(T).integers(0, 4, size=T).tolist())
        dc = DeviceCase(make_custom_case(92, "bf16", 256, 192, ids, {a: 8 for a in range(4)}))
        capfd.readouterr()
        dc.run(1)
        err = capfd.readouterr().err
        assert path in err and f"T={T} " in err and "lora_on=1" in err, err
    monkeypatch.delenv("MLORA_LOG")
