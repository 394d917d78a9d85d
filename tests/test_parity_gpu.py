"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle on the
same seeded inputs, element by element.

Tolerances: bf16 outputs |y - y_ref| <= 2e-2 (1 + |y_ref|); fp32 outputs
|y - y_ref| <= 1e-4 (1 + |y_ref|). Integer outputs (segmentation, token map)
are compared bit for bit.

Workloads at full size: every row where the oracle takes seconds, otherwise
the first and last row of every segment plus seeded random rows, computed by
the oracle one by one.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
from gpu_util import (BF16_TOL, DeviceCase, check_case, compare, i32, f32, log, oracle_threads,
                      sample_rows, y_host)
from mlora_inputs import PREFILL_SHAPES, make_case, make_custom_case

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=2)
def _dev(name, proj="q"):
    log(f"[parity] building {name} {proj}")
    return DeviceCase(make_case(name, proj))


@pytest.mark.parametrize("lora_on", [0, 1])
def test_tiny_f32(lora_on):
    log(f"[parity] tiny_f32 lora_on={lora_on}")
    check_case(_dev("tiny_f32"), lora_on)


@pytest.mark.parametrize("lora_on", [0, 1])
def test_decode_bf16(lora_on):
    log(f"[parity] decode_bf16 lora_on={lora_on}")
    check_case(_dev("decode_bf16"), lora_on)


@pytest.mark.parametrize("lora_on", [0, 1])
def test_verify_bf16(lora_on):
    # every row of the 128 x 2 batch: both tokens of every request
    log(f"[parity] verify_bf16 lora_on={lora_on} (all 256 rows)")
    check_case(_dev("verify_bf16"), lora_on)


def test_hetero_bf16_unsorted():
    log("[parity] hetero_bf16 (unsorted ids, library segments; all 256 rows)")
    dc = _dev("hetero_bf16")
    c = dc.case
    check_case(dc, 1)
    check_case(dc, 0)
    # integer outputs of the segmentation, bit for bit against the oracle
    import rank_adapter_gemm_segmented_amd as ml
    ti, ss, sa, sr, sc, ns = ml.build_segments(dc.token_adapter, dc.adapter_scale, dc.pool)
    torch.cuda.synchronize()
    o_ti, o_ss, o_sa = oracle.segment(c.token_adapter, c.capacity)
    S = int(ns.item())
    assert S == len(o_sa)
    assert np.array_equal(ti.cpu().numpy(), o_ti)
    assert np.array_equal(ss[:S + 1].cpu().numpy(), o_ss)
    assert np.array_equal(sa[:S].cpu().numpy(), o_sa)
    assert np.array_equal(sr[:S].cpu().numpy(), np.array([c.adapters[a].rank for a in o_sa]))
    assert np.array_equal(sc[:S].cpu().numpy(), c.adapter_scale[o_sa])
    # token map of the canonical segments
    ts, ta = ml.token_map(ss[:S + 1].contiguous(), sa[:S].contiguous(), c.n_tokens)
    o_ts, o_ta = oracle.token_map(o_ss, o_sa, c.n_tokens)
    assert np.array_equal(ts.cpu().numpy(), o_ts)
    assert np.array_equal(ta.cpu().numpy(), o_ta)


@pytest.mark.parametrize("proj", list(PREFILL_SHAPES))
def test_prefill_bf16(proj):
    log(f"[parity] prefill_bf16 {proj}")
    dc = _dev("prefill_bf16", proj)
    check_case(dc, 1, sample_rows(dc.case, 32))
    check_case(dc, 0, sample_rows(dc.case, 8, seed=2))


def test_decode_token_map_bit_exact():
    dc = _dev("decode_bf16")
    import rank_adapter_gemm_segmented_amd as ml
    ts, ta = ml.token_map(dc.seg_start, dc.seg_adapter, dc.case.n_tokens)
    o_ts, o_ta = oracle.token_map(dc.case.seg_start, dc.case.seg_adapter, dc.case.n_tokens)
    assert np.array_equal(ts.cpu().numpy(), o_ts)
    assert np.array_equal(ta.cpu().numpy(), o_ta)


# ---------------------------------------------------------------------------
# small edge cases, every row against the oracle
# ---------------------------------------------------------------------------

def _edge_cases():
    cases = []
    # (seed, dtype, d_in, d_out, ids, ranks, scales, sorted)
    cases.append((1, "bf16", 64, 64, [0], {0: 16}, None, True))                       # T = 1
    cases.append((2, "bf16", 72, 17, [0, 0, 1, 1, 1], {0: 3, 1: 7}, {0: -1.0, 1: 0.5}, True))
    cases.append((3, "bf16", 128, 1000, [-1, -1, 0, 2, 2, 2], {0: 1, 2: 8}, None, True))
    cases.append((4, "bf16", 4104, 96, list(range(17)), {a: 16 for a in range(17)}, None, True))
    cases.append((5, "bf16", 256, 320, [0] * 40 + [1] * 25, {0: 64, 1: 32}, {0: 0.0, 1: 2.0}, True))
    cases.append((6, "bf16", 512, 200, sorted(np.random.default_rng(6).integers(-1, 9, size=300).tolist()),
                  {a: [8, 16, 32, 64, 1, 3, 7, 24, 40][a] for a in range(9)}, None, True))
    cases.append((7, "bf16", 256, 130, np.random.default_rng(7).integers(-1, 12, size=77).tolist(),
                  {a: [8, 16, 32, 64][a % 4] for a in range(12)}, None, False))
    cases.append((8, "f32", 64, 48, [0, 0, 1, -1, 1, 1, 2], {0: 2, 1: 5, 2: 3}, {0: 1.5, 1: -2.0, 2: 0.25}, True))
    cases.append((9, "f32", 256, 256, np.random.default_rng(9).integers(-1, 4, size=33).tolist(),
                  {0: 8, 1: 8, 2: 4, 3: 1}, None, False))
    cases.append((10, "bf16", 64, 64, [0, 1], {0: 256, 1: 100}, None, True))          # large ranks
    # small-T path with device-built segments (unsorted ids)
    cases.append((11, "bf16", 320, 200, np.random.default_rng(11).integers(-1, 10, size=50).tolist(),
                  {a: [8, 16, 32, 64, 24][a % 5] for a in range(10)}, None, False))
    # 64 one-token segments on a single 64-row tile: one shrink segment per lane
    cases.append((12, "bf16", 192, 64, list(range(64)), {a: [8, 16, 4, 12][a % 4] for a in range(64)},
                  None, True))
    return cases


@pytest.mark.parametrize("idx", range(len(_edge_cases())))
def test_edge_case(idx):
    seed, dtype, d_in, d_out, ids, ranks, scales, srt = _edge_cases()[idx]
    log(f"[parity] edge case {idx}: {dtype} {d_in}->{d_out} T={len(ids)} sorted={srt}")
    c = make_custom_case(seed, dtype, d_in, d_out, ids, ranks, scales=scales, sorted_input=srt)
    dc = DeviceCase(c)
    check_case(dc, 1)
    check_case(dc, 0)


def test_empty_segments_and_base_only_segments():
    # explicit empty segments inside sorted metadata
    c = make_custom_case(21, "bf16", 128, 64, [0, 0, 1, 1, 1, 2], {0: 16, 1: 8, 2: 4})
    dc = DeviceCase(c)
    ss = np.array([0, 0, 2, 2, 5, 5, 6], np.int32)
    sa = np.array([1, 0, 2, 1, -1, 2], np.int32)
    sr = np.array([8, 16, 4, 8, 0, 4], np.int32)
    sc = np.array([1.0, 2.0, 3.0, -1.0, 0.0, 0.5], np.float32)
    import rank_adapter_gemm_segmented_amd as ml
    y = ml.linear(dc.x, dc.W, dc.pool, i32(ss), i32(sa), i32(sr), f32(sc), lora_on=1, workspace=dc.ws)
    torch.cuda.synchronize()
    pool = oracle.PackedPool(c.adapters, c.capacity, c.d_in, c.d_out)
    y_ref = oracle.linear(c.x, c.W, pool, ss, sa, sr, sc, None, 1)
    compare(y_host(y), y_ref, 2e-2, "empty segments")


def test_zero_tokens_is_noop():
    c = make_custom_case(22, "bf16", 64, 64, [0], {0: 8})
    dc = DeviceCase(c)
    import rank_adapter_gemm_segmented_amd as ml
    x0 = dc.x[:0]
    y0 = ml.linear(x0, dc.W, dc.pool, dc.seg_start, dc.seg_adapter, dc.seg_rank, dc.seg_scale,
                   lora_on=1, workspace=dc.ws)
    torch.cuda.synchronize()
    assert y0.shape == (0, 64)


def test_lora_off_ignores_null_metadata():
    c = make_case("decode_bf16")
    dc = _dev("decode_bf16")
    import rank_adapter_gemm_segmented_amd as ml
    y = ml.linear(dc.x, dc.W, dc.pool, None, None, None, None, lora_on=0, workspace=dc.ws)
    torch.cuda.synchronize()
    y_ref = oracle.linear(c.x, c.W, oracle.PackedPool({}, 1, c.d_in, c.d_out), None, None, None, None,
                          None, 0, threads=oracle_threads())
    compare(y_host(y), y_ref, 2e-2, "lora_off null metadata")


# ---------------------------------------------------------------------------
# both bf16 paths (split-K decode path and tiled GEMM path) on the same shapes
# ---------------------------------------------------------------------------

_FORCED_SHAPES = [
    # (seed, d_in, d_out, sorted ids, rank or {id: rank})
    (81, 4096, 4096, sorted(np.random.default_rng(81).integers(0, 32, size=64).tolist()), 16),
    (82, 1024, 520, sorted(np.random.default_rng(82).integers(-1, 6, size=40).tolist()), 32),
    (83, 2056, 64, [0] * 9 + [1] * 7, 64),
    (84, 8192, 300, sorted(np.random.default_rng(84).integers(0, 64, size=33).tolist()), 8),
    (85, 640, 4096, [3], 16),
    # rank chunks wider than 64 columns: max rank 80 (a 64 + 16 split) and 256
    (86, 512, 200, [0] * 30 + [1] * 20 + [2] * 14, {0: 80, 1: 40, 2: 72}),
    (87, 256, 136, [-1] * 3 + [0] * 25 + [1] * 36 + [2] * 3, {0: 256, 1: 100, 2: 1}),
    # short segments of mixed rank <= 16 over 100 tokens: the unsplit shrink
    # that writes the final scaled v (zero past each segment's rank)
    (88, 1024, 1000, sorted(np.random.default_rng(88).integers(-1, 50, size=100).tolist()),
     {a: [8, 16, 4, 12][a % 4] for a in range(50)}),
    # T > 128 on the direct-to-LDS GEMM ring with a d_in tail (1000 = 15 * 64 + 40)
    (89, 1000, 700, sorted(np.random.default_rng(89).integers(-1, 12, size=200).tolist()),
     {a: [8, 16, 32, 64][a % 4] for a in range(12)}),
]


@pytest.mark.parametrize("path", ["decode", "gemm", "gemv"])
@pytest.mark.parametrize("idx", range(len(_FORCED_SHAPES)))
def test_forced_paths(path, idx, monkeypatch):
    seed, d_in, d_out, ids, r = _FORCED_SHAPES[idx]
    monkeypatch.setenv("MLORA_FORCE_PATH", path)
    log(f"[parity] forced {path}: {d_in}->{d_out} T={len(ids)} r={r}")
    ranks = r if isinstance(r, dict) else {a: r for a in set(ids) if a >= 0}
    c = make_custom_case(seed, "bf16", d_in, d_out, ids, ranks)
    dc = DeviceCase(c)
    check_case(dc, 1, what=f"forced {path} lora_on=1")
    check_case(dc, 0, what=f"forced {path} lora_on=0")


@pytest.mark.gpu
@pytest.mark.parametrize("T", [1536, 160])
def test_mid_size_batches(T):
    # T = 1536 at 4096 outputs takes the 128-row direct-to-LDS GEMM tile; T =
    # 160 the 64x128 one across two token tiles. d_in = 328 leaves a k tail.
    rng = np.random.default_rng(90 + T)
    ids = sorted(rng.integers(-1, 40, size=T).tolist())
    ranks = {a: [16, 64, 8, 32][a % 4] for a in range(40)}
    log(f"[parity] mid-size batch T={T}: 328->4096")
    c = make_custom_case(90 + T, "bf16", 328, 4096, ids, ranks)
    dc = DeviceCase(c)
    check_case(dc, 1, sample_rows(c, 48), what=f"mid-size T={T} lora_on=1")
    check_case(dc, 0, sample_rows(c, 16, seed=1), what=f"mid-size T={T} lora_on=0")


@pytest.mark.gpu
def test_workspace_for_max_tokens_serves_smaller_batches():
    # mlora_workspace_bytes(pool, N) covers every call of up to N tokens: a
    # workspace sized for a 256-token batch also serves decode batches
    # (T <= 64), whose split-K partial tiles larger batches do not use
    log("[parity] one workspace for batches of 16, 64 and 256 tokens")
    import rank_adapter_gemm_segmented_amd as ml
    ids = sorted(np.random.default_rng(7).integers(0, 8, size=256).tolist())
    c = make_custom_case(95, "bf16", 1024, 1536, ids, {a: 16 for a in range(8)})
    dc = DeviceCase(c)
    ws = dc.pool.workspace(256)
    assert ws.numel() >= dc.pool.workspace_bytes(16) and ws.numel() >= dc.pool.workspace_bytes(64)
    for T in (16, 64, 256):
        # the first T rows of the batch, with their own segments
        sub = make_custom_case(95, "bf16", 1024, 1536, ids[:T], {a: 16 for a in range(8)})
        sub.W, sub.adapters, sub.x = c.W, c.adapters, c.x[:T]
        y = ml.linear(dc.x[:T], dc.W, dc.pool, i32(sub.seg_start), i32(sub.seg_adapter),
                      i32(sub.seg_rank), f32(sub.seg_scale), lora_on=1, workspace=ws)
        torch.cuda.synchronize()
        compare(y_host(y), oracle.case_linear(sub, 1, threads=oracle_threads()), 2e-2,
                f"shared workspace T={T}")


@pytest.mark.gpu
@pytest.mark.parametrize("T", [47, 48, 64])
def test_wide_layer_path_switch(T):
    # 48..64 tokens on a layer of >= 8192 outputs take the tiled GEMM path by
    # default, 47 tokens the split-K decode path; both match the oracle
    log(f"[parity] wide layer, default path, T={T}: 512->8200")
    ids = sorted(np.random.default_rng(300 + T).integers(-1, 20, size=T).tolist())
    c = make_custom_case(300 + T, "bf16", 512, 8200, ids, {a: [16, 8, 32][a % 3] for a in range(20)})
    dc = DeviceCase(c)
    check_case(dc, 1, what=f"wide T={T} lora_on=1")
    check_case(dc, 0, what=f"wide T={T} lora_on=0")


def _short_segment_ids(seed, n_seg, n_ad):
    # runs of 1-3 positions, a few of 5-9 (several items of one segment),
    # some base-only runs (id -1); at most two positions per segment on average
    rng = np.random.default_rng(seed)
    ids = []
    for s in range(n_seg):
        n = int(rng.choice([1, 1, 2, 2, 2, 3])) if s % 23 else int(rng.integers(5, 10))
        ids += [int(rng.integers(-1, n_ad))] * n
    return ids


@pytest.mark.parametrize("shrink", ["short", "mfma"])
def test_short_segment_shrink(shrink, monkeypatch):
    # a verify-shaped batch (T > 64, T <= 2 * segments, ranks <= 16) takes the
    # vector-ALU shrink; MLORA_FORCE_SHRINK=mfma keeps the MFMA one. Ranks 4 and
    # 12 leave partial 8-row groups; d_in = 4104 leaves a column-group tail.
    if shrink == "mfma":
        monkeypatch.setenv("MLORA_FORCE_SHRINK", "mfma")
    ids = _short_segment_ids(120, 90, 40)
    T = len(ids)
    n_seg = 1 + sum(1 for i in range(1, T) if ids[i] != ids[i - 1])
    assert 64 < T <= 2 * n_seg, (T, n_seg)
    ranks = {a: [4, 8, 12, 16][a % 4] for a in range(40)}
    log(f"[parity] short segments ({shrink} shrink): 4104->300, T={T}, {n_seg} segments")
    c = make_custom_case(120, "bf16", 4104, 300, ids, ranks)
    dc = DeviceCase(c)
    check_case(dc, 1, what=f"short segments {shrink} lora_on=1")
    check_case(dc, 0, what=f"short segments {shrink} lora_on=0")


def test_short_segment_shrink_verify_shape(monkeypatch):
    # the verify batch (128 requests x 2 tokens, 128 rank-16 adapters) with
    # the MFMA shrink forced: every row against the oracle (the default run,
    # with the vector-ALU shrink, is test_verify_bf16)
    dc = _dev("verify_bf16")
    monkeypatch.setenv("MLORA_FORCE_SHRINK", "mfma")
    log("[parity] verify_bf16 with the MFMA shrink (all 256 rows)")
    check_case(dc, 1, what="verify_bf16 mfma shrink lora_on=1")
    monkeypatch.delenv("MLORA_FORCE_SHRINK")


def test_short_segment_shrink_with_token_index(capfd, monkeypatch):
    # host-known sorted segments over gathered rows (token_index): the
    # short-segment shrink reads x through the permutation. ~150 tokens over
    # 100 adapters of ranks 4-16, so segments average under two positions.
    import rank_adapter_gemm_segmented_amd as ml
    rng = np.random.default_rng(130)
    ids = rng.integers(-1, 100, size=150).tolist()
    ranks = {a: [4, 8, 12, 16][a % 4] for a in range(100)}
    cu = make_custom_case(130, "bf16", 1032, 520, ids, ranks, sorted_input=False)
    ti, ss, sa = oracle.segment(cu.token_adapter, cu.capacity)
    assert 64 < cu.n_tokens <= 2 * (len(ss) - 1), (cu.n_tokens, len(ss) - 1)
    sr = np.array([ranks[a] if a >= 0 else 0 for a in sa], np.int32)
    sc = np.array([cu.adapter_scale[a] if a >= 0 else 0 for a in sa], np.float32)
    dc = DeviceCase(cu)
    monkeypatch.setenv("MLORA_LOG", "1")
    capfd.readouterr()
    y = ml.linear(dc.x, dc.W, dc.pool, i32(ss), i32(sa), i32(sr), f32(sc), lora_on=1,
                  token_index=i32(ti), workspace=dc.ws)
    torch.cuda.synchronize()
    err = capfd.readouterr().err
    assert "shrink=short" in err, err
    log(f"[parity] short segments with token_index: T={cu.n_tokens}, {len(ss) - 1} segments")
    y_ref = oracle.case_linear(cu, 1, threads=oracle_threads())
    compare(y_host(y), y_ref, BF16_TOL, "short segments with token_index")


@pytest.mark.parametrize("shrink", ["short", "mfma"])
def test_max_segments(shrink, monkeypatch):
    # MLORA_MAX_SEGMENTS one-token segments (adapter ids cycling over 64
    # adapters, so an adapter serves many segments) on a small layer: the
    # shrinks' segment scans and LDS tables at their largest, T = 16384
    if shrink == "mfma":
        monkeypatch.setenv("MLORA_FORCE_SHRINK", "mfma")
    S = 16384   # MLORA_MAX_SEGMENTS (include/mlora.h)
    ids = [s % 64 for s in range(S)]
    log(f"[parity] max segments ({shrink} shrink): 64->48, T={S}, {S} segments")
    c = make_custom_case(140, "bf16", 64, 48, ids, {a: [4, 8, 16][a % 3] for a in range(64)})
    assert len(c.seg_start) - 1 == S
    dc = DeviceCase(c)
    check_case(dc, 1, what=f"max segments {shrink} lora_on=1")


MAX_DIM = 1 << 17   # MLORA_MAX_DIM (include/mlora.h)


@pytest.mark.parametrize("d_in,d_out", [(MAX_DIM, 8), (64, MAX_DIM)])
@pytest.mark.parametrize("T", [40, 100])
def test_max_dims(d_in, d_out, T):
    # the largest d_in (128 decode chunks of 1024; a 4096-step GEMM k loop)
    # and the largest d_out (2048 decode tiles), on both paths
    rng = np.random.default_rng(150 + T)
    ids = sorted(rng.integers(-1, 4, size=T).tolist())
    log(f"[parity] max dims: {d_in}->{d_out}, T={T}")
    c = make_custom_case(150 + T, "bf16", d_in, d_out, ids, {0: 16, 1: 8, 2: 4, 3: 16})
    dc = DeviceCase(c)
    rows = sample_rows(c, 8) if d_out == MAX_DIM else None
    check_case(dc, 1, rows, what=f"max dims {d_in}->{d_out} T={T} lora_on=1")
    check_case(dc, 0, rows, what=f"max dims {d_in}->{d_out} T={T} lora_on=0")


@pytest.mark.parametrize("sorted_input", [True, False])
def test_max_rank_gemm_path(sorted_input):
    # MLORA_MAX_RANK (256) and odd large ranks on the tiled-GEMM path: the
    # epilogue's four 64-column rank chunks, the shrink's several passes
    rng = np.random.default_rng(160)
    ids = rng.integers(-1, 5, size=150)
    ids = np.sort(ids) if sorted_input else ids
    ranks = {0: 256, 1: 200, 2: 1, 3: 129, 4: 64}
    log(f"[parity] max rank on the GEMM path: 264->130, T=150, sorted={sorted_input}")
    c = make_custom_case(160, "bf16", 264, 130, ids.tolist(), ranks, sorted_input=sorted_input)
    dc = DeviceCase(c)
    check_case(dc, 1, what=f"max rank sorted={sorted_input} lora_on=1")
    check_case(dc, 0, what=f"max rank sorted={sorted_input} lora_on=0")


def test_unsorted_tokens_beyond_the_lds_table_bound():
    # 8192 unsorted tokens over about 3000 registered rank-8 adapters: the
    # host's segment bound (8192) is past the shrink's LDS table limit (4096)
    # while the device count (~2800) is under it. The shrink must lay out its
    # LDS by the host bound, which sized the allocation; every row against
    # the oracle.
    T, n_ad = 8192, 3000
    rng = np.random.default_rng(170)
    ids = rng.integers(-1, n_ad, size=T).tolist()
    log(f"[parity] unsorted T={T} over {n_ad} rank-8 adapters: 64->48")
    c = make_custom_case(170, "bf16", 64, 48, ids, {a: 8 for a in range(n_ad)}, sorted_input=False)
    n_used = len(set(ids) - {-1})
    assert 4096 < T and n_used + 1 <= 4096, n_used
    dc = DeviceCase(c)
    check_case(dc, 1, what=f"unsorted T={T} lora_on=1")
    check_case(dc, 0, what=f"unsorted T={T} lora_on=0")
