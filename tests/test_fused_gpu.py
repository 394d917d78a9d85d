"""GPU parity of fused multi-projection LoRA (``mlora_register_adapter_fused``).

Several projections of one decoder layer (q|k|v, gate|up) are stacked into one
base weight, and each adapter registers its per-projection (A_m, B_m) as one
slot: A stacked, B block-diagonal. One ``mlora_linear`` call then serves every
projection: one read of x, one shrink over the stacked A, and each projection's
rows expand only their own part of v. An adapter's config names its target
modules with one rank and one scaling ("Multi-LoRA Serving in Practice",
section "1. Define Adapter Asset Standards").

The oracle is the plain layer per projection, outputs side by side. Tolerance
is the layer's bf16 bound, |y - y_ref| <= 2e-2 (1 + |y_ref|).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import BF16_TOL, compare, f32, i32, log, oracle_threads, sample_rows, to_dev, y_host
from mlora_inputs import FUSED_WORKLOADS, make_fused_case

pytestmark = pytest.mark.gpu


class FusedDeviceCase:
    """Stacked projections resident on the GPU with fused adapters registered."""

    def __init__(self, slices):
        import rank_adapter_gemm_segmented_amd as ml
        self.ml = ml
        self.slices = slices
        c0 = slices[0]
        n = len(slices)
        self.d_out = sum(c.d_out for c in slices)
        self.R = sum(c.max_rank for c in slices)
        self.x = to_dev(c0.x, "bf16")
        self.W = to_dev(np.vstack([c.W for c in slices]), "bf16")
        self.pool = ml.Pool(c0.d_in, self.d_out, torch.bfloat16, self.R, c0.capacity)
        for aid in sorted(c0.adapters):
            self.pool.register_fused(aid, [(to_dev(c.adapters[aid].A, "bf16"), to_dev(c.adapters[aid].B, "bf16"))
                                           for c in slices])
        self.ws = self.pool.workspace(c0.n_tokens)
        self.seg_start = i32(c0.seg_start)
        self.seg_adapter = i32(c0.seg_adapter)
        # a segment's rank is its adapter's stacked rank (the slices' ranks added)
        self.seg_rank = i32(np.where(c0.seg_adapter >= 0, sum(c.seg_rank for c in slices), 0))
        self.seg_scale = f32(c0.seg_scale)

    def run(self, lora_on):
        y = self.ml.linear(self.x, self.W, self.pool, self.seg_start, self.seg_adapter, self.seg_rank,
                           self.seg_scale, lora_on=lora_on, workspace=self.ws)
        torch.cuda.synchronize()
        return y


@pytest.mark.parametrize("name", sorted(FUSED_WORKLOADS))
def test_fused_parity(name):
    slices = make_fused_case(name)
    c0 = slices[0]
    log(f"[fused] {name}: T={c0.n_tokens}, d_out {[c.d_out for c in slices]}, rank {c0.max_rank} x {len(slices)}")
    dc = FusedDeviceCase(slices)
    # full rows up to the verify batch; prefill: every segment's first and last row plus random rows
    rows = None if c0.n_tokens <= 256 else sample_rows(c0, 96, seed=5)
    for lora_on in (1, 0):
        y = y_host(dc.run(lora_on))
        y_ref = oracle.fused_case_linear(slices, lora_on, rows=rows, threads=oracle_threads())
        worst = compare(y if rows is None else y[rows], y_ref, BF16_TOL, f"{name} lora_on={lora_on}")
        log(f"  lora_on={lora_on}: max err/bound {worst:.3f}")


def test_fused_matches_separate_calls_in_lora_term():
    # the fused call's adapter term per slice equals that of a separate call on
    # the slice (both against LoRA-off of the same call, so the base product's
    # summation order drops out); the difference of two bf16 outputs is
    # bounded by their two roundings
    name = "fused_qkv_decode"
    slices = make_fused_case(name)
    log(f"[fused] {name}: fused vs separate adapter terms")
    import rank_adapter_gemm_segmented_amd as ml
    dc = FusedDeviceCase(slices)
    y_on = y_host(dc.run(1))
    y_off = y_host(dc.run(0))
    n0 = 0
    for c in slices:
        pool = ml.Pool(c.d_in, c.d_out, torch.bfloat16, c.max_rank, c.capacity)
        for aid in sorted(c.adapters):
            pool.register(aid, to_dev(c.adapters[aid].A, "bf16"), to_dev(c.adapters[aid].B, "bf16"))
        W = to_dev(c.W, "bf16")
        ys_on = ml.linear(dc.x, W, pool, i32(c.seg_start), i32(c.seg_adapter), i32(c.seg_rank),
                          f32(c.seg_scale), lora_on=1)
        ys_off = ml.linear(dc.x, W, pool, lora_on=0)
        torch.cuda.synchronize()
        d_fused = y_on[:, n0:n0 + c.d_out] - y_off[:, n0:n0 + c.d_out]
        d_sep = y_host(ys_on) - y_host(ys_off)
        mag = np.abs(y_on[:, n0:n0 + c.d_out]) + np.abs(y_off[:, n0:n0 + c.d_out])
        assert np.all(np.abs(d_fused - d_sep) <= 1.5 * 2.0 ** -7 * mag + 1e-6), c.name
        n0 += c.d_out


def test_fused_registration_errors():
    log("[fused] registration errors")
    import rank_adapter_gemm_segmented_amd as ml
    E = ml.STATUS_CODE
    pool = ml.Pool(64, 48, torch.bfloat16, 16, 2)
    A = torch.zeros(8, 64, dtype=torch.bfloat16, device="cuda")
    B = torch.zeros(24, 8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ml.MloraError) as e:       # rows 24 + 20 != 48
        pool.register_fused(0, [(A, B), (A, B[:20])])
    assert e.value.code == E["MLORA_ERR_SHAPE"]
    with pytest.raises(ml.MloraError) as e:       # rank 8 + 8 + 8 > max_rank 16
        pool.register_fused(0, [(A, B[:16]), (A, B[:16]), (A, B[:16])])
    assert e.value.code == E["MLORA_ERR_RANK"]
    pool.register_fused(1, [(A, B), (A, B)])
    assert pool.rank(1) == 16
    with pytest.raises(ml.MloraError) as e:
        pool.register_fused(1, [(A, B), (A, B)])
    assert e.value.code == E["MLORA_ERR_EXISTS"]
    # the pool's W stacks 24 + 24 rows now: other slicings and plain adapters are refused
    with pytest.raises(ml.MloraError) as e:
        pool.register_fused(0, [(A, B[:16]), (A, torch.zeros(32, 8, dtype=torch.bfloat16, device="cuda"))])
    assert e.value.code == E["MLORA_ERR_SHAPE"]
    with pytest.raises(ml.MloraError) as e:
        pool.register(0, A, torch.zeros(48, 8, dtype=torch.bfloat16, device="cuda"))
    assert e.value.code == E["MLORA_ERR_SHAPE"]
    plain = ml.Pool(64, 48, torch.bfloat16, 16, 2)
    plain.register(0, A, torch.zeros(48, 8, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ml.MloraError) as e:          # and a pool of plain adapters takes no fused one
        plain.register_fused(1, [(A, B), (A, B)])
    assert e.value.code == E["MLORA_ERR_SHAPE"]


def _custom_slices(seed, d_in, rows, ranks_per_slice, ids, n_ad):
    from mlora_inputs import make_custom_case
    import dataclasses
    cs = [make_custom_case(seed + m, "bf16", d_in, rows[m], ids, {a: ranks_per_slice[m] for a in range(n_ad)})
          for m in range(len(rows))]
    return [cs[0]] + [dataclasses.replace(c, x=cs[0].x) for c in cs[1:]]


@pytest.mark.parametrize("T", [40, 200])
@pytest.mark.parametrize("layout", ["unequal_ranks", "straddling_tiles"])
def test_fused_slicing_cases(T, layout):
    # unequal slice ranks turn the window off for the pool; slice boundaries
    # inside a row tile keep that tile's full rank range; both stay exact
    ids = sorted(np.random.default_rng(T).integers(-1, 6, size=T).tolist())
    if layout == "unequal_ranks":
        slices = _custom_slices(700, 512, [256, 64, 64], [16, 8, 8], ids, 6)
    else:
        slices = _custom_slices(710, 512, [200, 72, 136], [16, 16, 16], ids, 6)
    log(f"[fused] {layout}, T={T}, rows {[c.d_out for c in slices]}")
    dc = FusedDeviceCase(slices)
    for lora_on in (1, 0):
        y = y_host(dc.run(lora_on))
        y_ref = oracle.fused_case_linear(slices, lora_on, threads=oracle_threads())
        worst = compare(y, y_ref, BF16_TOL, f"{layout} T={T} lora_on={lora_on}")
        log(f"  lora_on={lora_on}: max err/bound {worst:.3f}")


def test_fused_unsorted_batch():
    # the unsorted entry point segments the batch itself and takes each
    # segment's rank from the slot (the stacked rank of the fused adapter)
    name = "fused_qkv_decode"
    slices = make_fused_case(name)
    c0 = slices[0]
    log(f"[fused] {name} through mlora_linear_tokens, rows shuffled")
    dc = FusedDeviceCase(slices)
    perm = np.random.default_rng(3).permutation(c0.n_tokens)
    tok = c0.token_adapter[perm]
    xp = dc.x[torch.from_numpy(perm).cuda()].contiguous()
    y = dc.ml.linear_tokens(xp, dc.W, dc.pool, i32(tok), f32(c0.adapter_scale), lora_on=1, workspace=dc.ws)
    torch.cuda.synchronize()
    y_ref = oracle.fused_case_linear(slices, 1, threads=oracle_threads())[perm]
    worst = compare(y_host(y), y_ref, BF16_TOL, f"{name} unsorted")
    log(f"  max err/bound {worst:.3f}")


def test_fused_merge_equals_per_projection_merges():
    # merging a fused adapter into the stacked W merges every projection with
    # its own A_m, B_m: the zero blocks of B add exactly nothing
    import rank_adapter_gemm_segmented_amd as ml
    slices = make_fused_case("fused_qkv_decode")
    log("[fused] merge of a fused adapter vs per-projection merges")
    dc = FusedDeviceCase(slices)
    Wm = y_host(ml.merge_adapter(dc.W, dc.pool, 5, 2.0))
    n0 = 0
    for c in slices:
        pool = ml.Pool(c.d_in, c.d_out, torch.bfloat16, c.max_rank, c.capacity)
        pool.register(5, to_dev(c.adapters[5].A, "bf16"), to_dev(c.adapters[5].B, "bf16"))
        ref = y_host(ml.merge_adapter(to_dev(c.W, "bf16"), pool, 5, 2.0))
        torch.cuda.synchronize()
        assert np.array_equal(Wm[n0:n0 + c.d_out], ref), c.name
        n0 += c.d_out


@pytest.mark.parametrize("T", [40, 200])
def test_fused_max_slices(T):
    # MLORA_MAX_SLICES (8) stacked projections of 48 rows, equal ranks (the
    # windowed expand), on the decode and the GEMM path; a ninth slice is refused
    ids = sorted(np.random.default_rng(170 + T).integers(-1, 5, size=T).tolist())
    slices = _custom_slices(720, 256, [48] * 8, [8] * 8, ids, 5)
    log(f"[fused] 8 slices of 48 rows, rank 8 each, T={T}")
    dc = FusedDeviceCase(slices)
    for lora_on in (1, 0):
        y = y_host(dc.run(lora_on))
        y_ref = oracle.fused_case_linear(slices, lora_on, threads=oracle_threads())
        worst = compare(y, y_ref, BF16_TOL, f"8 slices T={T} lora_on={lora_on}")
        log(f"  lora_on={lora_on}: max err/bound {worst:.3f}")
    ml = dc.ml
    pool = ml.Pool(64, 9 * 8, torch.bfloat16, 9 * 4, 1)
    A = torch.zeros(4, 64, dtype=torch.bfloat16, device="cuda")
    B = torch.zeros(8, 4, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ml.MloraError) as e:
        pool.register_fused(0, [(A, B)] * 9)
    assert e.value.code == ml.STATUS_CODE["MLORA_ERR_SHAPE"]
