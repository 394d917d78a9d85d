"""Seeded synthetic workloads for the multi-LoRA segmented linear layer.

This module only draws and lays out inputs. It holds none of the layer's
arithmetic: no products, no sums over d_in, no adapter terms. It is the one
piece of code shared by the fp64 oracle (``oracle/``) and the GPU path
(``rank_adapter_gemm_segmented_amd``), so both see identical input values.

Every tensor is returned as float32 numpy arrays whose values are exactly
representable in the case's storage dtype (bf16 values are rounded from the
float32 draw by round-to-nearest-even), plus the raw bf16 bit patterns where
the dtype is bf16.

Workloads (names and shapes follow the five benchmark configurations of the
layer; sigma in N(0, sigma) is a standard deviation):

* ``tiny_f32``      fp32, 256->256, 16 tokens, 4 adapters of rank 8, four
                    contiguous segments of 4 tokens, scale = 16/8.
* ``decode_bf16``   q_proj 4096->4096, 64 tokens (one per request), 32 adapters
                    of rank 16 drawn i.i.d. uniform per request, then sorted
                    into segments by the caller, scale = 32/16.
* ``verify_bf16``   gate/up 4096->14336, 128 requests x 2 tokens, adapter q for
                    request q, rank 16, scale 2; the same shape with
                    lora_on = 0 is the LoRA-off drafter pass.
* ``hetero_bf16``   5120->5120, 256 tokens, adapter ids from a Zipf(1.1)
                    truncated to a 512-adapter pool, ranks drawn uniformly
                    from {8, 16, 32, 64}, alpha = 2 rank, ids left unsorted.
* ``prefill_bf16``  4096 tokens in 64 segments with Zipf(1.1) sizes (min 1),
                    rank 64, over one decoder layer's projections.

Seeds: workload k (1..5 in the order above) uses
``numpy.random.default_rng(1000 + k)``; a prefill projection additionally
mixes in its index. Draw order is W, then A and B for every pool adapter in
id order, then x, then the token assignment.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

__all__ = [
    "Adapter", "Case", "bf16_round", "bf16_bits", "bf16_from_bits",
    "make_case", "make_custom_case", "WORKLOADS", "PREFILL_SHAPES",
    "sorted_metadata", "zipf_probs", "make_merge_inputs", "make_fused_case", "FUSED_WORKLOADS",
    "e4m3_quantize_rows", "make_fp8w_case",
]


# ---------------------------------------------------------------------------
# bf16 rounding (storage conversion only)
# ---------------------------------------------------------------------------

def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    r = ((u + bias) >> 16) & 0xFFFF
    nan = np.isnan(a)
    if nan.any():
        r = np.where(nan, 0x7FC0, r)
    return r.astype(np.uint16)


def bf16_from_bits(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (RNE); result is float32."""
    return bf16_from_bits(bf16_bits(a))


# ---------------------------------------------------------------------------
# Case container
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Adapter:
    rank: int
    A: np.ndarray      # [rank, d_in]  float32 (dtype-representable)
    B: np.ndarray      # [d_out, rank] float32 (dtype-representable)


@dataclasses.dataclass
class Case:
    name: str
    dtype: str                       # "f32" or "bf16"
    d_in: int
    d_out: int
    n_tokens: int
    x: np.ndarray                    # [T, d_in] float32, caller token order
    W: np.ndarray                    # [d_out, d_in] float32
    adapters: Dict[int, Adapter]     # pool contents by adapter id
    capacity: int                    # pool slots (ids 0..capacity-1)
    max_rank: int
    adapter_scale: np.ndarray        # [capacity] float32, scale per adapter id
    token_adapter: np.ndarray        # [T] int32 adapter id per token (-1 = base only)
    sorted_input: bool               # True: tokens already grouped by the caller
    # Segment metadata over sorted positions (present when sorted_input):
    seg_start: Optional[np.ndarray] = None    # [S+1] int32
    seg_adapter: Optional[np.ndarray] = None  # [S] int32
    seg_rank: Optional[np.ndarray] = None     # [S] int32
    seg_scale: Optional[np.ndarray] = None    # [S] float32
    token_index: Optional[np.ndarray] = None  # [T] int32 or None (identity)

    @property
    def n_seg(self) -> int:
        return 0 if self.seg_adapter is None else int(self.seg_adapter.shape[0])

    def touched_adapters(self) -> List[int]:
        ids = sorted(set(int(a) for a in self.token_adapter.tolist() if a >= 0))
        return ids

    def bits(self, a: np.ndarray) -> np.ndarray:
        assert self.dtype == "bf16"
        return bf16_bits(a)


# ---------------------------------------------------------------------------
# Helpers
# ---------------------------------------------------------------------------

def zipf_probs(n: int, s: float) -> np.ndarray:
    """Zipf law truncated to support 1..n: p(k) proportional to k^-s."""
    k = np.arange(1, n + 1, dtype=np.float64)
    p = k ** (-s)
    return p / p.sum()


def _normal(rng: np.random.Generator, shape, sigma: float, dtype: str) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        a = (a * np.float32(sigma)).astype(np.float32)
    return bf16_round(a) if dtype == "bf16" else a


def sorted_metadata(token_adapter_sorted: np.ndarray, adapters: Dict[int, Adapter],
                    adapter_scale: np.ndarray):
    """Segment metadata for tokens that the caller has already grouped.

    ``token_adapter_sorted`` lists the adapter id of every token in batch
    order; runs of equal ids form the segments. Returns
    (seg_start, seg_adapter, seg_rank, seg_scale).
    """
    ids = np.asarray(token_adapter_sorted, dtype=np.int64)
    T = ids.shape[0]
    starts = [0]
    seg_ad = []
    for t in range(T):
        if t == 0 or ids[t] != ids[t - 1]:
            if t != 0:
                starts.append(t)
            seg_ad.append(int(ids[t]))
    if T == 0:
        seg_ad = []
        starts = [0]
    else:
        starts.append(T)
    seg_rank = [adapters[a].rank if a >= 0 else 0 for a in seg_ad]
    seg_scale = [float(adapter_scale[a]) if a >= 0 else 0.0 for a in seg_ad]
    return (np.asarray(starts, dtype=np.int32), np.asarray(seg_ad, dtype=np.int32),
            np.asarray(seg_rank, dtype=np.int32), np.asarray(seg_scale, dtype=np.float32))


def _make_pool(rng, ids_ranks: List[Tuple[int, int]], d_in, d_out, sigma_a, sigma_b, dtype):
    pool: Dict[int, Adapter] = {}
    for aid, r in ids_ranks:
        A = _normal(rng, (r, d_in), sigma_a, dtype)
        B = _normal(rng, (d_out, r), sigma_b, dtype)
        pool[aid] = Adapter(r, A, B)
    return pool


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------

# One decoder layer's projections for the prefill workload: name -> (d_in, d_out)
PREFILL_SHAPES = {
    "q": (4096, 4096), "k": (4096, 1024), "v": (4096, 1024), "o": (4096, 4096),
    "gate": (4096, 14336), "up": (4096, 14336), "down": (14336, 4096),
}

WORKLOADS = ("tiny_f32", "decode_bf16", "verify_bf16", "hetero_bf16", "prefill_bf16")


def make_case(name: str, proj: str = "q", lora_on: int = 1) -> Case:
    """Build one workload by name (see module docstring). ``proj`` selects the
    prefill projection. ``lora_on`` is recorded only for convenience."""
    if name == "tiny_f32":
        rng = np.random.default_rng(1001)
        d_in = d_out = 256
        T, n_ad, r = 16, 4, 8
        W = _normal(rng, (d_out, d_in), 0.02, "f32")
        pool = _make_pool(rng, [(a, r) for a in range(n_ad)], d_in, d_out, 0.02, 0.02, "f32")
        x = _normal(rng, (T, d_in), 1.0, "f32")
        tok = np.repeat(np.arange(n_ad, dtype=np.int32), T // n_ad)
        scale = np.full(n_ad, 16.0 / r, dtype=np.float32)
        ss, sa, sr, sc = sorted_metadata(tok, pool, scale)
        return Case(name, "f32", d_in, d_out, T, x, W, pool, n_ad, r, scale, tok, True,
                    ss, sa, sr, sc, None)

    if name == "decode_bf16":
        rng = np.random.default_rng(1002)
        d_in = d_out = 4096
        T, n_ad, r = 64, 32, 16
        W = _normal(rng, (d_out, d_in), 0.02, "bf16")
        pool = _make_pool(rng, [(a, r) for a in range(n_ad)], d_in, d_out, 0.02, 0.01, "bf16")
        x = _normal(rng, (T, d_in), 1.0, "bf16")
        draw = rng.integers(0, n_ad, size=T).astype(np.int32)
        # the caller groups its requests by adapter before the call
        tok = np.sort(draw, kind="stable").astype(np.int32)
        scale = np.full(n_ad, 32.0 / r, dtype=np.float32)
        ss, sa, sr, sc = sorted_metadata(tok, pool, scale)
        return Case(name, "bf16", d_in, d_out, T, x, W, pool, n_ad, r, scale, tok, True,
                    ss, sa, sr, sc, None)

    if name == "verify_bf16":
        rng = np.random.default_rng(1003)
        d_in, d_out = 4096, 14336
        n_req, per_req, r = 128, 2, 16
        T = n_req * per_req
        W = _normal(rng, (d_out, d_in), 0.02, "bf16")
        pool = _make_pool(rng, [(a, r) for a in range(n_req)], d_in, d_out, 0.02, 0.01, "bf16")
        x = _normal(rng, (T, d_in), 1.0, "bf16")
        tok = np.repeat(np.arange(n_req, dtype=np.int32), per_req)
        scale = np.full(n_req, 32.0 / r, dtype=np.float32)
        ss, sa, sr, sc = sorted_metadata(tok, pool, scale)
        return Case(name, "bf16", d_in, d_out, T, x, W, pool, n_req, r, scale, tok, True,
                    ss, sa, sr, sc, None)

    if name == "hetero_bf16":
        rng = np.random.default_rng(1004)
        d_in = d_out = 5120
        T, n_pool = 256, 512
        ranks = rng.choice(np.array([8, 16, 32, 64]), size=n_pool)
        W = _normal(rng, (d_out, d_in), 0.02, "bf16")
        pool = _make_pool(rng, [(a, int(ranks[a])) for a in range(n_pool)], d_in, d_out,
                          0.02, 0.01, "bf16")
        x = _normal(rng, (T, d_in), 1.0, "bf16")
        tok = rng.choice(n_pool, size=T, p=zipf_probs(n_pool, 1.1)).astype(np.int32)
        scale = np.array([2.0 * pool[a].rank / pool[a].rank for a in range(n_pool)],
                         dtype=np.float32)
        return Case(name, "bf16", d_in, d_out, T, x, W, pool, n_pool, 64, scale, tok, False)

    if name == "prefill_bf16":
        if proj not in PREFILL_SHAPES:
            raise ValueError(f"unknown projection {proj!r}")
        pidx = list(PREFILL_SHAPES).index(proj)
        rng = np.random.default_rng([1005, pidx])
        d_in, d_out = PREFILL_SHAPES[proj]
        T, n_seg, r = 4096, 64, 64
        W = _normal(rng, (d_out, d_in), 0.02, "bf16")
        pool = _make_pool(rng, [(a, r) for a in range(n_seg)], d_in, d_out, 0.02, 0.01, "bf16")
        x = _normal(rng, (T, d_in), 1.0, "bf16")
        sizes = rng.multinomial(T, zipf_probs(n_seg, 1.1)).astype(np.int64)
        while (sizes == 0).any():      # every segment keeps at least one token
            sizes[int(np.argmin(sizes))] += 1
            sizes[int(np.argmax(sizes))] -= 1
        tok = np.repeat(np.arange(n_seg, dtype=np.int32), sizes)
        scale = np.full(n_seg, 2.0, dtype=np.float32)
        ss, sa, sr, sc = sorted_metadata(tok, pool, scale)
        return Case(f"prefill_bf16_{proj}", "bf16", d_in, d_out, T, x, W, pool, n_seg, r,
                    scale, tok, True, ss, sa, sr, sc, None)

    raise ValueError(f"unknown workload {name!r}")


def make_custom_case(seed: int, dtype: str, d_in: int, d_out: int, token_adapter,
                     ranks: Dict[int, int], capacity: Optional[int] = None,
                     max_rank: Optional[int] = None, scales: Optional[Dict[int, float]] = None,
                     sorted_input: bool = True, sigma_w: float = 0.02, sigma_a: float = 0.02,
                     sigma_b: float = 0.01, sigma_x: float = 1.0) -> Case:
    """A small seeded case with a caller-chosen token->adapter assignment.

    With ``sorted_input`` the assignment is taken as already grouped (runs of
    equal ids become segments, so a repeated id may form several segments);
    otherwise it is left for the library to segment.
    """
    rng = np.random.default_rng(seed)
    tok = np.asarray(token_adapter, dtype=np.int32)
    T = int(tok.shape[0])
    ids = sorted(ranks)
    if capacity is None:
        capacity = (max(ids) + 1) if ids else 1
    if max_rank is None:
        max_rank = max(ranks.values()) if ranks else 1
    W = _normal(rng, (d_out, d_in), sigma_w, dtype)
    pool = _make_pool(rng, [(a, ranks[a]) for a in ids], d_in, d_out, sigma_a, sigma_b, dtype)
    x = _normal(rng, (T, d_in), sigma_x, dtype)
    scale = np.zeros(capacity, dtype=np.float32)
    for a in ids:
        scale[a] = np.float32(scales[a]) if scales and a in scales else np.float32(2.0)
    case = Case("custom", dtype, d_in, d_out, T, x, W, pool, capacity, max_rank, scale, tok,
                sorted_input)
    if sorted_input:
        ss, sa, sr, sc = sorted_metadata(tok, pool, scale)
        case.seg_start, case.seg_adapter, case.seg_rank, case.seg_scale = ss, sa, sr, sc
    return case


def make_merge_inputs(seed: int, dtype: str, d_in: int, d_out: int, rank: int,
                      sigma_w: float = 0.02, sigma_a: float = 0.02, sigma_b: float = 0.01):
    """Base weight W [d_out, d_in] and one adapter (A [rank, d_in], B [d_out, rank])
    for merging, drawn in that order from ``default_rng(seed)`` with the
    workloads' Gaussian inits, rounded to the storage dtype."""
    rng = np.random.default_rng(seed)
    W = _normal(rng, (d_out, d_in), sigma_w, dtype)
    A = _normal(rng, (rank, d_in), sigma_a, dtype)
    B = _normal(rng, (d_out, rank), sigma_b, dtype)
    return W, Adapter(rank, A, B)


# Stacked projections served by one fused call: workload -> (batch, projections)
FUSED_WORKLOADS = {
    "fused_qkv_decode": ("decode_bf16", ("q", "k", "v")),
    "fused_gateup_verify": ("verify_bf16", ("gate", "up")),
    "fused_qkv_prefill": ("prefill_bf16", ("q", "k", "v")),
    "fused_gateup_prefill": ("prefill_bf16", ("gate", "up")),
}


def make_fused_case(name: str) -> List[Case]:
    """One Case per stacked projection, all over the same batch.

    The first projection is the batch workload itself (its x, token
    assignment, segments, scales, and its W and adapters when the shapes
    agree); every later projection draws its own W [d_out_m, d_in] and, for
    every pool adapter id in order, A_m [r, d_in] and B_m [d_out_m, r] (same
    rank as the batch's adapter) from ``default_rng([3000, workload index,
    m])``. Shapes: ``PREFILL_SHAPES`` (the decode batch's q projection is
    4096->4096, its k and v 4096->1024; the verify batch's gate and up are
    4096->14336)."""
    batch, projs = FUSED_WORKLOADS[name]
    base = make_case(batch, projs[0])
    widx = list(FUSED_WORKLOADS).index(name)
    cases = []
    for m, proj in enumerate(projs):
        d_in, d_out = PREFILL_SHAPES[proj]
        assert d_in == base.d_in
        if m == 0 and d_out == base.d_out:
            cases.append(dataclasses.replace(base, name=f"{name}_{proj}"))
            continue
        rng = np.random.default_rng([3000, widx, m])
        W = _normal(rng, (d_out, d_in), 0.02, base.dtype)
        pool = _make_pool(rng, [(a, base.adapters[a].rank) for a in sorted(base.adapters)],
                          d_in, d_out, 0.02, 0.01, base.dtype)
        cases.append(dataclasses.replace(base, name=f"{name}_{proj}", d_out=d_out, W=W, adapters=pool))
    return cases


def e4m3_quantize_rows(W: np.ndarray):
    """A base weight stored as FP8: per output row a float32 scale
    s = max|W_row| / 448 (448 is the largest e4m3 value) and e4m3 codes of
    W_row / s, rounded to nearest even by torch's float8_e4m3fn cast. Returns
    (codes uint8 [d_out, d_in], scale float32 [d_out]). Rows of zeros get
    scale 1."""
    import torch
    W = np.ascontiguousarray(W, dtype=np.float32)
    amax = np.max(np.abs(W), axis=1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = torch.from_numpy(W / scale[:, None]).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).numpy().copy(), scale


def make_fp8w_case(name: str = "decode_bf16", proj: str = "q"):
    """A workload whose base weight is stored as FP8 (e4m3 codes plus a
    float32 scale per output row, from the workload's own W); x, adapters and
    segments are the workload's, in bf16. Returns (case, codes, scale)."""
    case = make_case(name, proj)
    codes, scale = e4m3_quantize_rows(case.W)
    return case, codes, scale
