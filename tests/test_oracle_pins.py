"""Pins of the fp64 oracle against things other than itself.

Each ``pin_*`` function checks the oracle against a closed form, a library
routine (numpy fp64 products), an identity fixed by the pages, a hand-computed
example or exhaustive enumeration. ``test_oracle_mutants.py`` re-runs these
same pins against deliberately broken copies of the oracle to show that each
plausible mistake is caught by at least one of them.

Sources of the facts pinned:
* LoRA forward: "Multi-LoRA Serving in Practice", section "Core Principle"
  (displayed formula, base product plus scale times B applied to A x).
* Merged weights W = W0 + dW: "LoRA Inference" glossary, first paragraph
  (pinned for the layer and for the oracle's merge of one adapter).
* LoRA-off pass = base model alone; batch split among the adapters in use:
  "InvisibleLoRA" abstract.
* Grouping same-adapter requests: "Multi-LoRA Serving in Practice",
  section "4. Batching", the adapter-aware batching row of its table.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from mlora_inputs import Adapter, make_case, make_custom_case, bf16_round

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_example.json")


def _rel_err(a, b):
    return float(np.max(np.abs(a - b) / (1.0 + np.abs(b)))) if a.size else 0.0


def _pool(adapters, capacity, d_in, d_out):
    return oracle.PackedPool(adapters, capacity, d_in, d_out)


# ---------------------------------------------------------------------------
# pins (each takes the oracle library handle so mutants can be fed in)
# ---------------------------------------------------------------------------

def pin_hand_example(lib):
    g = json.load(open(GOLDEN))
    d_in, d_out = g["d_in"], g["d_out"]
    W = np.array(g["W"], np.float32)
    x = np.array(g["x"], np.float32)
    ads = {int(k): Adapter(v["rank"], np.array(v["A"], np.float32), np.array(v["B"], np.float32))
           for k, v in g["adapters"].items()}
    scale = np.array([g["adapters"][str(a)]["scale"] for a in range(2)], np.float32)
    ti, ss, sa = oracle.segment(g["token_adapter"], 2, lib=lib)
    assert ti.tolist() == g["expected_token_index"]
    assert ss.tolist() == g["expected_seg_start"]
    assert sa.tolist() == g["expected_seg_adapter"]
    sr = np.array([ads[a].rank if a >= 0 else 0 for a in sa], np.int32)
    sc = np.array([scale[a] if a >= 0 else 0 for a in sa], np.float32)
    pool = _pool(ads, 2, d_in, d_out)
    y_on = oracle.linear(x, W, pool, ss, sa, sr, sc, ti, 1, lib=lib)
    y_off = oracle.linear(x, W, pool, ss, sa, sr, sc, ti, 0, lib=lib)
    assert np.array_equal(y_on, np.array(g["expected_y_lora_on"], np.float64))
    assert np.array_equal(y_off, np.array(g["expected_y_lora_off"], np.float64))


def pin_base_is_library_product(lib):
    # lora_on = 0 is the base model alone; compare with numpy's fp64 product
    for seed, (T, d_in, d_out) in enumerate([(5, 7, 3), (9, 33, 17), (16, 64, 40)]):
        c = make_custom_case(seed, "f32", d_in, d_out, [0] * T, {0: 3})
        ref = c.x.astype(np.float64) @ c.W.astype(np.float64).T
        pool = _pool(c.adapters, c.capacity, d_in, d_out)
        y = oracle.linear(c.x, c.W, pool, c.seg_start, c.seg_adapter, c.seg_rank, c.seg_scale,
                          None, 0, lib=lib)
        assert _rel_err(y, ref) < 1e-12
        # an all-base-only batch with lora_on = 1 gives the same product
        y2 = oracle.linear(c.x, c.W, pool, np.array([0, T], np.int32), np.array([-1], np.int32),
                           np.array([0], np.int32), np.array([0], np.float32), None, 1, lib=lib)
        assert _rel_err(y2, ref) < 1e-12


def pin_lora_term_is_library_product(lib):
    # W = 0: y = scale_s * (x A^T) B^T per segment, compared with numpy
    T, d_in, d_out = 12, 40, 24
    ids = [0, 0, 0, 2, 2, 1, 1, 1, 1, -1, 2, 2]
    c = make_custom_case(11, "f32", d_in, d_out, ids, {0: 3, 1: 5, 2: 2},
                         scales={0: 0.5, 1: -1.5, 2: 3.0}, sigma_w=0.0)
    assert not c.W.any()
    pool = _pool(c.adapters, c.capacity, d_in, d_out)
    y = oracle.linear(c.x, c.W, pool, c.seg_start, c.seg_adapter, c.seg_rank, c.seg_scale,
                      None, 1, lib=lib)
    ref = np.zeros((T, d_out))
    for t, a in enumerate(ids):
        if a < 0:
            continue
        ad = c.adapters[a]
        v = c.x[t:t + 1].astype(np.float64) @ ad.A.astype(np.float64).T
        ref[t] = float(c.adapter_scale[a]) * (v @ ad.B.astype(np.float64).T)[0]
    assert _rel_err(y, ref) < 1e-12
    # a single adapter over the whole batch is one dense product
    c1 = make_custom_case(12, "f32", d_in, d_out, [1] * T, {1: 7}, scales={1: 1.25}, sigma_w=0.0)
    p1 = _pool(c1.adapters, c1.capacity, d_in, d_out)
    y1 = oracle.linear(c1.x, c1.W, p1, c1.seg_start, c1.seg_adapter, c1.seg_rank, c1.seg_scale,
                       None, 1, lib=lib)
    A = c1.adapters[1].A.astype(np.float64)
    B = c1.adapters[1].B.astype(np.float64)
    ref1 = 1.25 * ((c1.x.astype(np.float64) @ A.T) @ B.T)
    assert _rel_err(y1, ref1) < 1e-12


def pin_merged_weights(lib):
    # (W + scale_a B_a A_a) x_i: the merged-weight form of the same layer
    rng = np.random.default_rng(5)
    for trial in range(4):
        T = int(rng.integers(1, 17))
        d_in = int(rng.integers(1, 65))
        d_out = int(rng.integers(1, 65))
        n_ad = int(rng.integers(1, 5))
        ranks = {a: int(rng.integers(1, 9)) for a in range(n_ad)}
        ids = sorted(rng.integers(-1, n_ad, size=T).tolist())
        scales = {a: float(rng.normal()) for a in range(n_ad)}
        c = make_custom_case(100 + trial, "f32", d_in, d_out, ids, ranks, scales=scales)
        pool = _pool(c.adapters, c.capacity, d_in, d_out)
        y = oracle.linear(c.x, c.W, pool, c.seg_start, c.seg_adapter, c.seg_rank, c.seg_scale,
                          None, 1, lib=lib)
        W0 = c.W.astype(np.float64)
        for t, a in enumerate(ids):
            Wm = W0.copy()
            if a >= 0:
                ad = c.adapters[a]
                Wm += np.float64(np.float32(scales[a])) * (ad.B.astype(np.float64) @ ad.A.astype(np.float64))
            ref = Wm @ c.x[t].astype(np.float64)
            assert _rel_err(y[t], ref) < 1e-12, (trial, t)


def pin_vanishing_terms(lib):
    # B = 0, A = 0 or scale = 0 leave exactly the base output
    T, d_in, d_out = 8, 24, 20
    ids = [0, 0, 1, 1, 1, 2, 2, 2]
    base_case = make_custom_case(21, "f32", d_in, d_out, ids, {0: 4, 1: 2, 2: 6})
    pool = _pool(base_case.adapters, base_case.capacity, d_in, d_out)
    c = base_case
    y_off = oracle.linear(c.x, c.W, pool, c.seg_start, c.seg_adapter, c.seg_rank, c.seg_scale,
                          None, 0, lib=lib)
    for which in ("B", "A", "scale"):
        ads = {a: Adapter(ad.rank, ad.A.copy(), ad.B.copy()) for a, ad in c.adapters.items()}
        sc = c.seg_scale.copy()
        for ad in ads.values():
            if which == "B":
                ad.B[:] = 0
            elif which == "A":
                ad.A[:] = 0
        if which == "scale":
            sc[:] = 0
        p = _pool(ads, c.capacity, d_in, d_out)
        y = oracle.linear(c.x, c.W, p, c.seg_start, c.seg_adapter, c.seg_rank, sc, None, 1, lib=lib)
        assert np.array_equal(y, y_off), which
    # and with live adapters the output does differ from the base
    y_on = oracle.linear(c.x, c.W, pool, c.seg_start, c.seg_adapter, c.seg_rank, c.seg_scale,
                         None, 1, lib=lib)
    assert not np.array_equal(y_on, y_off)


def pin_one_hot_and_rank_one(lib):
    # integer-valued operands: every value below is exact in fp64
    rng = np.random.default_rng(9)
    d_in, d_out = 6, 5
    W = rng.integers(-3, 4, size=(d_out, d_in)).astype(np.float32)
    A0 = rng.integers(-2, 3, size=(3, d_in)).astype(np.float32)
    B0 = rng.integers(-2, 3, size=(d_out, 3)).astype(np.float32)
    ads = {0: Adapter(3, A0, B0)}
    pool = _pool(ads, 1, d_in, d_out)
    s = 0.75
    x = np.eye(d_in, dtype=np.float32)            # token k is e_k
    T = d_in
    y = oracle.linear(x, W, pool, np.array([0, T], np.int32), np.array([0], np.int32),
                      np.array([3], np.int32), np.array([s], np.float32), None, 1, lib=lib)
    for k in range(d_in):
        ref = W[:, k].astype(np.float64) + s * (B0.astype(np.float64) @ A0[:, k].astype(np.float64))
        assert np.array_equal(y[k], ref), k
    # rank one: A = e_k^T, B = e_n  =>  y_i[n] += s * x_i[k]
    k0, n0 = 4, 1
    A1 = np.zeros((1, d_in), np.float32); A1[0, k0] = 1
    B1 = np.zeros((d_out, 1), np.float32); B1[n0, 0] = 1
    p1 = _pool({0: Adapter(1, A1, B1)}, 1, d_in, d_out)
    xr = rng.integers(-4, 5, size=(3, d_in)).astype(np.float32)
    y1 = oracle.linear(xr, W, p1, np.array([0, 3], np.int32), np.array([0], np.int32),
                       np.array([1], np.int32), np.array([s], np.float32), None, 1, lib=lib)
    ref1 = xr.astype(np.float64) @ W.astype(np.float64).T
    ref1[:, n0] += s * xr[:, k0]
    assert np.array_equal(y1, ref1)


def pin_permutation(lib):
    # permuting the batch (tokens with their adapter ids) permutes the output rows
    rng = np.random.default_rng(13)
    T, d_in, d_out = 20, 48, 36
    ids = rng.integers(-1, 4, size=T).tolist()
    c = make_custom_case(31, "f32", d_in, d_out, ids, {0: 2, 1: 5, 2: 3, 3: 8},
                         scales={0: 1.0, 1: -0.5, 2: 2.0, 3: 0.25}, sorted_input=False)
    pool = _pool(c.adapters, c.capacity, d_in, d_out)

    def run(x, tok):
        ti, ss, sa = oracle.segment(tok, c.capacity, lib=lib)
        sr = np.array([c.adapters[a].rank if a >= 0 else 0 for a in sa], np.int32)
        sc = np.array([c.adapter_scale[a] if a >= 0 else 0 for a in sa], np.float32)
        return oracle.linear(x, c.W, pool, ss, sa, sr, sc, ti, 1, lib=lib)

    y = run(c.x, c.token_adapter)
    perm = rng.permutation(T)
    yp = run(c.x[perm], c.token_adapter[perm])
    assert np.array_equal(yp, y[perm])
    # the unsorted result agrees with the merged-weight form row by row
    for t in range(T):
        a = int(c.token_adapter[t])
        Wm = c.W.astype(np.float64)
        if a >= 0:
            ad = c.adapters[a]
            Wm = Wm + np.float64(c.adapter_scale[a]) * (ad.B.astype(np.float64) @ ad.A.astype(np.float64))
        assert _rel_err(y[t], Wm @ c.x[t].astype(np.float64)) < 1e-12


def pin_linearity(lib):
    T, d_in, d_out = 6, 16, 12
    ids = [0, 0, 1, 1, 1, 1]
    c = make_custom_case(41, "f32", d_in, d_out, ids, {0: 3, 1: 4})
    pool = _pool(c.adapters, c.capacity, d_in, d_out)

    def run(x, s):
        sc = np.full(c.seg_scale.shape, s, np.float32)
        return oracle.linear(x, c.W, pool, c.seg_start, c.seg_adapter, c.seg_rank, sc, None, 1, lib=lib)

    y0, y1, y2 = run(c.x, 0.0), run(c.x, 1.0), run(c.x, 2.0)
    assert _rel_err(y2 - y0, 2.0 * (y1 - y0)) < 1e-12
    # additivity in x with dyadic inputs (their float32 sum is exact)
    rng = np.random.default_rng(3)
    x1 = (rng.integers(-64, 65, size=(T, d_in)) / 16.0).astype(np.float32)
    x2 = (rng.integers(-64, 65, size=(T, d_in)) / 16.0).astype(np.float32)
    ya, yb, yab = run(x1, 1.5), run(x2, 1.5), run(x1 + x2, 1.5)
    assert _rel_err(yab, ya + yb) < 1e-12


def pin_segmentation_exhaustive(lib):
    # every id string of length <= 6 over {-1, 0, 1, 2} against a stable sort
    for T in range(0, 7):
        for ids in itertools.product((-1, 0, 1, 2), repeat=T):
            ti, ss, sa = oracle.segment(list(ids), 3, lib=lib)
            order = sorted(range(T), key=lambda t: ids[t])   # Python's sort is stable
            assert ti.tolist() == order, ids
            groups = []
            for t in order:
                if not groups or groups[-1][0] != ids[t]:
                    groups.append([ids[t], 0])
                groups[-1][1] += 1
            assert sa.tolist() == [g[0] for g in groups]
            assert ss.tolist() == [0] + list(np.cumsum([g[1] for g in groups]).tolist())


def pin_token_map(lib):
    rng = np.random.default_rng(17)
    for trial in range(200):
        S = int(rng.integers(1, 12))
        sizes = rng.integers(0, 5, size=S)          # empty segments allowed
        ss = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
        T = int(ss[-1])
        sa = rng.integers(-1, 7, size=S).astype(np.int32)
        ts, ta = oracle.token_map(ss, sa, T, lib=lib)
        exp_s = [s for s in range(S) for _ in range(int(sizes[s]))]
        assert ts.tolist() == exp_s
        assert ta.tolist() == [int(sa[s]) for s in exp_s]


# ---- merged weight W + c B A of one adapter (oracle.merge) ----------------
# "LoRA Inference" glossary, first paragraph: W = W0 + dW; dW = c B A is the
# low-rank term of the "Multi-LoRA Serving in Practice" LoRA forward.

def _merge_inputs(seed, d_in, d_out, r):
    rng = np.random.default_rng(seed)
    W = rng.normal(0, 0.02, (d_out, d_in)).astype(np.float32)
    A = rng.normal(0, 0.02, (r, d_in)).astype(np.float32)
    B = rng.normal(0, 0.01, (d_out, r)).astype(np.float32)
    return W, A, B


def pin_merge_is_library_product(lib):
    # a numpy fp64 matrix product of B and A, added to W
    for seed, (d_in, d_out, r, c) in enumerate([(40, 24, 5, 2.0), (17, 33, 1, -0.75), (64, 8, 16, 0.3)]):
        W, A, B = _merge_inputs(200 + seed, d_in, d_out, r)
        m = oracle.merge(W, A, B, c, lib=lib)
        ref = W.astype(np.float64) + np.float64(np.float32(c)) * (B.astype(np.float64) @ A.astype(np.float64))
        assert _rel_err(m, ref) < 1e-12, seed


def pin_merge_serves_like_adapter(lib):
    # a batch whose every token uses adapter a with scale c gives the same y
    # through the layer (LoRA-on) as through the merged weight alone
    rng = np.random.default_rng(9)
    for trial in range(3):
        T, d_in, d_out, r = int(rng.integers(1, 9)), int(rng.integers(2, 49)), int(rng.integers(2, 49)), int(rng.integers(1, 9))
        c = float(rng.normal())
        case = make_custom_case(300 + trial, "f32", d_in, d_out, [0] * T, {0: r}, scales={0: c})
        pool = _pool(case.adapters, case.capacity, d_in, d_out)
        y = oracle.linear(case.x, case.W, pool, case.seg_start, case.seg_adapter, case.seg_rank,
                          case.seg_scale, None, 1, lib=lib)
        m = oracle.merge(case.W, case.adapters[0].A, case.adapters[0].B, c, lib=lib)
        assert _rel_err(case.x.astype(np.float64) @ m.T, y) < 1e-12, trial


def pin_merge_closed_forms(lib):
    d_in, d_out = 12, 10
    W, _, _ = _merge_inputs(7, d_in, d_out, 1)
    # rank one with A = e_k^T, B = e_n: only W[n, k] moves, by exactly c
    for (n, k, c) in [(0, 0, 1.5), (9, 11, -2.0), (3, 7, 0.25)]:
        A = np.zeros((1, d_in), np.float32)
        A[0, k] = 1
        B = np.zeros((d_out, 1), np.float32)
        B[n, 0] = 1
        m = oracle.merge(W, A, B, c, lib=lib)
        ref = W.astype(np.float64)
        ref[n, k] += c
        assert np.array_equal(m, ref), (n, k)
    # c = 0 or B = 0 leave W exactly
    _, A, B = _merge_inputs(8, d_in, d_out, 4)
    assert np.array_equal(oracle.merge(W, A, B, 0.0, lib=lib), W.astype(np.float64))
    assert np.array_equal(oracle.merge(W, A, np.zeros_like(B), 3.0, lib=lib), W.astype(np.float64))


def pin_merge_unmerge_and_linearity(lib):
    W, A, B = _merge_inputs(11, 30, 20, 6)
    m1 = oracle.merge(W, A, B, 1.0, lib=lib)
    m2 = oracle.merge(W, A, B, 2.0, lib=lib)
    assert _rel_err(m2 - W, 2.0 * (m1 - W)) < 1e-12
    back = oracle.merge(m1.astype(np.float32), A, B, -1.0, lib=lib)
    # m1 rounded to float32 before unmerging: back to W within float32 rounding of m1
    assert np.max(np.abs(back - W)) <= 2.0 ** -24 * np.max(np.abs(m1)) * 2


def pin_fused_slices_are_block_diagonal(lib):
    # projections stacked into one W with their adapters' A stacked and B
    # block-diagonal give, through numpy fp64 products, the slices' outputs
    # side by side (the packing a fused adapter registration relies on)
    rng = np.random.default_rng(12)
    d_in, rows, ranks = 24, [10, 6, 6], [3, 3, 3]
    T = 9
    ids = sorted(rng.integers(-1, 3, size=T).tolist())
    scales = {a: float(rng.normal()) for a in range(3)}
    slices = [make_custom_case(400 + m, "f32", d_in, rows[m], ids, {a: ranks[m] for a in range(3)},
                               scales=scales) for m in range(3)]
    x = slices[0].x
    for c in slices[1:]:
        c.x = x
    y = np.concatenate([oracle.linear(c.x, c.W, _pool(c.adapters, c.capacity, d_in, c.d_out),
                                      c.seg_start, c.seg_adapter, c.seg_rank, c.seg_scale, None, 1,
                                      lib=lib) for c in slices], axis=1)
    Wcat = np.vstack([c.W for c in slices]).astype(np.float64)
    R = sum(ranks)
    ref = x.astype(np.float64) @ Wcat.T
    for t, a in enumerate(ids):
        if a < 0:
            continue
        Acat = np.vstack([c.adapters[a].A for c in slices]).astype(np.float64)
        Bbd = np.zeros((sum(rows), R))
        n0 = r0 = 0
        for m, c in enumerate(slices):
            Bbd[n0:n0 + rows[m], r0:r0 + ranks[m]] = c.adapters[a].B
            n0 += rows[m]
            r0 += ranks[m]
        ref[t] += np.float64(np.float32(scales[a])) * (Bbd @ (Acat @ x[t].astype(np.float64)))
    assert _rel_err(y, ref) < 1e-12


def pin_e4m3_decoder_matches_torch(lib):
    # every e4m3 code but the two NaNs, against torch's float8_e4m3fn
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy()
    finite = ~np.isnan(ref)
    assert int(np.sum(~finite)) == 2 and np.all(np.isnan(ours[~finite]))
    assert np.array_equal(ours[finite], ref[finite])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def pin_fp8w_layer_is_library_product(lib):
    # the FP8-weight layer: numpy fp64 products of the dequantized weight plus
    # the adapter term
    rng = np.random.default_rng(13)
    T, d_in, d_out = 6, 48, 20
    ids = sorted(rng.integers(-1, 3, size=T).tolist())
    c = make_custom_case(500, "f32", d_in, d_out, ids, {0: 4, 1: 2, 2: 8}, scales={0: 1.5, 1: -2.0, 2: 0.5})
    codes = rng.integers(0, 256, size=(d_out, d_in)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38          # no NaN codes
    w_scale = rng.uniform(0.5, 2.0, d_out).astype(np.float32)
    y = oracle.fp8w_case_linear(c, codes, w_scale, 1)
    Wd = w_scale[:, None].astype(np.float64) * oracle.e4m3_decode(codes).astype(np.float64)
    ref = c.x.astype(np.float64) @ Wd.T
    for t, a in enumerate(ids):
        if a >= 0:
            ad = c.adapters[a]
            ref[t] += np.float64(c.adapter_scale[a]) * (ad.B.astype(np.float64) @ (ad.A.astype(np.float64) @ c.x[t].astype(np.float64)))
    assert _rel_err(y, ref) < 1e-12


PINS = [pin_hand_example, pin_base_is_library_product, pin_lora_term_is_library_product,
        pin_merged_weights, pin_vanishing_terms, pin_one_hot_and_rank_one, pin_permutation,
        pin_linearity, pin_segmentation_exhaustive, pin_token_map, pin_merge_is_library_product,
        pin_merge_serves_like_adapter, pin_merge_closed_forms, pin_merge_unmerge_and_linearity,
        pin_fused_slices_are_block_diagonal, pin_e4m3_decoder_matches_torch,
        pin_fp8w_layer_is_library_product]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle.load())


# ---------------------------------------------------------------------------
# error semantics, row sampling, threads
# ---------------------------------------------------------------------------

def test_metadata_errors():
    lib = oracle.load()
    c = make_custom_case(51, "f32", 8, 8, [0, 0, 1, 1], {0: 2, 1: 3})
    pool = _pool(c.adapters, c.capacity, 8, 8)

    def run(ss, sa, sr, ti=None):
        return oracle.linear(c.x, c.W, pool, np.array(ss, np.int32), np.array(sa, np.int32),
                             np.array(sr, np.int32), np.ones(len(sa), np.float32),
                             None if ti is None else np.array(ti, np.int32), 1, lib=lib)

    run([0, 2, 4], [0, 1], [2, 3])
    with pytest.raises(oracle.OracleError) as e:
        run([0, 2, 3], [0, 1], [2, 3])          # seg_start[S] != T
    assert e.value.code == oracle.MLO_ERR_META
    with pytest.raises(oracle.OracleError) as e:
        run([0, 3, 2, 4], [0, 1, 1], [2, 3, 3])  # not monotone
    assert e.value.code == oracle.MLO_ERR_META
    with pytest.raises(oracle.OracleError) as e:
        run([0, 2, 4], [0, 5], [2, 3])          # id beyond capacity
    assert e.value.code == oracle.MLO_ERR_ADAPTER
    with pytest.raises(oracle.OracleError) as e:
        run([0, 2, 4], [0, 1], [2, 2])          # rank mismatch
    assert e.value.code == oracle.MLO_ERR_RANK
    with pytest.raises(oracle.OracleError) as e:
        run([0, 2, 4], [0, 1], [2, 3], ti=[0, 1, 1, 3])   # not a permutation
    assert e.value.code == oracle.MLO_ERR_META
    with pytest.raises(oracle.OracleError):
        oracle.segment([0, 3], 2, lib=lib)      # id beyond capacity


def test_row_subset_and_threads():
    c = make_case("tiny_f32")
    full1 = oracle.case_linear(c, 1, threads=1)
    full4 = oracle.case_linear(c, 1, threads=4)
    assert np.array_equal(full1, full4)
    rows = np.array([15, 0, 7, 7, 3], np.int32)
    sub = oracle.case_linear(c, 1, rows=rows)
    assert np.array_equal(sub, full1[rows])


def test_workload_generators():
    c1 = make_case("tiny_f32")
    assert c1.x.shape == (16, 256) and c1.W.shape == (256, 256)
    assert c1.seg_start.tolist() == [0, 4, 8, 12, 16] and c1.seg_scale.tolist() == [2.0] * 4
    c2 = make_case("decode_bf16")
    assert c2.x.shape == (64, 4096) and c2.n_seg <= 32
    assert np.array_equal(bf16_round(c2.W[:4]), c2.W[:4])           # bf16-representable
    assert np.all(np.diff(c2.token_adapter) >= 0)                   # grouped by the caller
    assert abs(float(np.std(c2.W[:256])) - 0.02) < 0.002
    c4 = make_case("hetero_bf16")
    assert not c4.sorted_input and c4.capacity == 512
    assert set(a.rank for a in c4.adapters.values()) == {8, 16, 32, 64}
    assert np.any(np.diff(c4.token_adapter) < 0)                    # really unsorted
    c5 = make_case("prefill_bf16", "k")
    assert c5.W.shape == (1024, 4096) and c5.n_seg == 64
    assert int(np.min(np.diff(c5.seg_start))) >= 1 and int(c5.seg_start[-1]) == 4096
