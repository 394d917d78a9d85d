#!/usr/bin/env python3
"""Benchmark of the multi-LoRA segmented linear layer on one MI355X.

One step = one call of the whole layer (segment lookup, shrink, base GEMM,
fused expand, store) over one synthetic batch. The default workload is the
decode-shaped batch: q_proj 4096->4096, 64 tokens (one per request), 32 rank-16
adapters assigned uniformly at random and grouped by the caller, bf16 with fp32
accumulation. Inputs are seeded synthetic data (no real model or adapters).

Timing: W untimed warm-up steps, then K steps back to back on one stream,
bracketed by synchronizations and HIP events recorded on that stream. Each
step uses a different buffer set (W, adapter pool, x, y, workspace), rotating
over >= 1 GiB so the 256 MB Infinity Cache cannot hold the working set: the
bytes come from HBM.

Reported (one JSON line on stdout):
  value      effective HBM GB/s of the LoRA-on pass = unique bytes / step time,
             unique bytes = W + touched adapters' A and B + x + y;
  tflops     effective TFLOP/s, flops = 2 T d_in d_out + sum_tokens 2 r (d_in + d_out);
  lora_off   the same shape with lora_on = 0 (the drafter pass), and the
             LoRA-on overhead t_on / t_off - 1 next to the byte-floor ratio;
  roofline   the layer kernel against MI355X's 8 TB/s HBM peak, with HBM
             traffic from rocprofv3 counters when they match the current
             kernel sources;
  cpu_baseline  the fp64 oracle on the host cores over the same batch.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("multi-LoRA linear eff. TFLOP/s + HBM GB/s (% roofline); "
          "LoRA-on vs LoRA-off overhead")
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "rank_adapter_gemm_segmented_amd", "csrc")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h")):
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(f.encode())
                h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="all",
                    help="all (default): the decode batch as the headline plus every other "
                         "configuration under 'configs'; or one workload",
                    choices=["all", "decode_bf16", "verify_bf16", "hetero_bf16", "prefill_bf16", "tiny_f32",
                             "merge_bf16", "fused_qkv_decode", "fused_gateup_verify",
                             "fused_qkv_prefill", "fused_gateup_prefill", "cycle_verify", "decode_fp8w",
                             "path_sweep"])
    ap.add_argument("--proj", default="q", help="prefill projection (also the merge shape)")
    ap.add_argument("--rank", type=int, default=64, help="adapter rank of the merge workload")
    ap.add_argument("--rotate-gib", type=float, default=1.0)
    ap.add_argument("--clock-warmup", type=float, default=0.5,
                    help="seconds of untimed sustained load before each workload's warm-up and "
                         "timed calls (the GPU's clocks ramp under load)")
    ap.add_argument("--graph", action="store_true",
                    help="time the K calls as HIP-graph replays (eager times are reported too)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time (wall x threads) of the oracle baseline")
    ap.add_argument("--profile", action="store_true",
                    help="short run for rocprofv3: a few steps plus one 256 MiB calibration copy")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="host only: turn the counter_collection.csv files of two --profile runs "
                         "(--pmc FETCH_SIZE, --pmc WRITE_SIZE) into the workload's entry of "
                         "profiles/traffic.json")
    ap.add_argument("--sweep-counters", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "MFMA_CSV"),
                    help="host only, path_sweep: turn the counter_collection.csv files of three "
                         "--profile runs (--pmc FETCH_SIZE, WRITE_SIZE, MfmaUtil) into per-call HBM "
                         "bytes and MFMA utilisation per (tokens, path, pass)")
    return ap.parse_args()


CALIB_BYTES = 256 << 20


def ingest_counters(workload: str, kernels, fetch_csv: str, write_csv: str) -> dict:
    """HBM traffic per layer call from two rocprofv3 --pmc runs of --profile.

    Each counter is scaled by what it reads for the calibration copy of
    CALIB_BYTES (the last __amd_rocclr_copyBuffer dispatch of the run: it
    reads and writes CALIB_BYTES). The layer's kernels are averaged over their LoRA-on
    dispatches and summed."""
    import csv

    def per_kernel(path):   # values per kernel name, in dispatch order
        rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"]))
        vals = {}
        for r in rows:
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    out = {"kernel_source_hash": kernel_source_hash(), "calibration_bytes": CALIB_BYTES}
    total = 0.0
    for key, path in (("fetch", fetch_csv), ("write", write_csv)):
        vals = per_kernel(path)
        # the calibration copy is the run's last device copy
        calib = vals.get("__amd_rocclr_copyBuffer", [0.0])[-1]
        if calib <= 0:
            raise SystemExit(f"{path}: no calibration copy found")
        factor = CALIB_BYTES / (calib * 1024.0)
        kib = {}
        for k in kernels:
            pat = re.compile(rf"::{k}[<(]")
            hits = [v for n, v in vals.items() if pat.search(n)]
            if not hits:
                raise SystemExit(f"{path}: kernel {k} not found")
            flat = [x for h in hits for x in h]
            kib[k] = sum(flat) / len(flat)
        out[f"{key}_kib_per_dispatch"] = {k: round(v, 1) for k, v in kib.items()}
        out[f"{key}_scale"] = round(factor, 4)
        total += sum(kib.values()) * 1024.0 * factor
    out["bytes_per_step"] = int(round(total))
    allt = {}
    if os.path.exists(TRAFFIC_FILE):
        allt = json.load(open(TRAFFIC_FILE))
    allt[workload] = out
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(allt, fh, indent=1, sort_keys=True)
        fh.write("\n")
    return out


def graph_timed(step, n_sets: int, steps: int, warmup: int, offset: int = 0) -> float:
    """ms per step over exactly `steps` calls replayed from HIP graphs: one
    graph holds n_sets consecutive calls (one per buffer set), a second one
    the remainder. Launch costs on the host drop out; the GPU runs the
    kernels back to back. Warm-up calls run eagerly first (and on the
    capture's side stream, as capture wants)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(max(warmup, 1)):
            step(offset + i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # the replays go on from the set after the warm-up's last
    o = offset + max(warmup, 1)
    full, tail = steps // n_sets, steps % n_sets
    g_full, g_tail = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    if full:
        with torch.cuda.graph(g_full):
            for i in range(n_sets):
                step(o + i)
    if tail:
        with torch.cuda.graph(g_tail):
            for i in range(tail):
                step(o + i)
    if full:
        g_full.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(full):
        g_full.replay()
    if tail:
        g_tail.replay()
    e1.record(stream)
    e1.synchronize()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def counted_traffic(workload: str):
    """HBM bytes per call from profiles/traffic.json, or None when the entry
    is missing or was taken on other kernel sources."""
    try:
        ent = json.load(open(TRAFFIC_FILE)).get(workload, {})
    except (ValueError, OSError):
        return None
    return ent.get("bytes_per_step") if ent.get("kernel_source_hash") == kernel_source_hash() else None


def shrink_split(case) -> int:
    """d_in chunks of the bf16 shrink, as the library picks them (api.hip and
    choose_shrink_split_bf16): one chunk for short segments of rank <= 16 and
    wherever the short-segment shrink runs, else enough chunks to fill the
    GPU."""
    T = case.n_tokens
    nseg = case.n_seg if case.sorted_input else T   # the host's segment bound
    if T <= 16 * nseg and case.max_rank <= 16:
        return 1
    if short_shrink(case):
        return 1
    groups = (case.d_in + 511) // 512
    # items: (block of 16 NRB positions, group of 16 NCB rank rows) per
    # segment; NRB = NCB = 4 for a mean segment longer than 16, else 1
    long_segs = T > 16 * nseg
    pb, ncb = (64, 4) if long_segs else (16, 1)
    items = (min(nseg, 16384) + (T + pb - 1) // pb) * max(1, (case.max_rank + 16 * ncb - 1) // (16 * ncb))
    ks = 1
    while ks < 4 and ks * 2 <= groups and items * ks < 1024:
        ks *= 2
    return ks


def short_shrink(case) -> bool:
    """The vector-ALU shrink for short segments (kernels_gemm.hip,
    shrink_short): host-known segments, at most two positions per segment on
    average, ranks <= 32, unless MLORA_FORCE_SHRINK=mfma."""
    return (case.dtype == "bf16" and case.sorted_input and case.n_tokens <= 2 * case.n_seg and
            case.max_rank <= 32 and os.environ.get("MLORA_FORCE_SHRINK") != "mfma")


def dense_expand(case):
    """Whether the library adds the adapter term as a dense fp32 tile
    (k_expand_delta) rather than in the GEMM epilogue (api.hip,
    use_dense_expand): plain bf16 pools of largest rank 32..64, d_out a
    multiple of 8, at most 512 tokens and 16 MiB of term; MLORA_EXPAND=dense
    or mfma forces either where eligible."""
    T, d_out, r = case.n_tokens, case.d_out, case.max_rank
    ok = (case.dtype == "bf16" and r <= 64 and d_out % 8 == 0 and T <= 512 and T * d_out * 4 <= (16 << 20))
    mode = os.environ.get("MLORA_EXPAND")
    if not ok or mode == "mfma":
        return False
    return mode == "dense" or r >= 32


def layer_kernels(case):
    """Kernels of one LoRA-on layer call, run back to back on one stream: the
    split-K stream + finish pair for T <= 64 in bf16 (T < 48 on layers of
    8192 outputs or more); above that segment build
    (unsorted input), the shrink, the v fold (only when the shrink splits d_in),
    the dense adapter term (dense_expand) and the tiled GEMM with the term
    added or expanded in its epilogue; shrink + GEMM for fp32."""
    wide = case.n_tokens >= 48 and case.d_out >= 8192    # api.hip sends these to the GEMM
    if case.dtype == "bf16" and case.n_tokens <= 64 and not wide:
        return ["k_stream_bf16", "k_finish_bf16"]
    if case.dtype == "bf16":
        # the vector-ALU shrink on host-known short segments
        short = short_shrink(case)
        return ((["k_build_segments"] if not case.sorted_input else []) +
                (["k_shrink_short"] if short else ["k_shrink2"]) +
                (["k_vfinal"] if shrink_split(case) > 1 and not dense_expand(case) else []) +
                (["k_expand_delta"] if dense_expand(case) else []) + ["k_gemm2"])
    return ["k_shrink_f32", "k_gemm_f32"]


def bench_merge(args):
    """Merge of one adapter into a base weight, W_out = W_in + scale * B A
    (out of place), for one decoder-layer projection shape. Algorithmic bytes:
    W read + W_out written + A and B read once."""
    import numpy as np
    import torch
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import rank_adapter_gemm_segmented_amd as ml
    from gpu_util import to_dev
    from mlora_inputs import PREFILL_SHAPES, make_merge_inputs

    d_in, d_out = PREFILL_SHAPES[args.proj]
    r = args.rank
    name = f"merge_bf16_{args.proj}_r{r}"
    if args.ingest_counters:
        print(json.dumps({name: ingest_counters(name, ["k_merge_bf16"], *args.ingest_counters)}))
        return
    torch.cuda.set_device(0)
    W, ad = make_merge_inputs(2000 + r, "bf16", d_in, d_out, r)
    W0 = to_dev(W, "bf16")
    pool0 = ml.Pool(d_in, d_out, torch.bfloat16, r, 1)
    pool0.register(0, to_dev(ad.A, "bf16"), to_dev(ad.B, "bf16"))
    es = 2
    alg = 2 * d_out * d_in * es + r * (d_in + d_out) * es
    set_bytes = 2 * W0.numel() * es + pool0.arena.numel()
    n_sets = 2 if args.profile else max(2, int(np.ceil(args.rotate_gib * (1 << 30) / set_bytes)))
    sets = []
    for i in range(n_sets):
        if i == 0:
            Wi, pool = W0, pool0
        else:
            Wi = W0.clone()
            pool = ml.Pool(d_in, d_out, torch.bfloat16, r, 1)
            pool.register(0, to_dev(ad.A, "bf16"), to_dev(ad.B, "bf16"))
        sets.append((Wi, torch.empty_like(Wi), pool))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def run(steps, warmup):
        for i in range(warmup):
            Wi, Wo, pool = sets[i % n_sets]
            ml.merge_adapter(Wi, pool, 0, 2.0, out=Wo)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(warmup, warmup + steps):   # on from the warm-up's last set
            Wi, Wo, pool = sets[i % n_sets]
            ml.merge_adapter(Wi, pool, 0, 2.0, out=Wo)
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / steps

    if args.profile:
        run(5, 2)
        print(f"[bench] {name}: 7 merge calls done", file=sys.stderr, flush=True)
        n = 256 << 20
        src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy of {n} bytes done", file=sys.stderr, flush=True)
        return
    ms = run(args.steps, args.warmup)
    gbs = alg / (ms * 1e-3) / 1e9
    # reference: a plain device copy of W over the same buffer sets (read + write, no dW)
    for i in range(args.warmup):
        sets[i % n_sets][1].copy_(sets[i % n_sets][0])
    torch.cuda.synchronize()
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for i in range(args.warmup, args.warmup + args.steps):
        sets[i % n_sets][1].copy_(sets[i % n_sets][0])
    c1.record(stream)
    c1.synchronize()
    ms_copy = c0.elapsed_time(c1) / args.steps
    copy_bytes = 2 * d_out * d_in * es
    print(f"[bench] {name}: {ms * 1e3:.2f} us/call, {n_sets} buffer sets of {set_bytes / 2**20:.1f} MiB",
          file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = max(1, min(len(os.sched_getaffinity(0)), 16))
        rows = max(1, min(d_out, int(2e9 / (d_in * r))))   # a bounded prefix of W's rows
        reps, t_total = 0, 0.0
        while t_total * threads < args.cpu_seconds or reps == 0:
            t0 = time.perf_counter()
            oracle.merge(W[:rows], ad.A, ad.B[:rows], 2.0, threads=threads)
            t_total += time.perf_counter() - t0
            reps += 1
            if reps >= 50:
                break
        t_full = t_total / reps * (d_out / rows)
        cpu = {"value": round(alg / t_full / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "sample": f"{rows} of {d_out} rows of W, fp64, {reps} repetitions, {t_total:.1f} s wall; "
                         f"value scaled to the whole weight",
               "seconds_per_merge": round(t_full, 4)}
    out = {
        "metric": "adapter merge W + scale*B*A, effective HBM GB/s (% roofline)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded Gaussian weight and adapter)",
        "config": {"workload": name, "d_in": d_in, "d_out": d_out, "rank": r, "buffer_sets": n_sets,
                   "algorithmic_bytes": alg},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": counted_traffic(name),
                     "algorithmic_bytes": alg,
                     "us_per_call": round(ms * 1e3, 3), "kernels": ["k_merge_bf16"],
                     "kernel_source_hash": kernel_source_hash()},
        "copy_reference": {"us_per_call": round(ms_copy * 1e3, 3),
                           "gbs": round(copy_bytes / (ms_copy * 1e-3) / 1e9, 1),
                           "what": "torch copy_ of W into W_out over the same buffer sets"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_fused(args):
    """Stacked projections (q|k|v or gate|up) in one fused call against the
    same projections as separate calls, both LoRA-on, over rotating buffer
    sets. Algorithmic bytes: stacked W + touched adapters' A_m and B_m of
    every projection + x + y (the zero blocks of the block-diagonal B are not
    counted)."""
    import numpy as np
    import torch
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import rank_adapter_gemm_segmented_amd as ml
    from gpu_util import f32, i32, to_dev
    from mlora_inputs import make_fused_case

    torch.cuda.set_device(0)
    slices = make_fused_case(args.workload)
    c0 = slices[0]
    n = len(slices)
    T, d_in = c0.n_tokens, c0.d_in
    d_out = sum(c.d_out for c in slices)
    R = sum(c.max_rank for c in slices)
    es = 2
    touched = c0.touched_adapters()
    alg = (d_out * d_in + T * d_in + T * d_out) * es + sum(
        (c.adapters[a].rank * d_in + c.d_out * c.adapters[a].rank) * es for c in slices for a in touched)
    ranks = np.array([c0.adapters[int(a)].rank if a >= 0 else 0 for a in c0.token_adapter])
    flops = 2.0 * T * d_in * d_out + float(np.sum(2.0 * ranks * (n * d_in + d_out)))
    x0 = to_dev(c0.x, "bf16")
    Wf0 = to_dev(np.vstack([c.W for c in slices]), "bf16")
    meta_f = (i32(c0.seg_start), i32(c0.seg_adapter), i32(np.where(c0.seg_adapter >= 0, c0.seg_rank * n, 0)),
              f32(c0.seg_scale))
    meta_s = (i32(c0.seg_start), i32(c0.seg_adapter), i32(c0.seg_rank), f32(c0.seg_scale))
    dev_ad = {a: [(to_dev(c.adapters[a].A, "bf16"), to_dev(c.adapters[a].B, "bf16")) for c in slices]
              for a in sorted(c0.adapters)}

    def fused_set(first):
        W = Wf0 if first else Wf0.clone()
        pool = ml.Pool(d_in, d_out, torch.bfloat16, R, c0.capacity)
        for a, sl in dev_ad.items():
            pool.register_fused(a, sl)
        return W, pool, torch.empty((T, d_out), dtype=torch.bfloat16, device="cuda"), pool.workspace(T)

    def sep_set():
        out = []
        for m, c in enumerate(slices):
            pool = ml.Pool(d_in, c.d_out, torch.bfloat16, c.max_rank, c.capacity)
            for a, sl in dev_ad.items():
                pool.register(a, *sl[m])
            out.append((to_dev(c.W, "bf16"), pool, torch.empty((T, c.d_out), dtype=torch.bfloat16,
                                                                device="cuda"), pool.workspace(T)))
        return out

    set_bytes = 2 * Wf0.numel() * es
    n_sets = max(2, int(np.ceil(args.rotate_gib * (1 << 30) / set_bytes)))
    fsets = [fused_set(i == 0) for i in range(n_sets)]
    ssets = [sep_set() for _ in range(n_sets)]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step_fused(i):
        W, pool, y, ws = fsets[i % n_sets]
        ml.linear(x0, W, pool, *meta_f, lora_on=1, out=y, workspace=ws)

    def step_sep(i):
        for W, pool, y, ws in ssets[i % n_sets]:
            ml.linear(x0, W, pool, *meta_s, lora_on=1, out=y, workspace=ws)

    def timed(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.warmup, args.warmup + args.steps):   # on from the warm-up's last set
            fn(i)
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms_f = timed(step_fused)
    ms_s = timed(step_sep)
    gbs = alg / (ms_f * 1e-3) / 1e9
    print(f"[bench] {args.workload}: fused {ms_f * 1e3:.2f} us/call, separate {ms_s * 1e3:.2f} us "
          f"({n} calls), {n_sets} buffer sets", file=sys.stderr, flush=True)
    big = c0.n_tokens > 256
    roof = ({"bound": "mfma", "achieved": round(flops / (ms_f * 1e-3) / 1e12, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
             "unit": "TFLOP/s", "frac": round(flops / (ms_f * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
            if big else
            {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(gbs / HBM_PEAK_GBS, 4)})
    roof.update({"traffic": None, "algorithmic_bytes": alg, "us_per_call": round(ms_f * 1e3, 3),
                 "kernel_source_hash": kernel_source_hash()})
    out = {
        "metric": "fused multi-projection multi-LoRA linear, effective GB/s and TFLOP/s; fused vs separate calls",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_f, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded Gaussian weights, adapters and activations)",
        "config": {"workload": args.workload, "tokens": T, "d_in": d_in,
                   "d_out_slices": [c.d_out for c in slices], "rank_per_slice": c0.max_rank,
                   "adapters_touched": len(touched), "segments": c0.n_seg, "buffer_sets": n_sets},
        "tflops": round(flops / (ms_f * 1e-3) / 1e12, 2),
        "separate_calls": {"ms_per_step": round(ms_s, 6), "calls": n,
                           "gbs": round(alg / (ms_s * 1e-3) / 1e9, 1)},
        "fused_speedup": round(ms_s / ms_f, 4),
        "roofline": roof,
    }
    print(json.dumps(out), flush=True)


def bench_cycle(args):
    """The InvisibleLoRA cycle at one gate/up layer (4096->14336, one rank-16
    adapter per request, scale 2): LoRA-on and LoRA-off passes over b tokens
    (one per request) and a LoRA-on pass over 2 b tokens (last committed token
    + draft per request), for several batch sizes b, with the per-token
    estimate and gate decision of rank_adapter_gemm_segmented_amd.cycle at the
    pages' median acceptance rates."""
    import numpy as np
    import torch
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import rank_adapter_gemm_segmented_amd as ml
    from rank_adapter_gemm_segmented_amd.cycle import break_even_alpha, cycle_estimate
    from gpu_util import f32, i32, to_dev
    from mlora_inputs import make_custom_case

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    b_max, d_in, d_out, r = 128, 4096, 14336, 16
    case = make_custom_case(4000, "bf16", d_in, d_out, np.repeat(np.arange(b_max), 2),
                            {a: r for a in range(b_max)}, scales={a: 2.0 for a in range(b_max)})
    W0 = to_dev(case.W, "bf16")
    x0 = to_dev(case.x, "bf16")
    dev_ad = [(to_dev(case.adapters[a].A, "bf16"), to_dev(case.adapters[a].B, "bf16")) for a in range(b_max)]
    set_bytes = W0.numel() * 2 + b_max * r * (d_in + d_out) * 2
    n_sets = max(2, int(np.ceil(args.rotate_gib * (1 << 30) / set_bytes)))
    sets = []
    for i in range(n_sets):
        pool = ml.Pool(d_in, d_out, torch.bfloat16, r, b_max)
        for a, (A, B) in enumerate(dev_ad):
            pool.register(a, A, B)
        sets.append((W0 if i == 0 else W0.clone(), pool, pool.workspace(2 * b_max),
                     torch.empty((2 * b_max, d_out), dtype=torch.bfloat16, device="cuda")))
    torch.cuda.synchronize()

    def meta(b, per_req):
        return (i32(np.arange(b + 1) * per_req), i32(np.arange(b)), i32(np.full(b, r)), f32(np.full(b, 2.0)))

    def timed(b, per_req, lora_on):
        T = b * per_req
        x = x0[:T]
        m = meta(b, per_req)

        def step(i):
            W, pool, ws, y = sets[i % n_sets]
            ml.linear(x, W, pool, *m, lora_on=lora_on, out=y[:T], workspace=ws)
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.warmup, args.warmup + args.steps):   # on from the warm-up's last set
            step(i)
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / args.steps * 1e3   # us per call

    rows = []
    for b in (16, 32, 64, 128):
        t_on_b, t_off_b, t_on_2b = timed(b, 1, 1), timed(b, 1, 0), timed(b, 2, 1)
        ent = {"requests": b, "t_on_b_us": round(t_on_b, 2), "t_off_b_us": round(t_off_b, 2),
               "t_on_2b_us": round(t_on_2b, 2),
               "break_even_alpha": round(break_even_alpha(t_on_b, t_off_b, t_on_2b), 4)}
        for alpha in (0.92, 0.97):
            est = cycle_estimate(t_on_b, t_off_b, t_on_2b, alpha)
            ent[f"alpha_{alpha}"] = {"per_token_us": round(est.per_token_cycle, 2),
                                    "speedup": round(est.speedup, 4), "draft": est.draft}
        rows.append(ent)
        print(f"[bench] cycle b={b}: on {t_on_b:.1f} off {t_off_b:.1f} on(2b) {t_on_2b:.1f} us, "
              f"break-even alpha {ent['break_even_alpha']:.3f}", file=sys.stderr, flush=True)
    last = rows[-1]
    out = {
        "metric": "InvisibleLoRA cycle at one layer: time per committed token, drafting vs plain LoRA-on decoding",
        "value": last["alpha_0.97"]["speedup"], "unit": "x (plain / cycle, alpha 0.97, 128 requests)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Gaussian weights, adapters and activations)",
        "config": {"workload": "cycle_verify", "d_in": d_in, "d_out": d_out, "rank": r,
                   "adapters": "one per request", "buffer_sets": n_sets},
        "batches": rows,
    }
    print(json.dumps(out), flush=True)


SWEEP_SHAPES = ((4096, 4096, (1, 2, 4, 8, 16, 32, 64, 128)),   # the decode batch's q projection
                (4096, 14336, (16, 32, 48, 64, 128)))            # a wide gate/up projection
SWEEP_PROFILE_CALLS = 3


def sweep_plan():
    """(d_out, tokens, path, lora_on) in the order the sweep runs them: the
    split-K decode pair and the GEMV-style stream up to 64 tokens, the tiled
    GEMM at every count."""
    plan = []
    for d_in, d_out, tokens in SWEEP_SHAPES:
        for T in tokens:
            for path in ("decode", "gemv", "gemm"):
                if path != "gemm" and T > 64:
                    continue
                for lora_on in (1, 0):
                    plan.append((d_out, T, path, lora_on))
    return plan


def sweep_case(d_in, d_out, T):
    """The decode recipe at T tokens: d_in -> d_out, 32 rank-16 adapters
    (scale 32 / 16), each token's adapter drawn uniformly at random and the
    tokens grouped by adapter (sorted segments)."""
    import numpy as np
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from mlora_inputs import make_custom_case
    rng = np.random.default_rng(5000 + T)
    tok = np.sort(rng.integers(0, 32, size=T).astype(np.int32), kind="stable")
    return make_custom_case(5000 + T, "bf16", d_in, d_out, tok, {a: 16 for a in range(32)},
                            scales={a: 2.0 for a in range(32)})


def bench_path_sweep(args):
    """Token-count sweep of the bf16 paths (decode pair, GEMV-style stream,
    tiled GEMM), each forced in turn with MLORA_FORCE_PATH, LoRA-on and
    LoRA-off, on the decode recipe at two layer shapes (SWEEP_SHAPES). With
    --profile: a few calls per (shape, tokens, path, pass) in sweep_plan order
    and one calibration copy, for rocprofv3 counter runs (--sweep-counters
    reads them back)."""
    import numpy as np
    import torch
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import rank_adapter_gemm_segmented_amd as ml
    from gpu_util import f32, i32, to_dev

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    prev = os.environ.get("MLORA_FORCE_PATH")
    rows = []
    try:
        for d_in, d_out, tokens in SWEEP_SHAPES:
            T_max = max(tokens)
            base = sweep_case(d_in, d_out, T_max)
            W0 = to_dev(base.W, "bf16")
            x0 = to_dev(base.x, "bf16")
            set_bytes = W0.numel() * 2 + 32 * 16 * (d_in + d_out) * 2
            n_sets = 2 if args.profile else max(2, int(np.ceil(args.rotate_gib * (1 << 30) / set_bytes)))
            sets = []
            for i in range(n_sets):
                pool = ml.Pool(d_in, d_out, torch.bfloat16, 16, 32)
                for a in range(32):
                    pool.register(a, to_dev(base.adapters[a].A, "bf16"), to_dev(base.adapters[a].B, "bf16"))
                sets.append((W0 if i == 0 else W0.clone(), pool, pool.workspace(T_max),
                             torch.empty((T_max, d_out), dtype=torch.bfloat16, device="cuda")))
            metas = {}
            for T in tokens:
                c = sweep_case(d_in, d_out, T)
                metas[T] = (i32(c.seg_start), i32(c.seg_adapter), i32(c.seg_rank), f32(c.seg_scale), int(c.n_seg))
            torch.cuda.synchronize()

            def step(i, T, lora_on):
                W, pool, ws, y = sets[i % n_sets]
                ss, sa, sr, sc, _ = metas[T]
                ml.linear(x0[:T], W, pool, ss, sa, sr, sc, lora_on=lora_on, out=y[:T], workspace=ws)

            for dout_p, T, path, lora_on in sweep_plan():
                if dout_p != d_out:
                    continue
                os.environ["MLORA_FORCE_PATH"] = path
                if args.profile:
                    for i in range(SWEEP_PROFILE_CALLS):
                        step(i, T, lora_on)
                    torch.cuda.synchronize()
                    continue
                for i in range(args.warmup):
                    step(i, T, lora_on)
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for i in range(args.warmup, args.warmup + args.steps):
                    step(i, T, lora_on)
                e1.record(stream)
                e1.synchronize()
                us = e0.elapsed_time(e1) / args.steps * 1e3
                rows.append({"d_in": d_in, "d_out": d_out, "tokens": T, "path": path, "lora_on": lora_on,
                             "us": round(us, 2), "segments": metas[T][4]})
                print(f"[bench] sweep {d_in}->{d_out} T={T} {path} lora_on={lora_on}: {us:.2f} us",
                      file=sys.stderr, flush=True)
            del sets, W0, x0
            torch.cuda.empty_cache()
    finally:
        if prev is None:
            os.environ.pop("MLORA_FORCE_PATH", None)
        else:
            os.environ["MLORA_FORCE_PATH"] = prev
    if args.profile:
        n = CALIB_BYTES
        src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] path sweep: {len(sweep_plan())} x {SWEEP_PROFILE_CALLS} calls, then a "
              f"calibration copy of {n} bytes", file=sys.stderr, flush=True)
        return
    print(json.dumps({
        "metric": "time per layer call by path and token count (decode recipe, two layer shapes)",
        "unit": "us", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": False, "dtype": "bf16",
        "data": "synthetic (seeded Gaussian weights, adapters and activations)",
        "config": {"workload": "path_sweep", "shapes": [[a, b] for a, b, _ in SWEEP_SHAPES],
                   "adapters": 32, "rank": 16},
        "rows": rows}), flush=True)


def ingest_sweep_counters(fetch_csv: str, write_csv: str, mfma_csv: str) -> list:
    """Per (shape, tokens, path, pass): HBM bytes per call (FETCH_SIZE and WRITE_SIZE
    scaled by the calibration copy, as ingest_counters does) and the
    dispatch-weighted MfmaUtil of the call's kernels, from three --pmc runs
    of `--workload path_sweep --profile`. The layer's dispatches are the
    non-copy dispatches of each run, in sweep_plan order."""
    import csv

    def dispatches(path):
        rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"]))
        out = []
        for r in rows:   # one row per (dispatch, counter); keep the first
            if out and out[-1][0] == int(r["Dispatch_Id"]):
                continue
            out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
        return out

    res = {}
    for key, path in (("fetch", fetch_csv), ("write", write_csv), ("mfma", mfma_csv)):
        ds = dispatches(path)
        copies = [d for d in ds if "rocclr" in d[1]]
        layer = [d for d in ds if "rocclr" not in d[1] and "k_set_slot_rank" not in d[1]
                 and "k_fill_u32" not in d[1]]
        factor = 1.0
        if key != "mfma":
            calib = copies[-1][2] if copies else 0.0
            if calib <= 0:
                raise SystemExit(f"{path}: no calibration copy found")
            factor = CALIB_BYTES / (calib * 1024.0)
        res[key] = (layer, factor)
    # a call's dispatches vary by path (decode pair, shrink + stream or GEMM,
    # an optional fold): walk each run's layer dispatches call by call
    out = []
    pos = {"fetch": 0, "write": 0, "mfma": 0}
    for d_out, T, path, lora_on in sweep_plan():
        ent = {"d_out": d_out, "tokens": T, "path": path, "lora_on": lora_on}
        for key in ("fetch", "write", "mfma"):
            layer, factor = res[key]
            vals, names = [], []
            for c in range(SWEEP_PROFILE_CALLS):
                # one call = the dispatches up to and including its last kernel
                call = []
                while True:
                    d = layer[pos[key]]
                    pos[key] += 1
                    call.append(d)
                    if _call_ends(d[1]):
                        break
                vals.append(call)
                names = [re.search(r"k_\w+(<[^>]*>)?", d[1]).group(0) for d in call]
            if key == "mfma":
                ent["kernels"] = names
                ent["mfma_util_pct"] = [round(sum(c[j][2] for c in vals) / len(vals), 2) for j in range(len(names))]
            else:
                tot = sum(sum(d[2] for d in c) for c in vals) / len(vals)
                ent[f"{key}_mb"] = round(tot * 1024.0 * factor / 1e6, 3)
        out.append(ent)
    return out


def _call_ends(kernel_name: str) -> bool:
    """The last kernel of a layer call on each bf16 path."""
    return any(k in kernel_name for k in ("k_finish_bf16", "k_gemv_bf16", "k_gemm2"))


def bench_fp8w(args):
    """The decode batch with the base weight stored as FP8 e4m3 (per-row
    float32 scales) and bf16 adapters, LoRA-on and LoRA-off, over rotating
    buffer sets. Algorithmic bytes: W codes + row scales + touched adapters'
    A and B + x + y."""
    import numpy as np
    import torch
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import rank_adapter_gemm_segmented_amd as ml
    from gpu_util import f32, i32, to_dev
    from mlora_inputs import make_fp8w_case

    case, codes, wsc = make_fp8w_case("decode_bf16")
    T, d_in, d_out = case.n_tokens, case.d_in, case.d_out
    touched = case.touched_adapters()
    lora_bytes = sum((case.adapters[a].rank * d_in + d_out * case.adapters[a].rank) * 2 for a in touched)
    base_bytes = d_out * d_in + d_out * 4 + (T * d_in + T * d_out) * 2
    bytes_on, bytes_off = base_bytes + lora_bytes, base_bytes
    if args.ingest_counters:
        print(json.dumps({"decode_fp8w": ingest_counters("decode_fp8w", ["k_stream_bf16", "k_finish_bf16"],
                                                          *args.ingest_counters)}))
        return
    torch.cuda.set_device(0)
    W80 = torch.from_numpy(codes).cuda()
    s0 = f32(wsc)
    x0 = to_dev(case.x, "bf16")
    pool0 = ml.Pool(d_in, d_out, torch.bfloat16, case.max_rank, case.capacity)
    for aid in sorted(case.adapters):
        ad = case.adapters[aid]
        pool0.register(aid, to_dev(ad.A, "bf16"), to_dev(ad.B, "bf16"))
    set_bytes = W80.numel() + pool0.arena.numel()
    n_sets = 2 if args.profile else max(2, int(np.ceil(args.rotate_gib * (1 << 30) / set_bytes)))
    sets = []
    for i in range(n_sets):
        if i == 0:
            W8, pool = W80, pool0
        else:
            W8 = W80.clone()
            pool = ml.Pool(d_in, d_out, torch.bfloat16, case.max_rank, case.capacity)
            pool.arena.copy_(pool0.arena)
        sets.append((W8, s0.clone(), pool, torch.empty((T, d_out), dtype=torch.bfloat16, device="cuda"),
                     pool.workspace(T)))
    meta = (i32(case.seg_start), i32(case.seg_adapter), i32(case.seg_rank), f32(case.seg_scale))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def timed(lora_on, steps, warmup):
        def step(i):
            W8, sc, pool, y, ws = sets[i % n_sets]
            ml.linear_fp8w(x0, W8, sc, pool, *meta, lora_on=lora_on, out=y, workspace=ws)
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(warmup, warmup + steps):   # on from the warm-up's last set
            step(i)
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / steps

    if args.profile:
        timed(1, 5, 2)
        print("[bench] decode_fp8w: 7 lora_on calls done", file=sys.stderr, flush=True)
        n = 256 << 20
        src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy of {n} bytes done", file=sys.stderr, flush=True)
        return
    ms_on_eager = timed(1, args.steps, args.warmup)
    ms_off_eager = timed(0, args.steps, args.warmup)
    ms_on, ms_off = ms_on_eager, ms_off_eager
    if args.graph:
        def gstep(lora_on):
            def f(i):
                W8, sc, pool, y, ws = sets[i % n_sets]
                ml.linear_fp8w(x0, W8, sc, pool, *meta, lora_on=lora_on, out=y, workspace=ws)
            return f
        ms_on = graph_timed(gstep(1), n_sets, args.steps, args.warmup)
        ms_off = graph_timed(gstep(0), n_sets, args.steps, args.warmup)
    print(f"[bench] decode_fp8w: lora_on {ms_on * 1e3:.2f} us/step, lora_off {ms_off * 1e3:.2f} us/step "
          f"({'graph replay' if args.graph else 'eager'}; eager {ms_on_eager * 1e3:.2f} / {ms_off_eager * 1e3:.2f}), "
          f"{n_sets} buffer sets", file=sys.stderr, flush=True)
    gbs_on = bytes_on / (ms_on * 1e-3) / 1e9
    out = {
        "metric": "multi-LoRA linear with an FP8 base weight, eff. HBM GB/s (% roofline); LoRA-on vs LoRA-off",
        "value": round(gbs_on, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_on, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8 e4m3 W, bf16 x/adapters/y, fp32 accumulate",
        "data": "synthetic (seeded Gaussian weights, adapters and activations; W quantized per row)",
        "config": {"workload": "decode_fp8w", "tokens": T, "d_in": d_in, "d_out": d_out,
                   "adapters_touched": len(touched), "buffer_sets": n_sets,
                   "unique_bytes_lora_on": bytes_on, "unique_bytes_lora_off": bytes_off},
        "lora_off": {"ms_per_step": round(ms_off, 6), "gbs": round(bytes_off / (ms_off * 1e-3) / 1e9, 1)},
        "lora_on_overhead": round(ms_on / ms_off - 1.0, 4),
        "timing": "K calls replayed from HIP graphs" if args.graph else "K eager calls",
        "eager": {"ms_per_step_lora_on": round(ms_on_eager, 6), "ms_per_step_lora_off": round(ms_off_eager, 6)},
        "roofline": {"bound": "hbm", "achieved": round(gbs_on, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs_on / HBM_PEAK_GBS, 4), "traffic": counted_traffic("decode_fp8w"),
                     "algorithmic_bytes": bytes_on, "us_per_call": round(ms_on * 1e3, 3),
                     "kernels": ["k_stream_bf16", "k_finish_bf16"], "kernel_source_hash": kernel_source_hash()},
    }
    print(json.dumps(out), flush=True)


def cpu_threads() -> int:
    """Host threads the oracle baseline runs on: every CPU in this process's
    affinity mask."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return max(1, os.cpu_count() or 1)


def case_work(case):
    """Algorithmic bytes and flops of one layer call, LoRA-on and LoRA-off:
    bytes = W + touched adapters' A and B + x + y; flops = 2 T d_in d_out +
    sum over tokens of 2 r (d_in + d_out)."""
    import numpy as np
    T, d_in, d_out = case.n_tokens, case.d_in, case.d_out
    es = 2 if case.dtype == "bf16" else 4
    touched = case.touched_adapters()
    lora_bytes = sum((case.adapters[a].rank * d_in + d_out * case.adapters[a].rank) * es for a in touched)
    base_bytes = (d_out * d_in + T * d_in + T * d_out) * es
    ranks = np.array([case.adapters[int(a)].rank if a >= 0 else 0 for a in case.token_adapter])
    flops_off = 2.0 * T * d_in * d_out
    flops_on = flops_off + float(np.sum(2.0 * ranks * (d_in + d_out)))
    return base_bytes + lora_bytes, base_bytes, flops_on, flops_off


def measure_layer(case, args, label: str):
    """LoRA-on and LoRA-off time of one workload's layer call (ms per call).

    Every call takes the next buffer set (W, adapter pool, x, y, workspace)
    of a rotation, counting on from the warm-up calls, so no timed call
    reads a set touched fewer than n_sets - 1 calls earlier. The rotation is
    sized by the bytes a LoRA-off call touches (W, x, y), not by whole sets:
    a set's adapter pool can dwarf its W (671 MB against 52 MB on the
    heterogeneous batch), and a LoRA-off call never reads it, so sizing by
    set bytes left that pass's W resident in the 256 MB Infinity Cache. With
    >= args.rotate_gib GiB of W, x and y in rotation the bytes come from HBM.
    Returns a dict of times and the set geometry."""
    import numpy as np
    import torch
    import rank_adapter_gemm_segmented_amd as ml
    from gpu_util import f32, i32, to_dev

    dev = torch.device("cuda:0")
    T, d_in, d_out = case.n_tokens, case.d_in, case.d_out
    es = 2 if case.dtype == "bf16" else 4
    tdt = torch.bfloat16 if case.dtype == "bf16" else torch.float32
    W0 = to_dev(case.W, case.dtype)
    x0 = to_dev(case.x, case.dtype)
    pool0 = ml.Pool(d_in, d_out, tdt, case.max_rank, case.capacity)
    for aid in sorted(case.adapters):
        ad = case.adapters[aid]
        pool0.register(aid, to_dev(ad.A, case.dtype), to_dev(ad.B, case.dtype))
    set_bytes = W0.numel() * es + pool0.arena.numel() + x0.numel() * es + T * d_out * es
    touch_bytes = (W0.numel() + x0.numel() + T * d_out) * es
    n_sets = 2 if args.profile else min(4096, max(3, int(np.ceil(args.rotate_gib * (1 << 30) / touch_bytes))))
    sets = []
    for i in range(n_sets):
        if i == 0:
            W, x, pool = W0, x0, pool0
        else:
            W, x = W0.clone(), x0.clone()
            pool = ml.Pool(d_in, d_out, tdt, case.max_rank, case.capacity)
            pool.arena.copy_(pool0.arena)
        sets.append((W, x, pool, torch.empty((T, d_out), dtype=tdt, device=dev), pool.workspace(T)))
    if case.sorted_input:
        meta = (i32(case.seg_start), i32(case.seg_adapter), i32(case.seg_rank), f32(case.seg_scale))
    else:
        tok, sc = i32(case.token_adapter), f32(case.adapter_scale)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    rot = [0]   # rotation position: the next call's buffer set

    def step(i, lora_on):
        W, x, pool, y, ws = sets[i % n_sets]
        if case.sorted_input:
            ml.linear(x, W, pool, *meta, lora_on=lora_on, out=y, workspace=ws)
        else:
            ml.linear_tokens(x, W, pool, tok, sc, lora_on=lora_on, out=y, workspace=ws)

    def timed(lora_on, steps, warmup):
        for _ in range(warmup):
            step(rot[0], lora_on)
            rot[0] += 1
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            step(rot[0], lora_on)
            rot[0] += 1
        e1.record(stream)
        e1.synchronize()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps   # ms per call

    res = {"n_sets": n_sets, "set_bytes": set_bytes}
    if args.profile:
        # counter runs: LoRA-on calls only, then a copy of known size
        timed(1, 5, 2)
        print(f"[bench] {label}: 7 lora_on calls done", file=sys.stderr, flush=True)
        n = 256 << 20
        src = torch.ones(n // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy of {n} bytes done", file=sys.stderr, flush=True)
        return res
    clock_warmup(lambda: (step(rot[0], 1), rot.__setitem__(0, rot[0] + 1)), args.clock_warmup)
    res["ms_on_eager"] = timed(1, args.steps, args.warmup)
    res["ms_off_eager"] = timed(0, args.steps, args.warmup)
    res["ms_on"], res["ms_off"] = res["ms_on_eager"], res["ms_off_eager"]
    if args.graph:
        for key, lo in (("ms_on", 1), ("ms_off", 0)):
            res[key] = graph_timed(lambda i, lo=lo: step(i, lo), n_sets, args.steps, args.warmup,
                                   offset=rot[0])
            rot[0] += args.warmup
    print(f"[bench] {label}: lora_on {res['ms_on'] * 1e3:.2f} us/call, lora_off {res['ms_off'] * 1e3:.2f} "
          f"us/call ({'graph replay' if args.graph else 'eager'}), {n_sets} buffer sets of "
          f"{set_bytes / 2**20:.1f} MiB", file=sys.stderr, flush=True)
    del sets, pool0, W0, x0
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def clock_warmup(call, seconds: float):
    """Untimed sustained load before a workload's timed calls: measured on
    the box, the same kernel ran up to 15% slower in the first ~100 ms of
    load (the GPU's clocks ramp), so a short timed loop after an idle host
    phase would read low. Runs `call` back to back for `seconds`."""
    import torch
    t_end = time.time() + seconds
    n = 0
    while time.time() < t_end:
        call()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def layer_summary(case, res, args) -> dict:
    """Per-workload figures of a measure_layer result: times, rates, the
    LoRA-on overhead beside its byte (or flop) floor ratio, and the roofline
    of the LoRA-on call (HBM-bound shapes against 8 TB/s, the prefill
    shapes against the 2.5 PFLOP/s bf16 MFMA peak)."""
    bytes_on, bytes_off, flops_on, flops_off = case_work(case)
    ms_on, ms_off = res["ms_on"], res["ms_off"]
    gbs_on = bytes_on / (ms_on * 1e-3) / 1e9
    gbs_off = bytes_off / (ms_off * 1e-3) / 1e9
    tf_on = flops_on / (ms_on * 1e-3) / 1e12
    tf_off = flops_off / (ms_off * 1e-3) / 1e12
    mfma = case.name.startswith("prefill")
    roof = {"bound": "hbm", "achieved": round(gbs_on, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs_on / HBM_PEAK_GBS, 4)}
    roof_off = {"frac": round(gbs_off / HBM_PEAK_GBS, 4)}
    if mfma:
        roof = {"bound": "mfma", "achieved": round(tf_on, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tf_on / MFMA_BF16_PEAK_TFLOPS, 4)}
        roof_off = {"frac": round(tf_off / MFMA_BF16_PEAK_TFLOPS, 4)}
    if case.dtype == "f32":
        roof["note"] = "bound by launch latency: its bytes take well under a microsecond at 8 TB/s"
    roof.update({"traffic": counted_traffic(case.name), "algorithmic_bytes": bytes_on,
                 "us_per_call": round(ms_on * 1e3, 3), "kernels": layer_kernels(case),
                 "kernel_source_hash": kernel_source_hash()})
    touched = case.touched_adapters()
    return {
        "tokens": case.n_tokens, "d_in": case.d_in, "d_out": case.d_out, "dtype": case.dtype,
        "adapters_touched": len(touched), "segments": case.n_seg if case.sorted_input else None,
        "sorted_input": bool(case.sorted_input),
        "ranks": sorted(set(case.adapters[a].rank for a in touched)),
        "us_lora_on": round(ms_on * 1e3, 3), "us_lora_off": round(ms_off * 1e3, 3),
        "gbs_lora_on": round(gbs_on, 1), "gbs_lora_off": round(gbs_off, 1),
        "tflops_lora_on": round(tf_on, 2), "tflops_lora_off": round(tf_off, 2),
        "unique_bytes_lora_on": bytes_on, "unique_bytes_lora_off": bytes_off,
        "lora_on_overhead": round(ms_on / ms_off - 1.0, 4),
        "floor_ratio": round((flops_on / flops_off) if mfma else (bytes_on / bytes_off), 4),
        "floor_ratio_of": "flops" if mfma else "bytes",
        "lora_off_frac": roof_off["frac"],
        "buffer_sets": res["n_sets"],
        "roofline": roof,
    }


def cpu_baseline(case, args) -> dict:
    """The fp64 oracle over a bounded sample of the workload's batch (the
    whole batch when it is small), timed on every CPU of the affinity mask
    and once on one thread; value scaled to the whole batch."""
    import numpy as np
    import oracle
    threads = cpu_threads()
    T, d_in, d_out = case.n_tokens, case.d_in, case.d_out
    bytes_on, _, flops_on, _ = case_work(case)
    pool_o = oracle.PackedPool(case.adapters, case.capacity, d_in, d_out)
    rows, n_rows = None, T
    max_rows = max(1, int(4e10 / (2.0 * d_in * d_out)))
    if T > max_rows:
        rows = np.arange(max_rows, dtype=np.int32)
        n_rows = max_rows
    reps, t_total = 0, 0.0
    while t_total * threads < args.cpu_seconds or reps == 0:
        t0 = time.perf_counter()
        oracle.case_linear(case, 1, rows=rows, threads=threads, pool=pool_o)
        t_total += time.perf_counter() - t0
        reps += 1
        if reps >= 50:
            break
    t_batch = t_total / reps * (T / n_rows)
    # the same sample on one thread, once (outputs are bitwise the same at any thread count)
    rows1 = rows if rows is not None else np.arange(min(T, max(1, n_rows // 4)), dtype=np.int32)
    t0 = time.perf_counter()
    oracle.case_linear(case, 1, rows=rows1, threads=1, pool=pool_o)
    t_1 = (time.perf_counter() - t0) * (T / len(rows1))
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(bytes_on / t_batch / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n_rows} of {T} rows of the {case.name} batch, lora_on=1, fp64, "
                      f"{reps} repetitions, {t_total:.1f} s wall on all {threads} CPUs of the affinity "
                      f"mask; value scaled to the whole batch",
            "seconds_per_batch": round(t_batch, 4),
            "single_thread": {"seconds_per_batch": round(t_1, 4),
                              "value": round(bytes_on / t_1 / 1e9, 4),
                              "sample": f"{len(rows1)} rows, once, scaled to the whole batch"},
            "gflops_fp64": round(flops_on / t_batch / 1e9, 2),
            "cpu_model": cpu_model}


# The configurations the default run measures besides the headline (decode):
# the fp32 tiny case, the verify pass, the heterogeneous-rank batch and the
# seven projections of one decoder layer at the prefill batch.
OTHER_CONFIGS = [("tiny_f32", "q"), ("verify_bf16", "q"), ("hetero_bf16", "q")] + [
    ("prefill_bf16", p) for p in ("q", "k", "v", "o", "gate", "up", "down")]


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this layer is built and timed on a single MI355X "
              "(no sharding or collectives); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.workload == "merge_bf16":
        bench_merge(args)
        return
    if args.workload.startswith("fused_"):
        bench_fused(args)
        return
    if args.workload == "cycle_verify":
        bench_cycle(args)
        return
    if args.workload == "decode_fp8w":
        bench_fp8w(args)
        return
    if args.workload == "path_sweep":
        if args.sweep_counters:
            print(json.dumps({"path_sweep_counters": ingest_sweep_counters(*args.sweep_counters)}))
            return
        bench_path_sweep(args)
        return

    import torch
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from mlora_inputs import make_case

    head = "decode_bf16" if args.workload == "all" else args.workload
    case = make_case(head, args.proj)
    if args.ingest_counters:
        ent = ingest_counters(case.name, layer_kernels(case), *args.ingest_counters)
        print(json.dumps({case.name: ent}))
        return
    torch.cuda.set_device(0)
    res = measure_layer(case, args, case.name)
    if args.profile:
        return
    summ = layer_summary(case, res, args)
    others = {}
    if args.workload == "all":
        for name, proj in OTHER_CONFIGS:
            c = make_case(name, proj)
            others[c.name] = layer_summary(c, measure_layer(c, args, c.name), args)
            del c
    cpu = None if args.no_cpu_baseline else cpu_baseline(case, args)

    bytes_on, bytes_off = summ["unique_bytes_lora_on"], summ["unique_bytes_lora_off"]
    cfg = {"workload": case.name, "tokens": case.n_tokens, "d_in": case.d_in, "d_out": case.d_out,
           "adapters_touched": summ["adapters_touched"], "segments": summ["segments"],
           "ranks": summ["ranks"], "lora_on": 1, "buffer_sets": res["n_sets"],
           "unique_bytes_lora_on": bytes_on, "unique_bytes_lora_off": bytes_off}
    ms_on, ms_off = res["ms_on"], res["ms_off"]
    out = {
        "metric": METRIC, "value": summ["gbs_lora_on"], "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_on, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": case.dtype,
        "data": "synthetic (seeded Gaussian weights, adapters and activations)",
        "config": cfg,
        "tflops": summ["tflops_lora_on"], "pct_hbm_roofline": round(100 * summ["gbs_lora_on"] / HBM_PEAK_GBS, 2),
        "lora_off": {"ms_per_step": round(ms_off, 6), "gbs": summ["gbs_lora_off"],
                     "tflops": summ["tflops_lora_off"],
                     "pct_hbm_roofline": round(100 * summ["gbs_lora_off"] / HBM_PEAK_GBS, 2)},
        "lora_on_overhead": summ["lora_on_overhead"],
        "byte_floor_ratio": round(bytes_on / bytes_off, 4),
        "timing": ("K calls replayed from HIP graphs (one graph per pass over the buffer sets)"
                   if args.graph else "K eager calls through the Python binding, buffer sets rotated "
                   "continuously from the warm-up on")
                  + f"; each workload first runs {args.clock_warmup} s of untimed LoRA-on calls (clock ramp)",
        "eager": {"ms_per_step_lora_on": round(res["ms_on_eager"], 6),
                  "ms_per_step_lora_off": round(res["ms_off_eager"], 6)},
        "roofline": summ["roofline"],
        "cpu_baseline": cpu,
    }
    if others:
        out["configs"] = others
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
