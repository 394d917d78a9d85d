"""Helpers shared by the GPU tests: move a generated case to the device, run the
HIP library through its C ABI, run the fp64 oracle on the same inputs, and
compare element by element."""
from __future__ import annotations

import os
import sys
from typing import Optional

import numpy as np
import torch

import oracle
from mlora_inputs import Case, bf16_bits

BF16_TOL = 2e-2      # |y_gpu - y_ref| <= 2e-2 * (1 + |y_ref|)  (bf16 out, fp32 accumulate)
F32_TOL = 1e-4       # |y_gpu - y_ref| <= 1e-4 * (1 + |y_ref|)  (fp32 config)


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def to_dev(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        bits = bf16_bits(a).view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(bits)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def i32(a, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def f32(a, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


class DeviceCase:
    """A generated case resident on the GPU with its adapters registered."""

    def __init__(self, case: Case, lib=None, register=True):
        import rank_adapter_gemm_segmented_amd as ml
        self.case = case
        self.ml = ml
        tdt = torch.bfloat16 if case.dtype == "bf16" else torch.float32
        self.tdt = tdt
        self.x = to_dev(case.x, case.dtype)
        self.W = to_dev(case.W, case.dtype)
        self.pool = ml.Pool(case.d_in, case.d_out, tdt, case.max_rank, case.capacity)
        if register:
            for aid in sorted(case.adapters):
                ad = case.adapters[aid]
                self.pool.register(aid, to_dev(ad.A, case.dtype), to_dev(ad.B, case.dtype))
        self.ws = self.pool.workspace(case.n_tokens)
        if case.sorted_input:
            self.seg_start = i32(case.seg_start)
            self.seg_adapter = i32(case.seg_adapter)
            self.seg_rank = i32(case.seg_rank)
            self.seg_scale = f32(case.seg_scale)
            self.token_index = None if case.token_index is None else i32(case.token_index)
        self.token_adapter = i32(case.token_adapter)
        self.adapter_scale = f32(case.adapter_scale)

    def run(self, lora_on: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        c = self.case
        if c.sorted_input:
            y = self.ml.linear(self.x, self.W, self.pool, self.seg_start, self.seg_adapter,
                               self.seg_rank, self.seg_scale, lora_on=lora_on,
                               token_index=self.token_index, out=out, workspace=self.ws)
        else:
            y = self.ml.linear_tokens(self.x, self.W, self.pool, self.token_adapter,
                                      self.adapter_scale, lora_on=lora_on, out=out,
                                      workspace=self.ws)
        torch.cuda.synchronize()
        return y


def y_host(y: torch.Tensor) -> np.ndarray:
    return y.float().cpu().numpy().astype(np.float64)


def sample_rows(case: Case, n_random: int, seed: int = 0) -> np.ndarray:
    """First and last batch row of every segment plus seeded random rows."""
    rng = np.random.default_rng(seed)
    rows = set()
    if case.sorted_input:
        ss = case.seg_start
        ti = case.token_index
        for s in range(len(ss) - 1):
            if ss[s + 1] > ss[s]:
                for p in (int(ss[s]), int(ss[s + 1]) - 1):
                    rows.add(int(ti[p]) if ti is not None else p)
    else:
        ta = case.token_adapter
        for a in np.unique(ta):
            idx = np.nonzero(ta == a)[0]
            rows.add(int(idx[0]))
            rows.add(int(idx[-1]))
    rows.update(rng.integers(0, case.n_tokens, size=n_random).tolist())
    rows.add(case.n_tokens - 1)
    return np.array(sorted(rows), dtype=np.int32)


def tolerance(case: Case) -> float:
    return F32_TOL if case.dtype == "f32" else BF16_TOL


def compare(y_gpu: np.ndarray, y_ref: np.ndarray, tol: float, what: str):
    assert y_gpu.shape == y_ref.shape, (y_gpu.shape, y_ref.shape)
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite GPU output"
    err = np.abs(y_gpu - y_ref)
    bound = tol * (1.0 + np.abs(y_ref))
    worst = float(np.max(err / bound)) if err.size else 0.0
    if worst > 1.0:
        i = np.unravel_index(int(np.argmax(err / bound)), err.shape)
        raise AssertionError(f"{what}: max err/bound {worst:.3f} at {i}: gpu {y_gpu[i]!r} ref {y_ref[i]!r}")
    return worst


def check_case(dc: DeviceCase, lora_on: int, rows: Optional[np.ndarray] = None, what: str = ""):
    """Run the GPU and the oracle on the same case and compare (all rows if
    ``rows`` is None)."""
    c = dc.case
    y = y_host(dc.run(lora_on))
    y_ref = oracle.case_linear(c, lora_on, rows=rows, threads=oracle_threads())
    yg = y if rows is None else y[rows]
    return compare(yg, y_ref, tolerance(c), what or f"{c.name} lora_on={lora_on}")
