"""Layer-level cost model of the InvisibleLoRA decoding cycle and its run-time gate.

Per the *InvisibleLoRA* abstract, the shared base model with every adapter
switched off drafts one token for each request, and a single pass with the
adapters switched on then checks all of those drafts together; the adapters
thus run once per cycle, not once per generated token. A gate decides at run
time whether a step drafts at all (drafting is dropped where it would not pay
for itself), and the abstract quotes median acceptance rates of 92-97%.

The abstract gives no formula for either. This module takes the plainest
reading that the rest supports:

* A cycle over a batch of ``b`` requests costs one LoRA-off pass over ``b``
  tokens (the draft) plus one LoRA-on pass over ``2 b`` tokens (each request's
  last committed token and its draft). With acceptance rate ``alpha`` it
  commits ``1 + alpha`` tokens per request on average: the verified draft with
  probability ``alpha``, and always the target's own next token.
* Plain multi-LoRA decoding commits one token per request per LoRA-on pass
  over ``b`` tokens.
* The gate drafts exactly when the cycle's expected time per committed token
  is below the plain step's:  (t_off(b) + t_on(2b)) / (1 + alpha) < t_on(b).

The times are one layer's (this library's measured calls). Attention, the KV
cache and sampling are outside the model.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class CycleEstimate:
    per_token_plain: float     # t_on(b): one LoRA-on pass per committed token
    per_token_cycle: float     # (t_off(b) + t_on(2b)) / (1 + alpha)
    speedup: float             # per_token_plain / per_token_cycle
    draft: bool                # the gate's decision


def cycle_estimate(t_on_b: float, t_off_b: float, t_on_2b: float, alpha: float) -> CycleEstimate:
    """Expected time per committed token with and without drafting, and the
    gate's decision, from one layer's measured pass times (any time unit)."""
    if not (0.0 <= alpha <= 1.0):
        raise ValueError("alpha is an acceptance rate in [0, 1]")
    if min(t_on_b, t_off_b, t_on_2b) <= 0.0:
        raise ValueError("pass times must be positive")
    cyc = (t_off_b + t_on_2b) / (1.0 + alpha)
    return CycleEstimate(t_on_b, cyc, t_on_b / cyc, cyc < t_on_b)


def break_even_alpha(t_on_b: float, t_off_b: float, t_on_2b: float) -> float:
    """Smallest acceptance rate at which drafting pays (may exceed 1: never)."""
    return (t_off_b + t_on_2b) / t_on_b - 1.0


def verify_segments(draft_seg_start, tokens_per_request: int = 2) -> np.ndarray:
    """Segment starts of the verification pass, from those of the draft pass.

    The draft pass holds one position per request, with requests grouped by
    adapter; the verification pass holds ``tokens_per_request`` consecutive
    positions per request (its last committed token, then its draft) in the
    same request order, so every segment keeps its adapter, rank and scale
    and its bounds scale by ``tokens_per_request``."""
    ss = np.asarray(draft_seg_start, dtype=np.int64)
    if tokens_per_request < 1:
        raise ValueError("a request holds at least one position")
    if ss.ndim != 1 or ss.size < 1 or ss[0] != 0 or np.any(np.diff(ss) < 0):
        raise ValueError("seg_start must start at 0 and be non-decreasing")
    return (ss * tokens_per_request).astype(np.int32)


def cycle_passes(linear, x_draft, x_verify, W, pool, seg_start, seg_adapter, seg_rank, seg_scale,
                 tokens_per_request: int = 2, workspace=None):
    """One decoding cycle of a layer through ``linear`` (the binding's
    ``mlora_linear``): the LoRA-off draft pass over ``x_draft`` (one row per
    request) and the LoRA-on verification pass over ``x_verify``
    (``tokens_per_request`` rows per request, request-major). ``seg_*`` are
    the draft pass's device metadata; the verification pass's starts come
    from ``verify_segments``. Returns (y_draft, y_verify)."""
    import torch
    b = int(x_draft.shape[0])
    if int(x_verify.shape[0]) != tokens_per_request * b:
        raise ValueError("the verification batch holds tokens_per_request rows per request")
    vss = torch.from_numpy(verify_segments(seg_start.cpu().numpy(), tokens_per_request)).to(seg_start.device)
    y_draft = linear(x_draft, W, pool, seg_start, seg_adapter, seg_rank, seg_scale, lora_on=0,
                     workspace=workspace)
    y_verify = linear(x_verify, W, pool, vss, seg_adapter, seg_rank, seg_scale, lora_on=1,
                      workspace=workspace)
    return y_draft, y_verify
