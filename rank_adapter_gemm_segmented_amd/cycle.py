"""Layer-level cost model of the InvisibleLoRA decoding cycle and its run-time gate.

The *InvisibleLoRA* abstract describes the cycle: one LoRA-off pass of the shared
base model proposes the next token of every request in the batch, and one
LoRA-on pass verifies all proposals, so adapter work runs once per cycle
instead of once per token. It adds a run-time gate that skips drafting on
steps where the adapter cost cannot repay a draft pass, and reports median
draft acceptance of 92-97%.

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
