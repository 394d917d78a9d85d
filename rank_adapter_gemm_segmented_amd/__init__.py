"""MI355X (gfx950) multi-LoRA segmented linear layer.

``y_i = W x_i + scale_s * B_a (A_a x_i)`` over a batch partitioned into
per-adapter segments, with a ``lora_on`` switch for the LoRA-off drafter pass.
The work runs in hand-written HIP kernels behind the C ABI of
``include/mlora.h`` (``csrc/``); this package is the thin Python binding.
"""
from .binding import (LIB_PATH, MLORA_BF16, MLORA_F32, STATUS, STATUS_CODE, MloraError, Pool,
                      build_segments, library, linear, linear_fp8w, linear_noalloc, linear_tokens,
                      merge_adapter, token_map, validate)

__all__ = ["LIB_PATH", "MLORA_BF16", "MLORA_F32", "STATUS", "STATUS_CODE", "MloraError", "Pool",
           "build_segments", "library", "linear", "linear_fp8w", "linear_noalloc", "linear_tokens",
           "merge_adapter",
           "token_map", "validate"]
