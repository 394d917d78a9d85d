/*
 * mlora.h -- C ABI of the MI355X (gfx950) multi-LoRA segmented linear layer.
 *
 * The layer computes, for every token i of a batch,
 *
 *     y_i = W x_i + scale_s * B_a (A_a x_i)       (lora_on = 1, a = adapter of i's segment)
 *     y_i = W x_i                                  (lora_on = 0, or a = -1)
 *
 * which is the LoRA forward of "Multi-LoRA Serving in Practice", section "Core
 * Principle" (displayed formula), applied per request with one shared base
 * weight W and a per-request adapter (same section: the request names the
 * adapter it uses). The batch is split into segments, one adapter per
 * segment (the "InvisibleLoRA" abstract divides a batch's requests among the
 * adapters in use; "Multi-LoRA Serving in Practice", section "4. Batching":
 * adapter-aware batching groups requests of one adapter). lora_on = 0 is the
 * InvisibleLoRA LoRA-off drafter pass (base model alone); lora_on = 1 is its
 * LoRA-on verification pass.
 *
 * Conventions for every entry point:
 *  - Layouts are row-major: x [T, d_in], W [d_out, d_in], y [T, d_out],
 *    A_a [rank, d_in], B_a [d_out, rank].
 *  - x, W, y and the adapter pool share one element type (mlora_dtype_t).
 *    bf16 inputs accumulate in fp32 and y is rounded to bf16 once
 *    (round-to-nearest-even); fp32 inputs accumulate and store in fp32.
 *  - Array arguments are DEVICE pointers unless stated otherwise, 16-byte
 *    aligned. Sizes and flags are host integers. Every call is asynchronous
 *    and stream-ordered on `stream` (NULL = the legacy default stream).
 *  - The library never allocates or frees device memory: the caller owns the
 *    pool arena, the workspace, and all inputs and outputs.
 *  - Errors: host-side validation returns a status and launches nothing.
 *    Device-side faults surface as MLORA_ERR_HIP on a later call or sync.
 *    Metadata that lies (adapter ids, ranks, segment bounds) never causes an
 *    out-of-bounds access: kernels clamp every metadata-derived index, and
 *    mlora_validate() reports such metadata. No C++ exception crosses the ABI.
 *  - Calls that share a pool or a workspace must be ordered by the caller
 *    (same stream, or events); the library takes no locks.
 */
#ifndef MLORA_H
#define MLORA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mlora_pool_s* mlora_pool_t;

typedef enum { MLORA_F32 = 0, MLORA_BF16 = 1 } mlora_dtype_t;

typedef enum {
  MLORA_OK = 0,
  MLORA_ERR_INVALID_ARG = 1, /* null pointer, misaligned pointer, bad flag        */
  MLORA_ERR_SHAPE = 2,       /* a size is out of the supported range              */
  MLORA_ERR_DTYPE = 3,       /* unknown element type                              */
  MLORA_ERR_RANK = 4,        /* rank < 1, rank > max_rank, or rank mismatch       */
  MLORA_ERR_ADAPTER = 5,     /* adapter id out of range or not registered         */
  MLORA_ERR_EXISTS = 6,      /* adapter id already registered                     */
  MLORA_ERR_WORKSPACE = 7,   /* workspace (or pool arena) too small               */
  MLORA_ERR_METADATA = 8,    /* segment metadata inconsistent                     */
  MLORA_ERR_HIP = 9          /* a HIP runtime call failed                         */
} mlora_status_t;

/* Supported ranges. d_in must be a multiple of 8 (bf16) or 4 (fp32) so rows
 * stay 16-byte aligned; d_out is free. */
#define MLORA_MAX_DIM (1 << 17)
#define MLORA_MAX_RANK 256
#define MLORA_MAX_TOKENS (1 << 20)
#define MLORA_MAX_UNSORTED_TOKENS 8192
#define MLORA_MAX_SEGMENTS 16384

/* Human-readable text for a status code (static storage). */
const char* mlora_status_string(int status);

/* ------------------------------------------------------------------------
 * Adapter pool: a fixed-slot, device-resident arena.
 *
 * Adapter slots are addressed by id in [0, capacity). Each slot can hold an
 * adapter of rank <= max_rank; only rank*(d_in+d_out) elements of a slot are
 * ever read. A device table of registered ranks sits at the end of the arena.
 * This is the serving side's bound on adapter rank ("Multi-LoRA Serving in
 * Practice", section "Go-Live Checklist": a maximum LoRA rank and a cap on the
 * adapters loaded per replica) and its runtime loading and per-adapter
 * disable (same page, section "2. Choose a Loading Mode" and the checklist).
 * ---------------------------------------------------------------------- */

/* Bytes of device memory a pool of this shape needs (0 if the shape is out of
 * range). */
size_t mlora_pool_bytes(int d_in, int d_out, int dtype, int max_rank, int capacity);

/* Create a pool handle over caller-owned device memory `dev_mem` of `bytes`
 * bytes (>= mlora_pool_bytes). Marks every slot empty (stream-ordered on
 * `stream`). On success *out receives the handle, which owns only host state. */
int mlora_pool_create(void* dev_mem, size_t bytes, int d_in, int d_out, int dtype, int max_rank,
                      int capacity, hipStream_t stream, mlora_pool_t* out);

/* Free the host handle. Device memory stays the caller's. NULL is a no-op. */
int mlora_pool_destroy(mlora_pool_t pool);

/* Copy adapter `adapter_id` into its slot: A [rank, d_in] and B [d_out, rank]
 * in the pool's element type, host or device pointers (copied with
 * hipMemcpyKind "default"). The copy is stream-ordered: a later mlora_linear on
 * the same stream sees the adapter, and A and B may be reused once the stream
 * has passed this call. Errors: MLORA_ERR_ADAPTER (id out of range),
 * MLORA_ERR_EXISTS (slot occupied), MLORA_ERR_RANK (rank < 1 or > max_rank),
 * MLORA_ERR_SHAPE (the pool holds fused adapters: see below). */
int mlora_register_adapter(mlora_pool_t pool, int adapter_id, int rank, const void* A,
                           const void* B, hipStream_t stream);

/* Register one adapter that targets several projections whose base weights
 * are stacked into the pool's W, e.g. W = [W_q; W_k; W_v] or [W_gate; W_up]
 * (an adapter's config lists its target modules, with one rank and one
 * scaling: "Multi-LoRA Serving in Practice", section "1. Define Adapter
 * Asset Standards", adapter_config.json). Slice m covers slice_rows[m]
 * consecutive output rows (the slices in order fill d_out exactly) and carries
 * A_m [slice_ranks[m], d_in] and B_m [slice_rows[m], slice_ranks[m]].
 * The slot holds them as one adapter of rank R = sum(slice_ranks):
 * A = [A_0; A_1; ...] stacked, so one shrink pass over x serves every slice,
 * and B block-diagonal [d_out, R], so slice m's rows expand only its own
 * part of v. mlora_linear then computes, for every slice at once,
 *     y[:, slice m] = W_m x + scale_s * B_m (A_m x)
 * with one scale per segment shared by the slices. Segments name the
 * adapter with seg_rank = R. A pool holds either plain adapters or fused
 * ones over one stacking of W: its first fused registration fixes the slice
 * rows, and later ones must repeat them. When every fused adapter of the
 * pool has equal slice ranks (one rank per adapter config), the expand of a
 * row tile inside one slice reads only that slice's rank columns; otherwise
 * it reads all R columns, zero blocks included. n_slices in
 * 1 .. MLORA_MAX_SLICES; slice_rows, slice_ranks, A and B are host arrays
 * (A[m], B[m] host or device pointers, copied as in mlora_register_adapter).
 * Errors as mlora_register_adapter, plus MLORA_ERR_SHAPE (slice rows do not
 * add up to d_out, the pool holds plain adapters, or its fused adapters
 * stack W differently) and MLORA_ERR_RANK (R > max_rank). */
#define MLORA_MAX_SLICES 8
int mlora_register_adapter_fused(mlora_pool_t pool, int adapter_id, int n_slices,
                                 const int* slice_rows, const int* slice_ranks,
                                 const void* const* A, const void* const* B, hipStream_t stream);

/* Mark a slot empty (stream-ordered). Segments that still name it are
 * reported by mlora_validate and contribute no adapter term. */
int mlora_unregister_adapter(mlora_pool_t pool, int adapter_id, hipStream_t stream);

/* Registered rank of a slot (0 if empty), or -1 for a bad handle or id. */
int mlora_adapter_rank(mlora_pool_t pool, int adapter_id);

/* ------------------------------------------------------------------------
 * Workspace
 * ---------------------------------------------------------------------- */

/* Bytes of workspace a call with up to `max_tokens` tokens needs on this pool
 * (covers mlora_linear, mlora_linear_tokens and mlora_build_segments). */
size_t mlora_workspace_bytes(mlora_pool_t pool, int max_tokens);

/* Zero-fill a workspace (stream-ordered). Must be called once on a newly
 * allocated workspace before its first use; the library leaves it in a
 * reusable state after every call. */
int mlora_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * The layer
 * ---------------------------------------------------------------------- */

/* y = W x + per-segment adapter term over a batch of n_tokens rows.
 *
 * Segment metadata (device, ignored and may be NULL when lora_on = 0):
 *   seg_start [n_seg + 1]  sorted positions: seg_start[0] = 0, non-decreasing,
 *                          seg_start[n_seg] = n_tokens. Empty segments allowed.
 *   seg_adapter [n_seg]    adapter id of each segment, or -1 for base only.
 *   seg_rank [n_seg]       rank of each segment's adapter (must equal the
 *                          registered rank; 0 for id -1).
 *   seg_scale [n_seg]      fp32 scale of each segment (any value, 0 allowed).
 *   token_index [n_tokens] or NULL: sorted position p holds batch row
 *                          token_index[p] of x and y (NULL = identity, i.e. the
 *                          caller already grouped its rows).
 * lora_on: 0 (LoRA-off drafter pass: y = W x) or 1.
 * n_seg: 1 .. MLORA_MAX_SEGMENTS when lora_on = 1.
 * Errors: MLORA_ERR_INVALID_ARG, MLORA_ERR_SHAPE, MLORA_ERR_WORKSPACE,
 * MLORA_ERR_METADATA (n_seg < 1) from host checks. Inconsistent device
 * metadata is not detected here (see mlora_validate), unless the environment
 * sets MLORA_DEBUG_VALIDATE=1: then the call first checks the metadata on
 * the device as mlora_validate does (synchronizing `stream`) and returns
 * MLORA_ERR_METADATA, MLORA_ERR_ADAPTER or MLORA_ERR_RANK without running
 * the layer (also for mlora_linear_fp8w). With MLORA_LOG=1 every layer call
 * prints one line on stderr: the path taken (decode, decode-fp8w, gemm, gemv,
 * f32), T, the shape, dtype, lora_on, the segment count, the d_in split,
 * the shrink kernel (short, mfma, fused into the decode stream, f32 or none)
 * and the pool's max rank. */
int mlora_linear(const void* x, const void* W, mlora_pool_t pool, const int32_t* seg_start,
                 const int32_t* seg_adapter, const int32_t* seg_rank, const float* seg_scale,
                 const int32_t* token_index, int n_tokens, int n_seg, int lora_on, void* y,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* mlora_linear without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. The call allocates nothing (no hipMalloc,
 * no hipFree, no allocating library routine); the layer's workspace is a
 * library-owned device array of MLORA_NOALLOC_SCRATCH_BYTES bytes, one per
 * GPU the library runs on, held until the process ends. Arguments, results
 * and errors as mlora_linear (same kernels, same bits). A call whose
 * workspace (mlora_workspace_bytes of its n_tokens) exceeds the scratch
 * returns MLORA_ERR_WORKSPACE and launches nothing. Every call on one GPU
 * shares that GPU's scratch, which keeps the last call's contents: calls on
 * one GPU must not overlap (one stream, or ordered by events), or they race.
 * The first call on a device looks up the scratch's device address
 * (hipGetSymbolAddress) with that device current. */
#define MLORA_NOALLOC_SCRATCH_BYTES (64u << 20)
int mlora_linear_noalloc(const void* x, const void* W, mlora_pool_t pool, const int32_t* seg_start,
                         const int32_t* seg_adapter, const int32_t* seg_rank, const float* seg_scale,
                         const int32_t* token_index, int n_tokens, int n_seg, int lora_on, void* y,
                         hipStream_t stream);

/* The layer with the base weight stored as FP8 and the adapters in bf16:
 *
 *     y_i = diag(w_scale) (Q x_i) + scale_s * B_a (A_a x_i),
 *
 * i.e. the dequantized weight W[n, k] = w_scale[n] * e4m3(W_fp8[n, k]).
 * Quantizing the weights of a LoRA-served model to FP8 is named by the "LoRA
 * Inference" glossary (the paragraph on inference optimizations for merged
 * weights); at decode the layer streams W from HBM, so one byte per weight
 * halves the dominant traffic. W_fp8 [d_out, d_in] holds OCP FP8 E4M3 codes
 * (bias 7, subnormals, no infinities; NaN codes are not supported), w_scale
 * [d_out] float32 (device). x, y and the pool are bf16; each e4m3 value is
 * exact in bf16, products accumulate in fp32, the row scale multiplies the
 * finished base sum, and y is rounded to bf16 once. Other arguments as
 * mlora_linear. Batches of 1 .. MLORA_MAX_FP8W_TOKENS tokens (the split-K
 * decode path) and d_in a multiple of 16.
 * Errors: as mlora_linear, plus MLORA_ERR_DTYPE (pool not bf16) and
 * MLORA_ERR_SHAPE (more tokens, more segments or ranks than the decode path
 * takes, or d_in not a multiple of 16). */
#define MLORA_MAX_FP8W_TOKENS 64
int mlora_linear_fp8w(const void* x, const uint8_t* W_fp8, const float* w_scale, mlora_pool_t pool,
                      const int32_t* seg_start, const int32_t* seg_adapter, const int32_t* seg_rank,
                      const float* seg_scale, const int32_t* token_index, int n_tokens, int n_seg,
                      int lora_on, void* y, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* Canonical segmentation of an unsorted batch on the device: tokens grouped
 * by adapter id in ascending id order (-1 first), tokens of one id in
 * ascending batch order. Outputs (device):
 *   token_index [n_tokens], seg_start [n_tokens + 2], seg_adapter [n_tokens + 1],
 *   seg_rank [n_tokens + 1] (registered ranks), seg_scale [n_tokens + 1]
 *   (adapter_scale[id], 0 for -1), n_seg_out [1].
 * Ids outside [-1, capacity) or unregistered become base-only segments of
 * their own id value and are reported by mlora_validate.
 * n_tokens <= MLORA_MAX_UNSORTED_TOKENS. */
int mlora_build_segments(const int32_t* token_adapter, const float* adapter_scale, int n_tokens,
                         mlora_pool_t pool, int32_t* token_index, int32_t* seg_start,
                         int32_t* seg_adapter, int32_t* seg_rank, float* seg_scale,
                         int32_t* n_seg_out, hipStream_t stream);

/* The layer on an unsorted batch: token_adapter [n_tokens] gives each row's
 * adapter id (-1 = base only), adapter_scale [capacity] the fp32 scale of each
 * adapter. The library segments the batch in the workspace (as
 * mlora_build_segments) and runs mlora_linear on it; x and y stay in the
 * caller's row order. n_tokens <= MLORA_MAX_UNSORTED_TOKENS. */
int mlora_linear_tokens(const void* x, const void* W, mlora_pool_t pool,
                        const int32_t* token_adapter, const float* adapter_scale, int n_tokens,
                        int lora_on, void* y, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/* Token map of sorted metadata: for each sorted position p < n_tokens, the
 * segment s with seg_start[s] <= p < seg_start[s+1] and its adapter id. The
 * same lookup the layer kernels use. Outputs are device int32 [n_tokens]. */
int mlora_token_map(const int32_t* seg_start, const int32_t* seg_adapter, int n_tokens, int n_seg,
                    int32_t* token_seg, int32_t* token_adapter_out, hipStream_t stream);

/* Check segment metadata on the device and wait for the answer (synchronizes
 * `stream`). Returns MLORA_OK, MLORA_ERR_METADATA (bounds, order, or
 * token_index not a permutation), MLORA_ERR_ADAPTER (id out of range or not
 * registered) or MLORA_ERR_RANK (seg_rank differs from the registered rank).
 * seg_rank and token_index may be NULL. Uses the first bytes of the
 * workspace. */
int mlora_validate(mlora_pool_t pool, const int32_t* seg_start, const int32_t* seg_adapter,
                   const int32_t* seg_rank, const int32_t* token_index, int n_tokens, int n_seg,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Merged weights
 * ---------------------------------------------------------------------- */

/* Merge registered adapter `adapter_id` into a base weight:
 *
 *     W_out = W_in + scale * B_a A_a          (W_in, W_out [d_out, d_in], pool dtype)
 *
 * The "LoRA Inference" glossary (first paragraph) serves an adapter merged into
 * the frozen weights, W = W0 + dW, at the base model's cost; dW is the scaled
 * low-rank term of the LoRA forward ("Multi-LoRA Serving in Practice", section
 * "Core Principle"). Its "Model Merging" paragraph combines adapters by
 * adding them: call once per adapter. A negative scale removes a merged
 * adapter (unmerge). bf16 accumulates dW in fp32 and rounds W_out once per
 * call (RNE), so unmerging restores W_in only to within that rounding; fp32
 * adds in fp32. Device pointers; W_out may equal W_in (in place) but must not
 * otherwise overlap it. Stream-ordered after the adapter's registration.
 * Errors: MLORA_ERR_INVALID_ARG (null or misaligned pointer, partial overlap),
 * MLORA_ERR_ADAPTER (id out of range or slot empty). */
int mlora_merge_adapter(const void* W_in, void* W_out, mlora_pool_t pool, int adapter_id,
                        float scale, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MLORA_H */
