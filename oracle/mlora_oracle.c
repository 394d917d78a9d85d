/*
 * mlora_oracle.c -- plain fp64 CPU oracle for the multi-LoRA linear layer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call
 * this file; only the tests, the package smoke check and the benchmark's CPU
 * baseline do. It shares no code with the GPU library.
 *
 * What it computes (per token, written out as the plain definition):
 *
 *   y_i = W x_i + scale_s * B_a (A_a x_i)        if lora_on and a >= 0
 *   y_i = W x_i                                   otherwise
 *
 * following the LoRA forward of "Multi-LoRA Serving in Practice", section
 * "Core Principle" (its displayed formula: the base product plus a scaled
 * low-rank product, with A applied first and B second). The adapter a and its
 * scale come from the token's segment: the batch is partitioned into segments,
 * one adapter each (the "InvisibleLoRA" abstract splits a batch's requests
 * among the adapters in use). lora_on = 0 is that abstract's LoRA-off drafter pass,
 * which runs the shared base model alone.
 *
 * Layouts (row-major): x [T, d_in], W [d_out, d_in], A_a [r_a, d_in],
 * B_a [d_out, r_a], y [T, d_out]. Inputs arrive as float32 (every bf16 and
 * fp32 input value is exactly a float32) and are widened to double at use.
 * Each dot product runs over k in ascending order in double; build with
 * -ffp-contract=off so no multiply-add is fused. Rows are independent, so the
 * result does not depend on the number of OpenMP threads.
 *
 * The segment of a token and the adapter of a segment are found by brute
 * force linear scans over the metadata, never by a prefix structure.
 *
 * Parity status: every function here is pinned by tests against closed
 * forms, library routines (numpy fp64 products), the merged-weight identity
 * W = W0 + dW of the "LoRA Inference" glossary (first paragraph), a
 * hand-computed example, or exhaustive enumeration.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define MLO_OK 0
#define MLO_ERR_ARG (-1)      /* bad sizes or null pointers               */
#define MLO_ERR_META (-2)     /* segment metadata inconsistent            */
#define MLO_ERR_ADAPTER (-3)  /* adapter id out of range or unregistered  */
#define MLO_ERR_RANK (-4)     /* segment rank differs from registered rank */

/*
 * Canonical segmentation of an unsorted batch.
 *
 * Groups tokens by adapter id, ids in ascending order with -1 (base only)
 * first, tokens of one id in ascending batch order (a stable grouping). Only
 * non-empty groups become segments. Brute force: one pass over all tokens
 * per candidate id.
 *
 * Out: token_index[p] = batch token at sorted position p (T entries),
 *      seg_start[0..S], seg_adapter[0..S-1]. Returns S, or an error code if a
 *      token id lies outside [-1, capacity).
 */
int mlo_segment(int n_tokens, const int32_t* token_adapter, int capacity,
                int32_t* token_index, int32_t* seg_start, int32_t* seg_adapter) {
  if (n_tokens < 0 || capacity < 0) return MLO_ERR_ARG;
  for (int t = 0; t < n_tokens; ++t)
    if (token_adapter[t] < -1 || token_adapter[t] >= capacity) return MLO_ERR_ADAPTER;
  int p = 0, s = 0;
  seg_start[0] = 0;
  for (int id = -1; id < capacity; ++id) {
    int count = 0;
    for (int t = 0; t < n_tokens; ++t) {
      if (token_adapter[t] == id) {
        token_index[p++] = t;
        ++count;
      }
    }
    if (count > 0) {
      seg_adapter[s] = id;
      seg_start[s + 1] = p;
      ++s;
    }
  }
  return s;
}

/*
 * Check that segment metadata describes a valid partition of T positions:
 * seg_start[0] = 0, non-decreasing, seg_start[S] = T; token_index (if given)
 * is a permutation of 0..T-1; every adapter id is -1 or a registered id, and
 * the segment rank equals the registered rank.
 */
int mlo_check_meta(int n_tokens, int n_seg, const int32_t* seg_start, const int32_t* seg_adapter,
                   const int32_t* seg_rank, const int32_t* token_index, int capacity,
                   const int32_t* adapter_rank) {
  if (n_tokens < 0 || n_seg < 0) return MLO_ERR_ARG;
  if (seg_start[0] != 0 || seg_start[n_seg] != n_tokens) return MLO_ERR_META;
  for (int s = 0; s < n_seg; ++s)
    if (seg_start[s + 1] < seg_start[s]) return MLO_ERR_META;
  if (token_index) {
    for (int i = 0; i < n_tokens; ++i) {
      int hits = 0;
      for (int p = 0; p < n_tokens; ++p) hits += (token_index[p] == i);
      if (hits != 1) return MLO_ERR_META;
    }
  }
  for (int s = 0; s < n_seg; ++s) {
    int a = seg_adapter[s];
    if (a == -1) continue;
    if (a < -1 || a >= capacity || adapter_rank[a] <= 0) return MLO_ERR_ADAPTER;
    if (seg_rank && seg_rank[s] != adapter_rank[a]) return MLO_ERR_RANK;
  }
  return MLO_OK;
}

/*
 * Token map over sorted positions: for every position p, the segment s with
 * seg_start[s] <= p < seg_start[s+1] (found by a linear scan) and that
 * segment's adapter id.
 */
int mlo_token_map(int n_tokens, int n_seg, const int32_t* seg_start, const int32_t* seg_adapter,
                  int32_t* token_seg, int32_t* token_adapter_out) {
  if (n_tokens < 0 || n_seg < 0) return MLO_ERR_ARG;
  for (int p = 0; p < n_tokens; ++p) {
    int found = -1;
    for (int s = 0; s < n_seg; ++s) {
      if (seg_start[s] <= p && p < seg_start[s + 1]) {
        found = s;
        break;
      }
    }
    if (found < 0) return MLO_ERR_META;
    token_seg[p] = found;
    token_adapter_out[p] = seg_adapter[found];
  }
  return MLO_OK;
}

/*
 * The layer itself, for a chosen list of output rows.
 *
 * Adapter pool: adapter_rank[id] (0 = empty slot); A of adapter id starts at
 * pool_a + a_off[id] ([rank, d_in] row-major), B at pool_b + b_off[id]
 * ([d_out, rank] row-major).
 *
 * rows[q] (q < n_rows) are batch token indices (the caller's order); row q of
 * y and y_base (each [n_rows, d_out]) receives token rows[q]. rows = NULL
 * computes every token in order (n_rows must then equal n_tokens).
 * y_base (optional) receives W x_i alone. n_threads <= 0 uses the OpenMP
 * default.
 */
int mlo_linear(int n_tokens, int d_in, int d_out, const float* x, const float* W,
               int capacity, const int32_t* adapter_rank, const int64_t* a_off,
               const int64_t* b_off, const float* pool_a, const float* pool_b, int n_seg,
               const int32_t* seg_start, const int32_t* seg_adapter, const int32_t* seg_rank,
               const float* seg_scale, const int32_t* token_index, int lora_on, int n_rows,
               const int32_t* rows, double* y, double* y_base, int n_threads) {
  if (n_tokens < 0 || d_in <= 0 || d_out <= 0 || n_rows < 0) return MLO_ERR_ARG;
  if (!rows && n_rows != n_tokens) return MLO_ERR_ARG;
  if (lora_on != 0 && lora_on != 1) return MLO_ERR_ARG;
  if (lora_on) {
    int rc = mlo_check_meta(n_tokens, n_seg, seg_start, seg_adapter, seg_rank, token_index,
                            capacity, adapter_rank);
    if (rc != MLO_OK) return rc;
  }
  for (int q = 0; q < n_rows; ++q) {
    int i = rows ? rows[q] : q;
    if (i < 0 || i >= n_tokens) return MLO_ERR_ARG;
  }
  int max_r = 0;
  for (int a = 0; a < capacity; ++a)
    if (adapter_rank[a] > max_r) max_r = adapter_rank[a];

  int err = MLO_OK;
#ifdef _OPENMP
  int nt = n_threads > 0 ? n_threads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
#endif
  {
    double* v = (double*)malloc(sizeof(double) * (size_t)(max_r > 0 ? max_r : 1));
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
    for (int q = 0; q < n_rows; ++q) {
      const int i = rows ? rows[q] : q;
      const float* xi = x + (size_t)i * d_in;
      double* yq = y + (size_t)q * d_out;

      /* base term: (W x_i)[n] = sum_k W[n,k] x_i[k] */
      for (int n = 0; n < d_out; ++n) {
        const float* wn = W + (size_t)n * d_in;
        double acc = 0.0;
        for (int k = 0; k < d_in; ++k) acc += (double)wn[k] * (double)xi[k];
        yq[n] = acc;
        if (y_base) y_base[(size_t)q * d_out + n] = acc;
      }
      if (!lora_on) continue;

      /* sorted position p of token i (brute force), then its segment s */
      int p = -1;
      if (token_index) {
        for (int pp = 0; pp < n_tokens; ++pp)
          if (token_index[pp] == i) { p = pp; break; }
      } else {
        p = i;
      }
      int s = -1;
      for (int ss = 0; ss < n_seg; ++ss)
        if (seg_start[ss] <= p && p < seg_start[ss + 1]) { s = ss; break; }
      if (p < 0 || s < 0) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
        err = MLO_ERR_META;
        continue;
      }
      const int a = seg_adapter[s];
      if (a < 0) continue;                       /* base-only token */
      const int r = adapter_rank[a];
      const double c = (double)seg_scale[s];
      const float* Aa = pool_a + a_off[a];
      const float* Ba = pool_b + b_off[a];

      /* shrink: v[j] = sum_k A_a[j,k] x_i[k] */
      for (int j = 0; j < r; ++j) {
        const float* aj = Aa + (size_t)j * d_in;
        double acc = 0.0;
        for (int k = 0; k < d_in; ++k) acc += (double)aj[k] * (double)xi[k];
        v[j] = acc;
      }
      /* expand and scale: y_i[n] += c * sum_j B_a[n,j] v[j] */
      for (int n = 0; n < d_out; ++n) {
        const float* bn = Ba + (size_t)n * r;
        double acc = 0.0;
        for (int j = 0; j < r; ++j) acc += (double)bn[j] * v[j];
        yq[n] = yq[n] + c * acc;
      }
    }
    free(v);
  }
  return err;
}

/*
 * Merged weight of one adapter: W_out = W + c * B A.
 *
 * The "LoRA Inference" glossary (first paragraph) merges an adapter into the
 * frozen weights as W = W0 + dW, and its "Model Merging" paragraph combines
 * adapters by adding them. The update of one adapter is the low-rank term of
 * the "Multi-LoRA Serving in Practice" LoRA forward (section "Core
 * Principle", displayed formula): scale times B applied after A, so
 * dW = c B A. A negative c removes a merged adapter again (unmerge).
 *
 * Plain definition in double, one output element at a time, j ascending:
 *   W_out[n,k] = W[n,k] + c * sum_{j<rank} B[n,j] * A[j,k]
 * with A [rank, d_in] and B [d_out, rank] row-major. Rows are independent, so
 * the result does not depend on the number of OpenMP threads.
 */
int mlo_merge(int d_in, int d_out, int rank, const float* W, const float* A, const float* B,
              double c, double* W_out, int n_threads) {
  if (d_in <= 0 || d_out <= 0 || rank < 0) return MLO_ERR_ARG;
  if (!W || !W_out || (rank > 0 && (!A || !B))) return MLO_ERR_ARG;
#ifdef _OPENMP
  int nt = n_threads > 0 ? n_threads : omp_get_max_threads();
#pragma omp parallel for num_threads(nt) schedule(static)
#endif
  for (int n = 0; n < d_out; ++n) {
    const float* bn = B + (size_t)n * rank;
    for (int k = 0; k < d_in; ++k) {
      double dw = 0.0;
      for (int j = 0; j < rank; ++j) dw += (double)bn[j] * (double)A[(size_t)j * d_in + k];
      W_out[(size_t)n * d_in + k] = (double)W[(size_t)n * d_in + k] + c * dw;
    }
  }
#ifndef _OPENMP
  (void)n_threads;
#endif
  return MLO_OK;
}
