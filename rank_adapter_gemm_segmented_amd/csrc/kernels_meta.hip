// kernels_meta.hip -- segment metadata kernels for gfx950.
//
// The batch is partitioned into segments, one adapter each ("InvisibleLoRA"
// abstract: requests are partitioned across active adapters). Requests of the
// same adapter are grouped before the low-rank work ("Multi-LoRA Serving in
// Practice", section "4. Batching", adapter-aware batching). These kernels
// (a) map sorted positions to segments and adapters, (b) group an unsorted
// batch into canonical segments, (c) check caller metadata.
#include "common.h"
#include "launch.h"

namespace mlora {

// ---------------------------------------------------------------------------
// Token map: per sorted position, its segment and adapter id (-1 if no
// segment covers it, which only happens for inconsistent metadata).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_token_map(const int32_t* __restrict__ seg_start,
                                                   const int32_t* __restrict__ seg_adapter, int T,
                                                   int S, int32_t* __restrict__ token_seg,
                                                   int32_t* __restrict__ token_adapter) {
  int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= T) return;
  int s = -1, a = -1;
  if (S > 0) {
    int c = find_segment(seg_start, S, p);
    if (seg_start[c] <= p && p < seg_start[c + 1]) {
      s = c;
      a = seg_adapter[c];
    }
  }
  token_seg[p] = s;
  token_adapter[p] = a;
}

void launch_token_map(const int32_t* seg_start, const int32_t* seg_adapter, int T, int S,
                      int32_t* token_seg, int32_t* token_adapter, hipStream_t st) {
  if (T <= 0) return;
  hipLaunchKernelGGL(k_token_map, dim3((T + 255) / 256), dim3(256), 0, st, seg_start, seg_adapter,
                     T, S, token_seg, token_adapter);
}

// ---------------------------------------------------------------------------
// Canonical segmentation (one workgroup).
//
// Sorted position of token t = #{t' : id[t'] < id[t]} + #{t' < t : id[t'] == id[t]},
// i.e. a stable grouping by ascending id (-1 first). The count is exact integer
// work, so the result is unique and independent of thread scheduling. Then a
// block scan over "segment starts" numbers the segments.
// ---------------------------------------------------------------------------
constexpr int kSegThreads = 1024;

__global__ __launch_bounds__(kSegThreads) void k_build_segments(
    const int32_t* __restrict__ token_adapter, const float* __restrict__ adapter_scale, int T,
    PoolView pv, int32_t* __restrict__ token_index, int32_t* __restrict__ seg_start,
    int32_t* __restrict__ seg_adapter, int32_t* __restrict__ seg_rank,
    float* __restrict__ seg_scale, int32_t* __restrict__ n_seg_out) {
  extern __shared__ int32_t ids[];  // [T] ids in batch order
  __shared__ int32_t part[kSegThreads];
  const int tid = threadIdx.x;

  for (int t = tid; t < T; t += kSegThreads) ids[t] = token_adapter[t];
  __syncthreads();

  for (int t = tid; t < T; t += kSegThreads) {
    const int key = ids[t];
    int pos = 0;
    for (int u = 0; u < T; ++u) {
      const int o = ids[u];
      pos += (o < key) | ((o == key) & (u < t));
    }
    token_index[pos] = t;
  }
  __threadfence_block();
  __syncthreads();
  // id at sorted position p
  auto sid = [&](int p) { return ids[token_index[p]]; };

  // each thread owns a contiguous chunk of positions
  const int chunk = (T + kSegThreads - 1) / kSegThreads;
  const int pb = tid * chunk;
  const int pe = min(pb + chunk, T);
  int cnt = 0;
  for (int p = pb; p < pe; ++p) cnt += (p == 0 || sid(p) != sid(p - 1));
  part[tid] = cnt;
  __syncthreads();
  // inclusive Hillis-Steele scan over kSegThreads partial counts
  for (int off = 1; off < kSegThreads; off <<= 1) {
    int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int s = part[tid] - cnt;  // exclusive prefix = index of this chunk's first new segment
  for (int p = pb; p < pe; ++p) {
    if (p == 0 || sid(p) != sid(p - 1)) {
      const int key = sid(p);
      const bool valid = key >= 0 && key < pv.capacity;
      const int r = valid ? pv.rank[key] : 0;
      seg_start[s] = p;
      seg_adapter[s] = key;
      seg_rank[s] = r;
      seg_scale[s] = valid ? adapter_scale[key] : 0.0f;
      ++s;
    }
  }
  if (tid == kSegThreads - 1) {
    const int S = part[kSegThreads - 1];
    seg_start[S] = T;
    n_seg_out[0] = S;
  }
}

size_t build_segments_lds_bytes(int T) { return (size_t)T * sizeof(int32_t); }

void launch_build_segments(const int32_t* token_adapter, const float* adapter_scale, int T,
                           const PoolView& pv, int32_t* token_index, int32_t* seg_start,
                           int32_t* seg_adapter, int32_t* seg_rank, float* seg_scale,
                           int32_t* n_seg_out, hipStream_t st) {
  hipLaunchKernelGGL(k_build_segments, dim3(1), dim3(kSegThreads), build_segments_lds_bytes(T), st,
                     token_adapter, adapter_scale, T, pv, token_index, seg_start, seg_adapter,
                     seg_rank, seg_scale, n_seg_out);
}

// ---------------------------------------------------------------------------
// Metadata validation (one workgroup). result[0] receives the status:
//   METADATA if bounds, order or the token_index permutation fail; otherwise
//   the error of the first segment (in segment order) whose adapter is out of
//   range or unregistered (ADAPTER) or whose rank differs (RANK).
// `counts` is T ints of scratch.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_validate(const int32_t* __restrict__ seg_start,
                                                   const int32_t* __restrict__ seg_adapter,
                                                   const int32_t* __restrict__ seg_rank,
                                                   const int32_t* __restrict__ token_index, int T,
                                                   int S, PoolView pv, int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ result) {
  __shared__ int meta_bad;
  __shared__ int first_bad;  // 2*s + (0 adapter | 1 rank)
  const int tid = threadIdx.x;
  if (tid == 0) {
    meta_bad = (seg_start[0] != 0 || seg_start[S] != T) ? 1 : 0;
    first_bad = 0x7fffffff;
  }
  if (token_index)
    for (int i = tid; i < T; i += blockDim.x) counts[i] = 0;
  __syncthreads();
  for (int s = tid; s < S; s += blockDim.x)
    if (seg_start[s + 1] < seg_start[s]) atomicOr(&meta_bad, 1);
  if (token_index) {
    for (int p = tid; p < T; p += blockDim.x) {
      int t = token_index[p];
      if (t < 0 || t >= T) atomicOr(&meta_bad, 1);
      else atomicAdd(&counts[t], 1);
    }
    __threadfence_block();
    __syncthreads();
    for (int i = tid; i < T; i += blockDim.x)
      if (counts[i] != 1) atomicOr(&meta_bad, 1);
  }
  for (int s = tid; s < S; s += blockDim.x) {
    const int a = seg_adapter[s];
    if (a == -1) continue;
    if (a < -1 || a >= pv.capacity || pv.rank[a] <= 0) {
      atomicMin(&first_bad, 2 * s);
    } else if (seg_rank && seg_rank[s] != pv.rank[a]) {
      atomicMin(&first_bad, 2 * s + 1);
    }
  }
  __syncthreads();
  if (tid == 0) {
    int st = MLORA_OK;
    if (meta_bad) st = MLORA_ERR_METADATA;
    else if (first_bad != 0x7fffffff) st = (first_bad & 1) ? MLORA_ERR_RANK : MLORA_ERR_ADAPTER;
    result[0] = st;
  }
}

void launch_validate(const int32_t* seg_start, const int32_t* seg_adapter, const int32_t* seg_rank,
                     const int32_t* token_index, int T, int S, const PoolView& pv, int32_t* counts,
                     int32_t* result, hipStream_t st) {
  hipLaunchKernelGGL(k_validate, dim3(1), dim3(1024), 0, st, seg_start, seg_adapter, seg_rank,
                     token_index, T, S, pv, counts, result);
}

// ---------------------------------------------------------------------------
// Small fills (used instead of memset so the calls stay capturable)
// ---------------------------------------------------------------------------
__global__ void k_fill_u32(uint32_t* __restrict__ p, size_t n, uint32_t v) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

void launch_fill_u32(void* p, size_t n_words, uint32_t v, hipStream_t st) {
  if (n_words == 0) return;
  size_t blocks = (n_words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)blocks), dim3(256), 0, st, (uint32_t*)p, n_words, v);
}

__global__ void k_set_slot_rank(int32_t* __restrict__ table, int id, int rank) { table[id] = rank; }

void launch_set_slot_rank(int32_t* table, int id, int rank, hipStream_t st) {
  hipLaunchKernelGGL(k_set_slot_rank, dim3(1), dim3(1), 0, st, table, id, rank);
}

}  // namespace mlora
