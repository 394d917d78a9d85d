// kernels_meta.hip -- segment metadata kernels for gfx950.
//
// The batch is split into segments, one adapter each (the "InvisibleLoRA"
// abstract divides a batch's requests among the adapters in use). Requests of the
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
// scan over "segment starts" numbers the segments.
//
// Latency: every global load happens up front (ids, then each token's
// registered rank and scale); the sort, the segment flags and the scan stay in
// LDS (one wave-level scan, one cross-wave step). The rank and scale loads stay
// in flight through the stable count (its barrier waits for LDS only) and land
// in LDS just before the segment phase, which is their first use.
//
// The count is O(T^2) compares, so it is laid out for the vector ALUs: a wave
// takes 64 consecutive tokens (one per lane) against a range of the other
// tokens u, read as 4 ids per 16-byte LDS read at a wave-uniform address
// (a broadcast). Every u below the wave's 64 tokens precedes each of them, so
// it counts when id[u] <= id[t]; every u above them counts when id[u] < id[t];
// only the 64 u of the wave's own tokens need the full test. With few tokens
// the u range is split over several waves whose counts are added in LDS.
// ---------------------------------------------------------------------------
constexpr int kSegThreads = 1024;
constexpr int kSegWaves = kSegThreads / kWave;
constexpr int kSegPerThread = MLORA_MAX_UNSORTED_TOKENS / kSegThreads;   // tokens per thread (8)

__device__ __forceinline__ int count_le4(int4 o, int k) { return (o.x <= k) + (o.y <= k) + (o.z <= k) + (o.w <= k); }
__device__ __forceinline__ int count_lt4(int4 o, int k) { return (o.x < k) + (o.y < k) + (o.z < k) + (o.w < k); }

__global__ __launch_bounds__(kSegThreads) void k_build_segments(
    const int32_t* __restrict__ token_adapter, const float* __restrict__ adapter_scale, int T,
    PoolView pv, int32_t* __restrict__ token_index, int32_t* __restrict__ seg_start,
    int32_t* __restrict__ seg_adapter, int32_t* __restrict__ seg_rank,
    float* __restrict__ seg_scale, int32_t* __restrict__ n_seg_out) {
  // LDS: ids [Tp] (batch order, padded to a multiple of 4 with INT_MAX, which
  // no count includes), srt [T] (sorted position -> batch row), trk [T] and
  // tsc [T] (registered rank and scale of each batch row's adapter)
  extern __shared__ __attribute__((aligned(16))) int32_t sm[];
  const int Tp = (T + 3) & ~3;
  int32_t* ids = sm;
  int32_t* srt = sm + Tp;
  int32_t* trk = sm + Tp + T;
  float* tsc = (float*)(sm + Tp + 2 * T);
  __shared__ int wtot[kSegWaves];
  __shared__ int part[kSegThreads];   // per-range counts when the u range is split
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;

  // ---- ids, ranks, scales: token t = tid + kSegThreads * i -----------------
  int key[kSegPerThread];
#pragma unroll
  for (int i = 0; i < kSegPerThread; ++i) {
    const int t = tid + kSegThreads * i;
    key[i] = t < T ? token_adapter[t] : -1;
  }
  int rk[kSegPerThread];
  float sc[kSegPerThread];
#pragma unroll
  for (int i = 0; i < kSegPerThread; ++i) {
    const int t = tid + kSegThreads * i;
    const bool valid = key[i] >= 0 && key[i] < pv.capacity;
    rk[i] = valid ? pv.rank[key[i]] : 0;
    sc[i] = valid ? adapter_scale[key[i]] : 0.0f;
    if (t < T) ids[t] = key[i];
  }
  if (tid < Tp - T) ids[T + tid] = 0x7fffffff;
  lds_barrier();

  // ---- stable rank of every token ------------------------------------------
  // task q (wave-uniform): token group q % ntg (64 tokens), u range q / ntg of G
  const int ntg = (T + kWave - 1) / kWave;
  const int G = ntg >= kSegWaves ? 1 : kSegWaves / max(ntg, 1);
  const int q4 = Tp / 4;
  for (int q = wave; q < ntg * G; q += kSegWaves) {
    const int tg = q % ntg, g = q / ntg;
    const int t = tg * kWave + lane;
    const int k = t < T ? ids[t] : 0;
    const int ua = 4 * (int)((long long)q4 * g / G), ub = 4 * (int)((long long)q4 * (g + 1) / G);
    const int lo = tg * kWave, hi = min(lo + kWave, Tp);
    int pos = 0;
    for (int u = ua; u < min(ub, lo); u += 4) pos += count_le4(*(const int4*)&ids[u], k);
    for (int u = max(ua, lo); u < min(ub, hi); u += 4) {
      const int4 o = *(const int4*)&ids[u];
      // lane j's own token is u = lo + j: tokens of lower lanes precede it
      const int j = u - lo;
      pos += lane > j + 0 ? (o.x <= k) : (o.x < k);
      pos += lane > j + 1 ? (o.y <= k) : (o.y < k);
      pos += lane > j + 2 ? (o.z <= k) : (o.z < k);
      pos += lane > j + 3 ? (o.w <= k) : (o.w < k);
    }
    for (int u = max(ua, hi); u < ub; u += 4) pos += count_lt4(*(const int4*)&ids[u], k);
    if (G == 1) {
      if (t < T) {
        srt[pos] = t;
        token_index[pos] = t;
      }
    } else {
      part[g * ntg * kWave + t] = pos;   // G * ntg <= kSegWaves: within part
    }
  }
  if (G > 1) {   // uniform
    lds_barrier();
    if (tid < T) {   // T <= ntg * 64 <= kSegThreads / 2 here
      int pos = 0;
      for (int g = 0; g < G; ++g) pos += part[g * ntg * kWave + tid];
      srt[pos] = tid;
      token_index[pos] = tid;
    }
  }
#pragma unroll
  for (int i = 0; i < kSegPerThread; ++i) {
    const int t = tid + kSegThreads * i;
    if (t < T) {
      trk[t] = rk[i];
      tsc[t] = sc[i];
    }
  }
  __syncthreads();

  // ---- segment starts: thread owns positions [pb, pe) ----------------------
  const int chunk = (T + kSegThreads - 1) / kSegThreads;
  const int pb = min(tid * chunk, T), pe = min(pb + chunk, T);
  int cnt = 0;
  for (int p = pb; p < pe; ++p) cnt += (p == 0 || ids[srt[p]] != ids[srt[p - 1]]);
  int inc = cnt;   // inclusive scan: the wave, then the waves before it
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int up = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += up;
  }
  if (lane == kWave - 1) wtot[wave] = inc;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wtot[w];
  int s = before + inc - cnt;   // index of this thread's first new segment
  for (int p = pb; p < pe; ++p) {
    const int t = srt[p];
    if (p == 0 || ids[t] != ids[srt[p - 1]]) {
      seg_start[s] = p;
      seg_adapter[s] = ids[t];
      seg_rank[s] = trk[t];
      seg_scale[s] = tsc[t];
      ++s;
    }
  }
  if (tid == kSegThreads - 1) {   // the last thread holds the total
    seg_start[s] = T;
    n_seg_out[0] = s;
  }
}

size_t build_segments_lds_bytes(int T) { return (size_t)(((T + 3) & ~3) + 3 * T) * sizeof(int32_t); }

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
