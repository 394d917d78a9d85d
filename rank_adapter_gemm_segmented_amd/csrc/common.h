// common.h -- device-side types and helpers shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlora {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// fp32 -> bf16 bits, round to nearest even (NaN -> quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Pack 8 floats into a bf16x8 operand (RNE).
__device__ __forceinline__ bf16x8_t pack_bf16x8(const float* v) {
  u32x4_t r;
  r.x = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
  r.y = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
  r.z = (uint32_t)f32_to_bf16_bits(v[4]) | ((uint32_t)f32_to_bf16_bits(v[5]) << 16);
  r.w = (uint32_t)f32_to_bf16_bits(v[6]) | ((uint32_t)f32_to_bf16_bits(v[7]) << 16);
  return __builtin_bit_cast(bf16x8_t, r);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ u32x4_t zero_u32x4() { return u32x4_t{0u, 0u, 0u, 0u}; }

// 16-byte global load (streamed data: non-temporal hint).
__device__ __forceinline__ u32x4_t ld_nt16(const void* p) {
  return __builtin_nontemporal_load((const u32x4_t*)p);
}
__device__ __forceinline__ u32x4_t ld16(const void* p) { return *(const u32x4_t*)p; }

// Element offset of B[n][j] in a bf16 slot's B region. Rank columns are
// stored in blocks of 16: block b holds columns 16 b .. 16 b + 15 of every
// row, [d_out][16] contiguous, so one block's columns over 32 consecutive
// rows are 1 KB of consecutive bytes (an MFMA operand load of 32 rows then
// touches 8 cache lines, not one per row). Columns past a rank are zero.
__device__ __forceinline__ long long bblk_off(int n, int j, int d_out) {
  return ((long long)(j >> 4) * d_out + n) * 16 + (j & 15);
}

// p where cond holds, else alt, chosen with integer masks. A pointer select
// on a per-lane condition may be compiled into divergent branches, whose
// join waits for every load in flight; this form stays one vector select.
// The address not chosen is never dereferenced.
__device__ __forceinline__ const void* sel_addr(bool cond, const void* p, const void* alt) {
  const unsigned long long m = 0ull - (unsigned long long)cond;
  return (const void*)(((unsigned long long)p & m) | ((unsigned long long)alt & ~m));
}

// Segment containing sorted position p: largest s in [0, n_seg) with
// seg_start[s] <= p (binary search; seg_start assumed non-decreasing). Returns
// a value in [0, n_seg-1] for any p, so callers must still check
// seg_start[s] <= p < seg_start[s+1].
__device__ __forceinline__ int find_segment(const int32_t* __restrict__ seg_start, int n_seg, int p) {
  int lo = 0, hi = n_seg - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (seg_start[mid] <= p) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ int round_up8(int r) { return (r + 7) & ~7; }

// Workgroup barrier for LDS data only: waits for this wave's LDS (and scalar)
// operations, not for its outstanding global loads, which __syncthreads
// would wait for too. The memory clobber keeps the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

constexpr int kZeroBlockElems = 2048;   // bf16 elements in the pool's zero block (4 KB)

// Everything a kernel needs to find an adapter in the pool.
struct PoolView {
  const void* base;        // slot 0
  const void* zeros;       // 4 KB of zeros (read in place of absent operands)
  const int32_t* rank;     // registered rank per slot (device table)
  long long slot_elems;    // elements per slot
  long long b_offset;      // element offset of B inside a slot (= max_rank * d_in)
  int capacity;
  int max_rank;
  // Stacked projections (a pool of fused adapters): W's rows fall into
  // n_slices slices ending at slice_end[m]; an adapter of rank R holds slice
  // m's rank columns [m R / n_slices, (m + 1) R / n_slices) and zeros
  // elsewhere in those rows. n_slices = 0: no slicing (or slices of unequal
  // rank), every rank column may be nonzero.
  int n_slices;
  int slice_end[8];
};

// Rank columns [*w0, *w1) that can be nonzero in rows [r0, r1) for an
// adapter of rank R: one slice's window when the rows lie inside one slice,
// else all of [0, R).
__device__ __forceinline__ void slice_window(const PoolView& pv, int r0, int r1, int R, int* w0, int* w1) {
  *w0 = 0;
  *w1 = R;
  int start = 0;
  for (int m = 0; m < pv.n_slices && m < 8; ++m) {
    const int end = pv.slice_end[m];
    if (r0 >= start && r1 <= end) {
      const int rs = R / pv.n_slices;
      *w0 = m * rs;
      *w1 = (m + 1) * rs;
      return;
    }
    start = end;
  }
}

// Metadata of one call over sorted positions.
struct SegView {
  const int32_t* seg_start;    // [n_seg + 1]
  const int32_t* seg_adapter;  // [n_seg]
  const int32_t* seg_rank;     // [n_seg]
  const float* seg_scale;      // [n_seg]
  const int32_t* token_index;  // [T] or null
  const int32_t* n_seg_dev;    // device segment count, or null (use n_seg)
  int n_seg;                   // host segment count (upper bound when n_seg_dev is set)
};

__device__ __forceinline__ int seg_count(const SegView& sv) {
  if (sv.n_seg_dev) {
    int s = *sv.n_seg_dev;
    return s < 0 ? 0 : (s > sv.n_seg ? sv.n_seg : s);
  }
  return sv.n_seg;
}

// Adapter of segment s after clamping: returns -1 for base-only, for any id
// the pool cannot serve and for an empty (unregistered) slot; *rank receives
// min(seg_rank, registered rank), so a lying rank never reads past the
// registered adapter (0 when -1 is returned).
__device__ __forceinline__ int seg_adapter_checked(const SegView& sv, const PoolView& pv, int s, int* rank) {
  const int a = sv.seg_adapter[s];
  const int r = sv.seg_rank ? sv.seg_rank[s] : 0;
  *rank = 0;
  if (a < 0 || a >= pv.capacity || r <= 0) return -1;
  const int rs = pv.rank[a];
  if (rs <= 0) return -1;
  *rank = r < rs ? r : rs;
  return a;
}

}  // namespace mlora
