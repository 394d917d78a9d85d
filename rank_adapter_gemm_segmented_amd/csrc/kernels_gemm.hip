// kernels_gemm.hip -- bf16 multi-LoRA linear for larger token counts on gfx950.
//
// y_i = W x_i + scale_s * B_a (A_a x_i) ("Multi-LoRA Serving in Practice",
// section "Core Principle", displayed formula), per adapter segment
// ("InvisibleLoRA" abstract). Two or three launches:
//
//  k_shrink2  v = A_a x per segment, fp32, split over d_in chunks into
//             deterministic partials; also writes a per-position table
//             {segment, adapter, rank, scale}; k_vfinal folds the partials in
//             chunk order and applies the scale (v_fin, read by the epilogue).
//             With a single chunk the shrink writes v_fin itself.
//             k_shrink_short replaces it on batches of one- or two-position
//             segments of rank <= 32 (vector-ALU dot products, real rows only).
//  k_gemm2    W x as a tiled GEMM on v_mfma_f32_32x32x16_bf16: block tile of
//             BR W rows x BT sorted positions over the whole of d_in, both
//             operands staged through LDS by direct-to-LDS loads (a ring of
//             NB W stages and one of NX position stages). The
//             epilogue adds scale * B_a v on the same accumulators with MFMAs
//             (v split into a bf16 high and low part, ~16 mantissa bits) and
//             stores y once, through an LDS transpose.
//
// MFMA 32x32x16 bf16 layout: lane l supplies row l%32 and k-slots 8*(l/32)..+7
// of each operand; result register v of lane l is row 8*(v/4)+4*(l/32)+v%4,
// column l%32. The A operand is W (rows = output features) and the B operand
// is x (columns = tokens), so each lane ends with runs of 4 consecutive
// features of one token.
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace mlora {

__device__ __forceinline__ f32x4_t mfma16g(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma32g(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Shrink. grid (items, d_in chunks), 4 waves. An item is one block of 16 NRB
// positions (one pass) of one segment times one group of 16 NCB rank rows
// (longer segments or higher ranks give several items, so neither a long
// segment nor a rank-64 adapter leaves one workgroup streaming all of its A);
// each workgroup finds its item with a scan of the segment starts in LDS,
// where the segments' adapter ids and ranks are loaded in the same round, so
// the A loads can start right after the scan (the pool's slot table is read
// alongside and only decides the per-position table). Chunk c covers k-steps
// [c*nks/ks, (c+1)*nks/ks) of 32; wave w takes every fourth k-step starting
// at w. A k-step loads NRB position blocks of x and NC <= NCB rank blocks of
// A (16 each): 16 / (NRB + NC) k-steps of operands in flight in registers (at
// most 64 operand VGPRs). Absent operands read the pool's zero block (every
// load is unconditional, no loaded value is selected). The four waves are
// summed in a fixed order through LDS into v_part[c][p][j] (unscaled). MFMA
// rows = positions, columns = rank index.
// ---------------------------------------------------------------------------
constexpr int kShrMaxSeg = MLORA_MAX_SEGMENTS;  // segments the item scan handles
constexpr int kShrMaxSplit = 4;                 // d_in chunks of the MFMA shrink at most
constexpr int kShrLdsSeg = 4096;                // up to this many, adapters and ranks go to LDS too

// Whether the shrinks keep the segments' adapters and ranks in LDS next to
// the starts. Decided from the host's segment bound (sv.n_seg), never from a
// device count, so the kernels' LDS layout and the host's allocation
// (shrink_lds_bytes) always agree.
__host__ __device__ __forceinline__ bool shrink_meta_in_lds(int n_seg_bound) {
  return (n_seg_bound < kShrMaxSeg ? n_seg_bound : kShrMaxSeg) <= kShrLdsSeg;
}

// Dynamic LDS of a shrink launch: starts [S + 1] and, by the rule above,
// adapters [S] and ranks [S], for S = the host's bound. The device count,
// when there is one, never exceeds it.
static size_t shrink_lds_bytes(int n_seg_bound) {
  const int nseg = n_seg_bound < kShrMaxSeg ? n_seg_bound : kShrMaxSeg;
  return (size_t)(shrink_meta_in_lds(n_seg_bound) ? 3 * nseg + 1 : nseg + 1) * sizeof(int);
}

template <int NRB, int NCB>
__global__ __launch_bounds__(256) void k_shrink2(LinearArgs a) {
  constexpr int NQ = NRB * NCB * 4;     // accumulator floats per lane
  const int item = blockIdx.x, c = blockIdx.y;
  const SegView& sv = a.sv;
  const int S = min(seg_count(sv), kShrMaxSeg);
  const int T = a.T, d_in = a.d_in;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  // segment starts [S + 1], and the adapters [S] and ranks [S] when the
  // host's segment bound is at most kShrLdsSeg. The choice follows the host
  // bound, the count the host sized the dynamic LDS from (shrink_lds_bytes):
  // with device-built segments S is read on the device and may be smaller
  // than the bound, and a layout chosen from S could outgrow the allocation.
  extern __shared__ int sdyn[];
  const bool meta_lds = shrink_meta_in_lds(sv.n_seg);
  int* sst = sdyn;
  int* sad = sdyn + S + 1;
  int* srk = sdyn + 2 * S + 1;
  __shared__ int wsum[4];
  __shared__ int found[2];
  __shared__ float red[4][kWave][NQ + 1];

  // ---- which (segment, block) is this item? --------------------------------
  // All of a round's loads are issued before its LDS stores: the metadata
  // pointers are generic, so a store placed between them would make every
  // load wait for the one before it.
  for (int i0 = 0; i0 <= S; i0 += 256) {
    const int i = i0 + tid;
    const bool in = i <= S, meta = meta_lds && i < S;
    const int st = in ? sv.seg_start[i] : 0;
    const int ad = meta ? sv.seg_adapter[i] : 0;
    const int rk = meta && sv.seg_rank ? sv.seg_rank[i] : 0;
    if (in) sst[i] = st;
    if (meta) {
      sad[i] = ad;
      srk[i] = rk;
    }
  }
  if (tid == 0) found[0] = -1;
  __syncthreads();
  // items of segment i: its blocks of 16 NRB positions (one pass each) times
  // its groups of 16 NCB rank rows (at least one, which also writes the
  // position table)
  constexpr int PB = 16 * NRB;
  auto n_items = [&](int i) {
    const int len = min(sst[i + 1], T) - max(sst[i], 0);
    if (len <= 0) return 0;
    const int ad = meta_lds ? sad[i] : sv.seg_adapter[i];
    const int rk = meta_lds ? srk[i] : (sv.seg_rank ? sv.seg_rank[i] : 0);
    const int ra = ad >= 0 && ad < a.pv.capacity ? min(max(rk, 0), a.pv.max_rank) : 0;
    return (len + PB - 1) / PB * max((ra + 16 * NCB - 1) / (16 * NCB), 1);
  };
  const int per = (S + 255) / 256;
  int cnt = 0;
  for (int i = tid * per; i < min(S, tid * per + per); ++i) cnt += n_items(i);
  int inc = cnt;   // inclusive scan: wave, then the waves before it
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int up = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += up;
  }
  if (lane == kWave - 1) wsum[wave] = inc;
  __syncthreads();
  for (int w = 0; w < wave; ++w) inc += wsum[w];
  {
    const int lo = inc - cnt;   // items before this thread's segments
    if (item >= lo && item < inc) {
      int acc = lo;
      for (int i = tid * per; i < min(S, tid * per + per); ++i) {
        const int nb = n_items(i);
        if (item < acc + nb) {
          found[0] = i;
          found[1] = item - acc;
          break;
        }
        acc += nb;
      }
    }
  }
  __syncthreads();
  const int s = found[0];
  if (s < 0) return;   // uniform: past the last item
  // adapter and A rows to read: the segment's own id and rank, clamped into
  // the pool; the slot table (registration) is applied to the position table
  const int ad0 = meta_lds ? sad[s] : sv.seg_adapter[s];
  const int rk0 = meta_lds ? srk[s] : (sv.seg_rank ? sv.seg_rank[s] : 0);
  const bool adok = ad0 >= 0 && ad0 < a.pv.capacity;
  const int ra = adok ? min(max(rk0, 0), a.pv.max_rank) : 0;
  const int ng = max((ra + 16 * NCB - 1) / (16 * NCB), 1);   // rank groups of the segment
  const int pb = found[1] / ng, grp = found[1] % ng;
  const int ps = max(sst[s], 0) + PB * pb;
  const int pe = min(min(sst[s + 1], T), ps + PB);
  const int jg0 = 16 * NCB * grp;                  // this item's rank rows [jg0, jg1)
  const int jg1 = min(ra, jg0 + 16 * NCB);
  // The registered rank and the scale are only needed once the first sums
  // exist. Their loads are vector loads (offset vz is zero but held in a
  // vector register; a scalar load's wait would come with the next LDS wait),
  // issued now and consumed after the first k-loop (the asm pins their use
  // there), so the A and x loads do not wait behind them.
  int vz;
  asm volatile("v_mov_b32 %0, 0" : "=v"(vz));
  int reg_rank = a.pv.rank[(adok ? ad0 : 0) + vz];
  float scl = sv.seg_scale[s + vz];
  int r_eff = 0;   // rank the expand applies: the segment's, capped by the registered one
  auto resolve = [&]() {
    asm volatile("" : "+v"(reg_rank), "+v"(scl));
    r_eff = adok && reg_rank > 0 && ra > 0 ? min(ra, reg_rank) : 0;
  };
  // With one d_in chunk (ks == 1) the sum is final: this kernel writes
  // v_fin = scale * v itself (zero past r_eff, up to the row pitch) and no
  // finalize launch follows.
  const bool fused = a.ks == 1;
  auto write_pos = [&]() {
    if (c != 0 || grp != 0) return;   // once per position block
    resolve();
    const int ad = r_eff > 0 ? ad0 : -1;
    for (int p = ps + tid; p < pe; p += 256) a.pos_info[p] = make_int4(s, ad, r_eff, __float_as_int(r_eff > 0 ? scl : 0.f));
    if (fused) {   // v_fin columns [ra, r_ws) of the item's positions
      const int nz = a.r_ws - ra;
      for (int e = tid; e < (pe - ps) * nz; e += 256) a.v_fin[(long long)(ps + e / nz) * a.r_ws + ra + e % nz] = 0.f;
    }
  };
  if (ra == 0) {
    write_pos();
    return;
  }

  const uint16_t* __restrict__ x = (const uint16_t*)a.x;
  const uint16_t* __restrict__ Aa = (const uint16_t*)a.pv.base + (long long)ad0 * a.pv.slot_elems;
  const uint16_t* zeros = (const uint16_t*)a.pv.zeros;
  const int nks = (d_in + 31) / 32;
  const int kb = (int)((long long)c * nks / a.ks);
  const int ke = (int)((long long)(c + 1) * nks / a.ks);
  const int nst = (ke - kb - wave + 3) / 4;            // this wave's k-steps
  const int nst_w = (ke - kb + 3) / 4;                 // wave 0's (the most); uniform loop bound
  const int l16 = lane % 16, kq = 8 * (lane / 16);

  for (int pg = ps; pg < pe; pg += 16 * NRB) {
    // x rows of this position group (fixed over k); absent positions read zeros
    // (gathered rows: every index load is issued before any is used)
    const uint16_t* xrow[NRB];
    int prow[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) prow[rb] = min(pg + rb * 16 + l16, pe - 1);
    if (sv.token_index) {   // uniform
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) prow[rb] = sv.token_index[prow[rb]];
    }
    bool xok[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int p = pg + rb * 16 + l16;
      const int row = min(max(prow[rb], 0), T - 1);
      xrow[rb] = x + (long long)row * d_in;
      xok[rb] = p < pe;
    }
    const int nrb = min(NRB, (pe - pg + 15) / 16);
    for (int jg = jg0; jg < jg1; jg += 16 * NCB) {   // (one pass: the item's rank group)
      const int ncb = min(NCB, (jg1 - jg + 15) / 16);
      // one pass over rank columns [jg, jg + 16 NC): NC column blocks of 16
      // A rows are loaded per k-step. The pass takes the smallest NC that
      // holds the segment's rows, so a low-rank segment in a pool of a high
      // max rank loads no zero blocks for its absent rows and keeps a deeper
      // ring (DD k-steps in flight).
      auto pass = [&](auto nc_tag) {
        constexpr int NC = decltype(nc_tag)::value;
        constexpr int DD = 16 / (NRB + NC);
        const int nst_pd = (nst_w + DD - 1) / DD * DD;
        const uint16_t* arow[NC];
        bool aok[NC];
#pragma unroll
        for (int cb = 0; cb < NC; ++cb) {
          const int j = jg + cb * 16 + l16;
          arow[cb] = Aa + (long long)min(j, jg1 - 1) * d_in;
          aok[cb] = j < jg1;
        }
        f32x4_t acc[NRB][NC];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
          for (int cb = 0; cb < NC; ++cb) acc[rb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        u32x4_t af[DD][NC], xf[DD][NRB];
        auto load = [&](int slot, int i) {   // this wave's i-th k-step
          const int k = (kb + wave + 4 * i) * 32 + kq;
          const bool kin = i < nst && k < d_in;
#pragma unroll
          for (int cb = 0; cb < NC; ++cb) af[slot][cb] = ld16(sel_addr(kin && aok[cb], arow[cb] + k, zeros + kq));
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) xf[slot][rb] = ld16(sel_addr(kin && xok[rb], xrow[rb] + k, zeros + kq));
        };
#pragma unroll
        for (int u = 0; u < DD; ++u) load(u, u);
        for (int i0 = 0; i0 < nst_pd; i0 += DD) {
#pragma unroll
          for (int u = 0; u < DD; ++u) {
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
              for (int cb = 0; cb < NC; ++cb)
                if (rb < nrb && cb < ncb) acc[rb][cb] = mfma16g(xf[u][rb], af[u][cb], acc[rb][cb]);
            load(u, i0 + u + DD);   // past the end: zero-block reads
          }
        }
        resolve();
        // fixed-order sum of the four waves, spread over all threads: entry
        // e = (q, l) is accumulator value q of lane l
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
          for (int cb = 0; cb < NC; ++cb)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[wave][lane][(rb * NC + cb) * 4 + v] = acc[rb][cb][v];
        __syncthreads();
        for (int e = tid; e < NRB * NC * 4 * kWave; e += 256) {
          const int q = e / kWave, l = e % kWave;
          const int rb = q / (NC * 4), cb = (q / 4) % NC, v = q % 4;
          if (rb < nrb && cb < ncb) {
            const float sum = ((red[0][l][q] + red[1][l][q]) + red[2][l][q]) + red[3][l][q];
            const int p = pg + rb * 16 + 4 * (l / 16) + v;
            const int j = jg + cb * 16 + (l % 16);
            if (p < pe && j < jg1) {
              if (fused) a.v_fin[(long long)p * a.r_ws + j] = j < r_eff ? scl * sum : 0.f;
              else a.v_part[((long long)c * T + p) * a.r_ws + j] = sum;
            }
          }
        }
        __syncthreads();
      };
      if constexpr (NCB >= 2) {
        if (ncb == 1) {   // uniform
          pass(std::integral_constant<int, 1>{});
          continue;
        }
      }
      if constexpr (NCB >= 4) {
        if (ncb == 2) {
          pass(std::integral_constant<int, 2>{});
          continue;
        }
      }
      pass(std::integral_constant<int, NCB>{});
    }
  }
  write_pos();
}

// ---------------------------------------------------------------------------
// Shrink for batches of short segments (a verify batch: a draft and a bonus
// token per request, each request with its own adapter), one d_in chunk.
// The MFMA shrink above spends most of its loads there on absent positions
// (a 16-position operand for one or two tokens). Here grid.y is the item, a
// block of up to kSsPos positions of one segment, and grid.x a group of
// kSsRows rank rows, so only real A rows and real tokens are read, and a
// rank-16 adapter's A is shared by two workgroups. Thread tid takes the 8-column
// groups tid, tid + 256, ... of d_in and accumulates kSsRows x kSsPos fp32
// dot products on the vector ALUs; the 256 threads' sums are then added
// through LDS in a fixed order (deterministic). Writes v_fin = scale * v and
// the position table, as the one-chunk MFMA shrink does.
// ---------------------------------------------------------------------------
constexpr int kSsPos = 2;      // positions per item (a verify request's two tokens; 4 took the
                               // verify LoRA-on call 0.6-0.9 us longer, 1 about 2 us longer)
constexpr int kSsRows = 8;     // rank rows per workgroup (4 measured the same, 16 slower)
constexpr int kSsMaxRank = 32; // largest pool rank it takes
constexpr int kSsUnroll = 2;   // column groups per thread whose loads are in flight together
constexpr int kSsPitch = 256 + 8;

__device__ __forceinline__ float dot8_bf16(u32x4_t a, u32x4_t b, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = fmaf(__uint_as_float(a[i] << 16), __uint_as_float(b[i] << 16), acc);
    acc = fmaf(__uint_as_float(a[i] & 0xffff0000u), __uint_as_float(b[i] & 0xffff0000u), acc);
  }
  return acc;
}

__global__ __launch_bounds__(256) void k_shrink_short(LinearArgs a) {
  // rank groups vary fastest, so the workgroups of real items come first and
  // spread one per CU
  const int g = blockIdx.x, item = blockIdx.y;
  const SegView& sv = a.sv;
  const int S = min(seg_count(sv), kShrMaxSeg);
  const int T = a.T, d_in = a.d_in;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  extern __shared__ int sdyn[];
  const bool meta_lds = shrink_meta_in_lds(sv.n_seg);   // same rule as k_shrink2
  int* sst = sdyn;
  int* sad = sdyn + S + 1;
  int* srk = sdyn + 2 * S + 1;
  __shared__ int wsum[4];
  __shared__ int found[2];
  __shared__ float red[kSsRows * kSsPos][kSsPitch];

  // ---- which (segment, block) is this item? (as in k_shrink2, blocks of kSsPos)
  for (int i0 = 0; i0 <= S; i0 += 256) {
    const int i = i0 + tid;
    const bool in = i <= S, meta = meta_lds && i < S;
    const int st = in ? sv.seg_start[i] : 0;
    const int ad = meta ? sv.seg_adapter[i] : 0;
    const int rk = meta && sv.seg_rank ? sv.seg_rank[i] : 0;
    if (in) sst[i] = st;
    if (meta) {
      sad[i] = ad;
      srk[i] = rk;
    }
  }
  if (tid == 0) found[0] = -1;
  __syncthreads();
  const int per = (S + 255) / 256;
  int cnt = 0;
  for (int i = tid * per; i < min(S, tid * per + per); ++i) {
    const int len = min(sst[i + 1], T) - max(sst[i], 0);
    cnt += len > 0 ? (len + kSsPos - 1) / kSsPos : 0;
  }
  int inc = cnt;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int up = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += up;
  }
  if (lane == kWave - 1) wsum[wave] = inc;
  __syncthreads();
  for (int w = 0; w < wave; ++w) inc += wsum[w];
  {
    const int lo = inc - cnt;
    if (item >= lo && item < inc) {
      int acc = lo;
      for (int i = tid * per; i < min(S, tid * per + per); ++i) {
        const int len = min(sst[i + 1], T) - max(sst[i], 0);
        const int nb = len > 0 ? (len + kSsPos - 1) / kSsPos : 0;
        if (item < acc + nb) {
          found[0] = i;
          found[1] = item - acc;
          break;
        }
        acc += nb;
      }
    }
  }
  __syncthreads();
  const int s = found[0];
  if (s < 0) return;   // uniform: past the last item
  const int ps = max(sst[s], 0) + kSsPos * found[1];
  const int pe = min(min(sst[s + 1], T), ps + kSsPos);
  const int np = pe - ps;
  const int ad0 = meta_lds ? sad[s] : sv.seg_adapter[s];
  const int rk0 = meta_lds ? srk[s] : (sv.seg_rank ? sv.seg_rank[s] : 0);
  const bool adok = ad0 >= 0 && ad0 < a.pv.capacity;
  const int ra = adok ? min(max(rk0, 0), a.pv.max_rank) : 0;
  const int j0 = kSsRows * g;
  const int nr = min(kSsRows, ra - j0);   // rows of this workgroup (<= 0: none)

  const uint16_t* __restrict__ x = (const uint16_t*)a.x;
  const uint16_t* __restrict__ Aa = (const uint16_t*)a.pv.base + (long long)(adok ? ad0 : 0) * a.pv.slot_elems;
  const uint16_t* arow[kSsRows];
#pragma unroll
  for (int r = 0; r < kSsRows; ++r) arow[r] = Aa + (long long)(j0 + min(r, max(nr - 1, 0))) * d_in;
  int prow[kSsPos];
#pragma unroll
  for (int t = 0; t < kSsPos; ++t) prow[t] = min(ps + t, pe - 1);
  if (sv.token_index) {   // uniform
#pragma unroll
    for (int t = 0; t < kSsPos; ++t) prow[t] = sv.token_index[prow[t]];
  }
  const uint16_t* xrow[kSsPos];
#pragma unroll
  for (int t = 0; t < kSsPos; ++t) xrow[t] = x + (long long)min(max(prow[t], 0), T - 1) * d_in;
  // the registered rank and the scale are needed at the end only: vector
  // loads (offset vz is zero but held in a vector register), consumed after
  // the dot products, so the A and x loads do not wait behind them
  int vz;
  asm volatile("v_mov_b32 %0, 0" : "=v"(vz));
  int reg_rank = a.pv.rank[(adok ? ad0 : 0) + vz];
  float scl = sv.seg_scale[s + vz];
  // position table and v_fin columns [ra, r_ws) of the item's positions
  auto write_pos = [&]() {
    asm volatile("" : "+v"(reg_rank), "+v"(scl));
    const int r_eff = adok && reg_rank > 0 && ra > 0 ? min(ra, reg_rank) : 0;
    if (g != 0) return r_eff;
    const int ad = r_eff > 0 ? ad0 : -1;
    for (int p = ps + tid; p < pe; p += 256) a.pos_info[p] = make_int4(s, ad, r_eff, __float_as_int(r_eff > 0 ? scl : 0.f));
    const int nz = a.r_ws - ra;
    for (int e = tid; e < np * nz; e += 256) a.v_fin[(long long)(ps + e / nz) * a.r_ws + ra + e % nz] = 0.f;
    return r_eff;
  };
  if (nr <= 0) {   // uniform
    write_pos();
    return;
  }

  // ---- dot products over the thread's column groups --------------------------
  float acc[kSsRows][kSsPos];
#pragma unroll
  for (int r = 0; r < kSsRows; ++r)
#pragma unroll
    for (int t = 0; t < kSsPos; ++t) acc[r][t] = 0.f;
  const int ncg = d_in / 8;
  for (int cg0 = tid; cg0 < ncg; cg0 += 256 * kSsUnroll) {
    u32x4_t av[kSsUnroll][kSsRows], xv[kSsUnroll][kSsPos];
#pragma unroll
    for (int u = 0; u < kSsUnroll; ++u) {
      const int cg = cg0 + 256 * u;
      const int col = 8 * (cg < ncg ? cg : cg0);
#pragma unroll
      for (int r = 0; r < kSsRows; ++r) av[u][r] = r < nr ? ld16(arow[r] + col) : zero_u32x4();
#pragma unroll
      for (int t = 0; t < kSsPos; ++t) xv[u][t] = t < np ? ld16(xrow[t] + col) : zero_u32x4();
    }
#pragma unroll
    for (int u = 0; u < kSsUnroll; ++u)
      if (cg0 + 256 * u < ncg) {
#pragma unroll
        for (int r = 0; r < kSsRows; ++r)
#pragma unroll
          for (int t = 0; t < kSsPos; ++t) acc[r][t] = dot8_bf16(av[u][r], xv[u][t], acc[r][t]);
      }
  }

  // ---- fixed-order sum over the 256 threads -----------------------------------
  // output o = r * kSsPos + t; TPO threads per output each add 256 / TPO
  // partials (columns q, q + TPO, ...), then the TPO sums are combined by a
  // shuffle tree
  constexpr int NO = kSsRows * kSsPos;
  constexpr int TPO = 256 / NO;
  static_assert(NO * TPO == 256 && TPO >= 1 && TPO <= kWave, "outputs must divide the workgroup");
#pragma unroll
  for (int r = 0; r < kSsRows; ++r)
#pragma unroll
    for (int t = 0; t < kSsPos; ++t) red[r * kSsPos + t][tid] = acc[r][t];
  __syncthreads();
  const int o = tid / TPO, q = tid % TPO;
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 256 / TPO; ++i) sum += red[o][q + TPO * i];
#pragma unroll
  for (int off = 1; off < TPO; off <<= 1) sum += __shfl_xor(sum, off, TPO);
  const int r_eff = write_pos();
  const int r = o / kSsPos, t = o % kSsPos;
  if (q == 0 && r < nr && t < np) {
    const int j = j0 + r;
    a.v_fin[(long long)(ps + t) * a.r_ws + j] = j < r_eff ? scl * sum : 0.f;
  }
}

// ---------------------------------------------------------------------------
// Finalize: v_fin[p][j] = scale_p * sum_c v_part[c][p][j] (chunk order) for
// j < rank_p, else 0. One thread per 4 rank columns of one position; all the
// chunk loads are in flight at once. Every row tile of the GEMM then reads
// one v per position instead of re-reading the chunk partials.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_vfinal(LinearArgs a) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int q4 = a.r_ws / 4;
  if (e >= a.T * q4) return;
  const int p = e / q4, j = 4 * (e % q4);
  // the chunk partials are requested together with the position entry (their
  // addresses do not depend on it), not after it
  f32x4_t part[kMaxShrinkSplit];
#pragma unroll
  for (int c = 0; c < kMaxShrinkSplit; ++c)
    part[c] = *(const f32x4_t*)(a.v_part + ((long long)min(c, a.ks - 1) * a.T + p) * a.r_ws + j);
  const int4 pi = a.pos_info[p];
  const int rk = (pi.y >= 0 && pi.y < a.pv.capacity) ? min(pi.z, a.pv.max_rank) : 0;
  f32x4_t sum = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (j < rk) {
#pragma unroll
    for (int c = 0; c < kMaxShrinkSplit; ++c)
      if (c < a.ks) {
        sum[0] += part[c][0];
        sum[1] += part[c][1];
        sum[2] += part[c][2];
        sum[3] += part[c][3];
      }
    const float sc = __int_as_float(pi.w);
#pragma unroll
    for (int i = 0; i < 4; ++i) sum[i] = (j + i < rk) ? sum[i] * sc : 0.f;
  }
  *(f32x4_t*)(a.v_fin + (long long)p * a.r_ws + j) = sum;
}

// ---------------------------------------------------------------------------
// Adapter term as a dense fp32 tile, for batches of many short segments of
// mixed rank: delta[p][n] = sum over j < r of B_a[n][j] * v_fin[p][j] for
// every sorted position p whose table entry names an adapter, and zero for
// every other position below T. One workgroup per (position, block of
// kDxRows rows). L lanes share a row (L = the row's 16-byte chunks, rounded
// up to a power of two: 1, 2, 4 or 8), lane c taking chunk c (columns
// 8c .. 8c + 7), so a load instruction covers 64 / L whole rows, each block
// of 16 columns contiguous over them; the L partial sums of a row are added
// in a fixed order
// (xor partners 1, 2, 4). All of a workgroup's B loads are in flight before
// its first product. The position's v row, the same for every thread,
// passes through LDS. Both the padding of B past the rank and v_fin past it
// are zero, so whole chunks are multiplied. The tiled GEMM adds delta to its
// accumulators before the single rounding of y.
// ---------------------------------------------------------------------------
// One wave per workgroup, 64 rows: on the heterogeneous batch the LoRA-on
// call took 77.6 us, against 77.8 with 128 rows on 128 threads, 78.6 with 256
// on 256, 81.0 with 512 on 256 and 84.0 with 1024 on 256 (same bits). Small
// workgroups spread each position's rows over more CUs.
constexpr int kDxRows = 64;      // rows per workgroup
constexpr int kDxThreads = 64;   // threads per workgroup
static_assert(kDxRows % kDxThreads == 0 && kDxThreads >= kDxMaxRank / 4,
              "whole passes at every L; the threads that stage the v row exist");

template <int L>
__device__ __forceinline__ void expand_rows(const LinearArgs& a, const uint16_t* bslot, int pitch, int n_base,
                                            f32x4_t vq, bool vt, float* vs, float* __restrict__ drow) {
  constexpr int RP = kDxThreads / L;                 // rows per pass
  constexpr int NP = kDxRows / RP;                   // passes
  const int tid = threadIdx.x, c = tid % L, ro = tid / L;
  const bool c_ok = 8 * c < pitch;
  const uint16_t* zeros = (const uint16_t*)a.pv.zeros;
  u32x4_t b[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const int n = n_base + k * RP + ro;
    // chunks past the row's pitch and rows past d_out read the zero block
    b[k] = ld16(c_ok && n < a.d_out ? bslot + bblk_off(n, 8 * c, a.d_out) : zeros);
  }
  if (vt) *(f32x4_t*)&vs[4 * tid] = vq;              // waits for the v row alone
  __syncthreads();
  const f32x4_t v0 = c_ok ? *(const f32x4_t*)&vs[8 * c] : f32x4_t{0.f, 0.f, 0.f, 0.f};
  const f32x4_t v1 = c_ok ? *(const f32x4_t*)&vs[8 * c + 4] : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t wd = b[k][e / 2];
      const float bv = __uint_as_float((e & 1) ? (wd & 0xffff0000u) : (wd << 16));
      s = fmaf(bv, e < 4 ? v0[e] : v1[e - 4], s);
    }
    if constexpr (L > 1) s += __shfl_xor(s, 1, L);
    if constexpr (L > 2) s += __shfl_xor(s, 2, L);
    if constexpr (L > 4) s += __shfl_xor(s, 4, L);
    const int n = n_base + k * RP + ro;
    if (c == 0 && n < a.d_out) drow[n] = s;
  }
}

__global__ __launch_bounds__(kDxThreads) void k_expand_delta(LinearArgs a) {
  __shared__ __attribute__((aligned(16))) float vs[kDxMaxRank];
  const int p = blockIdx.y, tid = threadIdx.x;
  const int n_base = blockIdx.x * kDxRows;
  float* __restrict__ drow = a.delta + (long long)p * a.d_out;
  const int4 pi = a.pos_info[p];
  const bool live = pi.y >= 0 && pi.y < a.pv.capacity && pi.z > 0;
  if (!live) {                                        // uniform: a zero term
    for (int n = n_base + tid; n < min(n_base + kDxRows, a.d_out); n += kDxThreads) drow[n] = 0.f;
    return;
  }
  const int r = min(min(pi.z, a.pv.max_rank), kDxMaxRank);
  const int pitch = round_up8(r);
  const uint16_t* bslot = (const uint16_t*)a.pv.base + (long long)pi.y * a.pv.slot_elems + a.pv.b_offset;
  // the v row is requested before the B rows and staged in LDS after them
  // (that store then waits for the v row alone). With a d_in split of the
  // shrink (ks > 1) no k_vfinal runs: the row is the chunk partials summed in
  // chunk order and scaled, zero past the rank, as k_vfinal would write it.
  const bool vt = tid < kDxMaxRank / 4 && 4 * tid < a.r_ws;
  f32x4_t vq;
  if (a.ks > 1) {   // uniform
    f32x4_t part[kShrMaxSplit];
#pragma unroll
    for (int c = 0; c < kShrMaxSplit; ++c)
      part[c] = *(const f32x4_t*)(vt ? a.v_part + ((long long)min(c, a.ks - 1) * a.T + p) * a.r_ws + 4 * tid
                                     : (const float*)a.pv.zeros);
    vq = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kShrMaxSplit; ++c)
      if (c < a.ks) {
#pragma unroll
        for (int i = 0; i < 4; ++i) vq[i] += part[c][i];
      }
    const float sc = __int_as_float(pi.w);
#pragma unroll
    for (int i = 0; i < 4; ++i) vq[i] = 4 * tid + i < r ? vq[i] * sc : 0.f;
  } else {
    vq = *(const f32x4_t*)(vt ? a.v_fin + (long long)p * a.r_ws + 4 * tid : (const float*)a.pv.zeros);
  }
  if (pitch <= 8) expand_rows<1>(a, bslot, pitch, n_base, vq, vt, vs, drow);
  else if (pitch <= 16) expand_rows<2>(a, bslot, pitch, n_base, vq, vt, vs, drow);
  else if (pitch <= 32) expand_rows<4>(a, bslot, pitch, n_base, vq, vt, vs, drow);
  else expand_rows<8>(a, bslot, pitch, n_base, vq, vt, vs, drow);
}

// ---------------------------------------------------------------------------
// GEMM + fused expand
// ---------------------------------------------------------------------------
constexpr int kBatch = 8;           // independent loads per thread in bulk LDS copies
constexpr int kEpiRing = 16;        // B operand loads in flight per lane in the expand epilogue
constexpr int kEpiMaxUnits = 128;   // work units one wave lists per rank chunk (more: further passes)

// LDS address (byte offset in the workgroup's LDS) of a pointer into __shared__ memory
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Direct global -> LDS load (gfx950 LDS DMA): the wave's 64 lanes each fetch
// 16 bytes from their own global address and the data lands in LDS, lane l at
// byte m0 + 16 l, without passing through registers. Issued as inline
// assembly so that the compiler, which would otherwise wait for every
// outstanding DMA before any LDS read, leaves the waits to the stage ring
// below. One wait state separates the M0 write from its use.
__device__ __forceinline__ void dma16(const void* g, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0)
               : "memory", "m0");
}

// Wait until at most N of this wave's vector memory operations are in flight,
// then a workgroup barrier (LDS and scalar counters drained too; nothing else).
// The same load marked nontemporal, for W rows that the launch reads once
// (at most two position tiles, which run in the same round): measured on the
// verify and heterogeneous batches, their LoRA-off passes took 1-2 us less
// (45.2-46.3 against 47.3-47.8 us, 38.0 against 39.1 us). Where more position
// tiles re-read a W panel in later rounds (prefill) the mark lost about 10%
// (gate/up), and the positions' rows, re-read by every row tile, lost 5-18%.
__device__ __forceinline__ void dma16_nt(const void* g, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "s"(m0)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// KB: k per stage (32 or 64). A stage is the tile's BR W rows and its BT
// positions over KB columns. The stages reach LDS by direct loads into two
// rings, one for the W rows (NB slots, NB - 1 stages in flight while one is
// multiplied) and one for the positions (NX slots, NX - 1 in flight). Rows
// are 2 KB bytes (KB bf16), unpadded, and 16-byte chunk c of row r sits in slot
// c ^ gswz(r) of the row, so the rows read together by one fragment load fall
// in distinct LDS banks.
template <int BR, int BT, int WR, int WT, int NB, int KB, int NX>
struct GCfg {
  static constexpr int NWR = BR / WR, NWT = BT / WT;
  static constexpr int NW = NWR * NWT;
  static constexpr int NT = NW * kWave;
  static constexpr int MR = WR / 32, MT = WT / 32;        // 32x32 blocks per wave
  static constexpr int RB = 2 * KB;                        // bytes per LDS row
  static constexpr int WSTAGE_B = BR * RB, XSTAGE_B = BT * RB;   // ring slots
  static constexpr int DPW_W = BR * 2 * KB / 1024 / NW;    // 1 KB loads per wave per stage: W rows
  static constexpr int DPW_X = BT * 2 * KB / 1024 / NW;    // and positions
  static constexpr int DPW = DPW_W + DPW_X;
  static constexpr int XRING = NB * WSTAGE_B;              // byte offset of the position ring
  static constexpr int MAIN_BYTES = NB * WSTAGE_B + NX * XSTAGE_B;
  // DMAs a wave has issued after stage st's position DMAs when stage st is
  // multiplied (its W DMAs were issued earlier still)
  static constexpr int VMC = (NX - 2) * DPW;
  // small row tiles get extra LDS so the epilogue stages many segment runs at
  // once; the y tile of the store passes through the same LDS
  static constexpr int YT_BYTES = NW * WT * (2 * WR + 16);
  static constexpr int LDS_BYTES0 = MAIN_BYTES > 96 * 1024 ? MAIN_BYTES : 96 * 1024;
  static constexpr int LDS_BYTES = LDS_BYTES0 > YT_BYTES ? LDS_BYTES0 : YT_BYTES;
  static_assert(KB == 32 || KB == 64, "stage depth");
  static_assert((BR * 2 * KB) % (1024 * NW) == 0 && (BT * 2 * KB) % (1024 * NW) == 0,
                "each ring's stage splits into whole loads per wave");
  static_assert(NB >= 2 && NX >= 2 && NB >= NX && VMC <= 63, "ring depths and vmcnt range");
};

// Slot permutation of row r (depends on r mod 16 only). A fragment read has
// lane l take row l % 32 at one chunk. gfx950 serves a 16-byte LDS read 16
// lanes (256 bytes) at a time, so the 16 rows of a lane group must land on
// 16 distinct 16-byte bank groups modulo 256 bytes. KB = 64: two rows per
// 256 bytes; rows of equal parity take distinct slots through r >> 1, and
// the parity flips the slot's top bit. KB = 32: four rows per 256 bytes,
// separated through r >> 2. Both were checked with the LDS bank-conflict
// counter on a read-pattern probe (no conflicts), where the plain r & 7 and
// (r >> 1) & 3 permutations conflicted two ways.
template <int KB>
__device__ __forceinline__ int gswz(int r) {
  return KB == 64 ? (((r >> 1) ^ ((r & 1) << 2)) & 7) : ((r >> 2) & 3);
}

// Scheduling hint for one k-step: the R fragment reads of the next k-step
// spread over the M MFMAs of this one (one read, then its share of MFMAs).
template <int R, int M, int J = 0>
__device__ __forceinline__ void sched_reads_over_mfma() {
  if constexpr (J < R) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                          // DS read
    __builtin_amdgcn_sched_group_barrier(0x008, M * (J + 1) / R - M * J / R, 0);  // MFMA
    sched_reads_over_mfma<R, M, J + 1>();
  }
}

// One workgroup per CU (the LDS stages take most of it): the register
// allocator may then use the whole register file share of its waves (one
// wave per SIMD for 4 waves, two for 8).
template <int BR, int BT, int WR, int WT, int NB, int KB, int NX>
__global__ __launch_bounds__((BR / WR) * (BT / WT) * kWave)
__attribute__((amdgpu_waves_per_eu((BR / WR) * (BT / WT) / 4, (BR / WR) * (BT / WT) / 4)))
void k_gemm2(LinearArgs a) {
  using C = GCfg<BR, BT, WR, WT, NB, KB, NX>;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[C::LDS_BYTES / 2];
  __shared__ int4 pinfo[BT];

  // wave index made scalar: every per-wave quantity below is then uniform
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int l32 = lane % 32, kh = 8 * (lane / 32);
  const int T = a.T, d_in = a.d_in, d_out = a.d_out;
  const int n_rt = (d_out + BR - 1) / BR;
  // Block order. One round of blocks (a block per CU or fewer): row tiles
  // fastest, so the position tiles of one row tile (n_rt apart, on the same
  // XCD when n_rt % 8 == 0) run together and share that row tile's W in one
  // L2. More than one round (gorder): block b goes to XCD b % 8, which takes
  // row tiles xcd, xcd + 8, ... in turn with their position tiles one after
  // another, so a row tile's W is still read into one L2 once rather than
  // once per round. One round of large tiles (gorder 2, prefill's 256x256
  // tiles): XCD x takes a block of n_rt / 4 row tiles by n_tt / 2 position
  // tiles, so its L2 fills with 4 W panels' and n_tt / 2 position panels'
  // worth rather than 2 and n_tt (LoRA-off prefill q 125.4 -> 122.2 us, down
  // 411 -> 401 us, same bits).
  int rt, tt;
  if (a.gorder == 2) {   // uniform; the host sets it only when n_rt % 4 == 0 and n_tt % 2 == 0
    const int n_tt = (T + BT - 1) / BT, x = blockIdx.x & 7, j = blockIdx.x >> 3, fr = n_rt / 4;
    rt = (x & 3) * fr + j % fr;
    tt = (x >> 2) * (n_tt / 2) + j / fr;
  } else if (a.gorder) {   // uniform; the host sets it only when n_rt % 8 == 0
    const int j = blockIdx.x >> 3, n_tt = (T + BT - 1) / BT;
    rt = (j / n_tt) * 8 + (blockIdx.x & 7);
    tt = j % n_tt;
  } else {
    rt = blockIdx.x % n_rt;
    tt = blockIdx.x / n_rt;
  }
  const int r0 = rt * BR, t0 = tt * BT;
  const int wr = wave / C::NWT, wt = wave % C::NWT;
  const uint16_t* __restrict__ x = (const uint16_t*)a.x;
  const uint16_t* __restrict__ W = (const uint16_t*)a.W;
  const uint16_t* zeros = (const uint16_t*)a.pv.zeros;

  // loader: load i < DPW_W of wave w fills the W slot's 1 KB chunk
  // J = i NW + w, load DPW_W + i the position slot's chunk J; lane l writes
  // its byte J 1024 + 16 l of the slot, i.e. row r, slot l % (KB/8), and so
  // fetches chunk (slot ^ gswz(r)) of that row (W rows, or the gathered rows of
  // the tile's positions)
  const uint16_t* src[C::DPW];
  int scol[C::DPW];
#pragma unroll
  for (int i = 0; i < C::DPW; ++i) {
    const int J = (i >= C::DPW_W ? i - C::DPW_W : i) * C::NW + wave;
    int r = J * (1024 / (2 * KB)) + lane / (KB / 8);
    const int c = (lane % (KB / 8)) ^ gswz<KB>(r);
    if (i >= C::DPW_W) r += BR;   // a row of the position slot
    scol[i] = c * 8;
    if (r < BR) {
      src[i] = W + (long long)min(r0 + r, d_out - 1) * d_in + c * 8;
    } else {
      const int p = min(t0 + r - BR, T - 1);
      int row = a.sv.token_index ? a.sv.token_index[p] : p;
      row = min(max(row, 0), T - 1);
      src[i] = x + (long long)row * d_in + c * 8;
    }
  }
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));
  // W rows of stage st -> W slot st % NB, positions -> position slot
  // st % NX; stages past d_in (and the k tail) read the zero block, so every
  // stage issues the same DMA count and the rings' vmcnt waits stay exact
  // (W rows: i0 == 0, nontemporal when a.wnt; positions: i0 == DPW_W)
  const bool wnt = a.wnt != 0;
  auto issue_part = [&](int st, int i0, int n, uint32_t sb) {
    const int k0 = st * KB;
    if (k0 + KB <= d_in) {   // uniform: whole stage inside d_in
#pragma unroll
      for (int i = 0; i < n; ++i) {
        if (i0 == 0 && wnt) dma16_nt(src[i0 + i] + k0, sb + (uint32_t)i * C::NW * 1024);
        else dma16(src[i0 + i] + k0, sb + (uint32_t)i * C::NW * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < n; ++i) {
        const void* g = k0 + scol[i0 + i] < d_in ? src[i0 + i] + k0 : zeros;
        if (i0 == 0 && wnt) dma16_nt(g, sb + (uint32_t)i * C::NW * 1024);
        else dma16(g, sb + (uint32_t)i * C::NW * 1024);
      }
    }
  };
  auto issue_w = [&](int st) {
    issue_part(st, 0, C::DPW_W, lds0 + (uint32_t)(st % NB) * C::WSTAGE_B + (uint32_t)wave * 1024);
  };
  auto issue_x = [&](int st) {
    issue_part(st, C::DPW_W, C::DPW_X, lds0 + C::XRING + (uint32_t)(st % NX) * C::XSTAGE_B + (uint32_t)wave * 1024);
  };

  f32x16_t acc[C::MR][C::MT];
#pragma unroll
  for (int m = 0; m < C::MR; ++m)
#pragma unroll
    for (int n = 0; n < C::MT; ++n)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[m][n][v] = 0.f;

  // fragment reads: row R (a multiple of 32 plus l32), chunk kk 2 + kh / 8
  int fcol[KB / 16];
#pragma unroll
  for (int kk = 0; kk < KB / 16; ++kk)
    fcol[kk] = ((kk * 2 + kh / 8) ^ gswz<KB>(l32)) * 16;
  // the fragments of k-step kk + 1 are read while k-step kk is multiplied
  // (Lw: the stage's W rows, Lx: its positions)
  auto compute = [&](const char* Lw, const char* Lx) {
    u32x4_t af[2][C::MR], bf[2][C::MT];
    auto frag = [&](int kk, u32x4_t* fa, u32x4_t* fb) {
#pragma unroll
      for (int m = 0; m < C::MR; ++m)
        fa[m] = *(const u32x4_t*)(Lw + (wr * WR + m * 32 + l32) * C::RB + fcol[kk]);
#pragma unroll
      for (int n = 0; n < C::MT; ++n)
        fb[n] = *(const u32x4_t*)(Lx + (wt * WT + n * 32 + l32) * C::RB + fcol[kk]);
    };
    frag(0, af[0], bf[0]);
#pragma unroll
    for (int kk = 0; kk < KB / 16; ++kk) {
      if (kk + 1 < KB / 16) frag(kk + 1, af[(kk + 1) & 1], bf[(kk + 1) & 1]);
#pragma unroll
      for (int m = 0; m < C::MR; ++m)
#pragma unroll
        for (int n = 0; n < C::MT; ++n) acc[m][n] = mfma32g(af[kk & 1][m], bf[kk & 1][n], acc[m][n]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, C::MR + C::MT, 0);
#pragma unroll
    for (int kk = 0; kk + 1 < KB / 16; ++kk) sched_reads_over_mfma<C::MR + C::MT, C::MR * C::MT>();
    __builtin_amdgcn_sched_group_barrier(0x008, C::MR * C::MT, 0);
  };

  const int nst = (d_in + KB - 1) / KB;
  // Rings: iteration st requests the W rows of stage st + NB - 1, then the
  // positions of stage st + NX - 1. Before stage st is multiplied, this
  // wave's DMAs of stage st have landed (only those of later position
  // stages and the W stages issued with them may still be in flight: VMC
  // DMAs) and, past the barrier, so have every wave's; every wave is also
  // done with stage st - 1, whose slots then take the new requests. The
  // prologue issues the first stages in the same order the loop would.
  const char* L = (const char*)lds;
#pragma unroll
  for (int st = 0; st < NB - NX; ++st) issue_w(st);
#pragma unroll
  for (int j = 0; j < NX - 1; ++j) {
    issue_w(NB - NX + j);
    issue_x(j);
  }
  for (int st = 0; st < nst; ++st) {
    vm_barrier<C::VMC>();
    issue_w(st + NB - 1);
    issue_x(st + NX - 1);
    compute(L + (st % NB) * C::WSTAGE_B, L + C::XRING + (st % NX) * C::XSTAGE_B);
  }
  // the dense adapter term of k_expand_delta (zero where a position has no
  // adapter): lane (l32, h) takes rows 8 q + 4 h .. + 3 of each 32-row block
  // at its position. Small tiles request it here, so it lands while the
  // ring drains; positions past T and rows past d_out are clamped (neither is
  // stored).
  // Tiles whose y tile fits the LDS in fp32 add the term while storing y
  // (kDeltaTile, below), where consecutive lanes read consecutive rows of one
  // position; the others add it here, from per-lane 16-byte pieces.
  constexpr bool kDeltaTile = C::NW * WT * (4 * WR + 16) <= C::LDS_BYTES;
  constexpr bool kDeltaEarly = !kDeltaTile && C::MR * C::MT <= 4;
  const bool use_delta = a.lora_on && a.delta != nullptr;
  auto delta_ptr = [&](int n, int m, int q) {
    const int p = min(t0 + wt * WT + n * 32 + l32, T - 1);
    return a.delta + (long long)p * d_out + min(r0 + wr * WR + m * 32 + 8 * q + 4 * (lane / 32), d_out - 4);
  };
  f32x4_t dpre[kDeltaEarly ? C::MT : 1][kDeltaEarly ? C::MR : 1][4];
  if constexpr (kDeltaEarly) {
    if (use_delta) {
#pragma unroll
      for (int n = 0; n < C::MT; ++n)
#pragma unroll
        for (int m = 0; m < C::MR; ++m)
#pragma unroll
          for (int q = 0; q < 4; ++q) dpre[n][m][q] = *(const f32x4_t*)delta_ptr(n, m, q);
    }
  }
  // the ring's last DMAs (zero stages) land before the LDS is reused
  vm_barrier<0>();
  if (!kDeltaTile && use_delta) {
#pragma unroll
    for (int n = 0; n < C::MT; ++n)
#pragma unroll
      for (int m = 0; m < C::MR; ++m) {
        f32x4_t dv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if constexpr (kDeltaEarly) dv[q] = dpre[n][m][q];
          else dv[q] = *(const f32x4_t*)delta_ptr(n, m, q);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[m][n][4 * q + i] += dv[q][i];
      }
  }

  // ---- expand: acc += B_a (scale v) per segment run, on MFMA ---------------
  // scale*v of the tile's positions is staged in LDS (per rank chunk of up to
  // 64 columns), split into bf16 high and low parts so the MFMA keeps about
  // 16 mantissa bits of v. Each wave then walks the segment runs of its own
  // WT positions on its own, with no block barrier: a work unit is (run,
  // 16 rank columns); the unit's B slice (the wave's WR rows) is loaded from
  // the pool straight into MFMA operand registers, a ring of kEpiRing units
  // ahead of the unit being multiplied. (With the dense term of
  // k_expand_delta, added above, none of this runs.)
  if (a.lora_on && !a.delta) {
    const int RC = a.r_ws < 64 ? a.r_ws : 64;        // rank columns per chunk (16, 32 or 64)
    const int VP = RC + 8;                           // hi/lo row pitch (bf16)
    uint16_t* vsh = lds;
    uint16_t* vsl = lds + BT * VP;
    constexpr int WRUNS = WT + 1;
    __shared__ int wstart[C::NW][WRUNS];             // per-wave run starts (tile positions)
    __shared__ int4 udesc[C::NW][kEpiMaxUnits];      // per-wave work units of a rank chunk

    const int teff = min(BT, T - t0);
    for (int t = tid; t < BT; t += C::NT) {
      const int p = t0 + t;
      int4 e = make_int4(-1, -1, 0, 0);
      if (p < T) {
        e = a.pos_info[p];
        // clamp whatever the table holds (only meaningful for valid metadata)
        if (e.y < 0 || e.y >= a.pv.capacity || e.z <= 0) { e.y = -1; e.z = 0; }
        e.z = min(e.z, a.pv.max_rank);
      }
      pinfo[t] = e;
    }
    __syncthreads();

    // runs of this wave's positions [wb, we): a run starts where the segment changes
    const int wb = wt * WT, we = min(wb + WT, teff);
    int nrw = 0;                                     // runs of this wave (uniform)
    for (int c0 = wb; c0 < we; c0 += kWave) {
      const int t = c0 + lane;
      const bool st = t < we && (t == wb || pinfo[t].x != pinfo[t - 1].x);
      const unsigned long long m = __ballot(st);
      if (st) wstart[wave][nrw + __popcll(m & ((1ull << lane) - 1ull))] = t;
      nrw += __popcll(m);
    }
    nrw = __builtin_amdgcn_readfirstlane(nrw);
    if (lane == 0) wstart[wave][nrw] = we;
    // (wave-private table: the wave's own LDS writes are ordered before its reads)

    constexpr int P = kEpiRing / C::MR;              // units in flight
    for (int jc0 = 0; jc0 < a.r_ws; jc0 += RC) {
      const int rc = min(RC, a.r_ws - jc0);
      if (jc0 > 0) __syncthreads();                  // previous chunk's v reads are done
      // scale * v of the tile's positions, split into bf16 high and low parts
      const int nvs = BT * (rc / 4);
      for (int e0 = tid; e0 < nvs; e0 += C::NT * kBatch) {
        f32x4_t v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int e = min(e0 + u * C::NT, nvs - 1);
          const int t = e / (rc / 4), q = e % (rc / 4);
          const int tt = t < teff ? t : 0;
          v[u] = *(const f32x4_t*)(a.v_fin + (long long)(t0 + tt) * a.r_ws + jc0 + 4 * q);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int e = e0 + u * C::NT;
          if (e < nvs) {
            const int t = e / (rc / 4), q = e % (rc / 4);
            uint32_t h[2], l[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              const float v0 = t < teff ? v[u][2 * i] : 0.f, v1 = t < teff ? v[u][2 * i + 1] : 0.f;
              const uint16_t h0 = f32_to_bf16_bits(v0), h1 = f32_to_bf16_bits(v1);
              h[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
              l[i] = (uint32_t)f32_to_bf16_bits(v0 - bf16_bits_to_f32(h0)) |
                     ((uint32_t)f32_to_bf16_bits(v1 - bf16_bits_to_f32(h1)) << 16);
            }
            *(u32x2_t*)&vsh[t * VP + 4 * q] = u32x2_t{h[0], h[1]};
            *(u32x2_t*)&vsl[t * VP + 4 * q] = u32x2_t{l[0], l[1]};
          }
        }
      }
      __syncthreads();

      // unit list of this wave (wave-private LDS), built in parallel: lane l
      // takes run k0 + l and writes one descriptor per 16 rank columns it has
      // in this chunk: {rs | re << 16, jc, adapter, rank rounded up to 8}. A pass
      // lists at most kEpiMaxUnits units; longer lists take further passes.
      // A fused adapter over stacked projections is nonzero in this wave's
      // rows only in its slice's window of rank columns; units cover that
      // window (rounded out to 16 columns, whose extra columns are zero).
      const int wr0 = r0 + wr * WR, wr1 = min(wr0 + WR, d_out);
      for (int pb = 0;; pb += kEpiMaxUnits) {
      int nu_tot = 0;                                // units of the chunk (uniform)
      for (int k0 = 0; k0 < nrw; k0 += kWave) {
        const int k = k0 + lane;
        int rs = 0, re = 0, ad = -1, pitch = 0, cnt = 0, lo = 0;
        if (k < nrw) {
          rs = wstart[wave][k];
          re = wstart[wave][k + 1];
          const int4 pi = pinfo[rs];
          int w0 = 0, w1 = pi.z;
          if (pi.y >= 0) slice_window(a.pv, wr0, wr1, pi.z, &w0, &w1);
          lo = max(w0 - jc0, 0) & ~15;
          const int hi = pi.y >= 0 ? min(min(w1, pi.z) - jc0, rc) : 0;
          cnt = hi > lo ? (hi - lo + 15) / 16 : 0;
          ad = pi.y;
          pitch = round_up8(pi.z);
        }
        int inc = cnt;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
          const int up = __shfl_up(inc, off, kWave);
          if (lane >= off) inc += up;
        }
        const int base = nu_tot + inc - cnt;
        for (int i = 0; i < cnt; ++i) {
          const int g = base + i - pb;
          if (g >= 0 && g < kEpiMaxUnits) udesc[wave][g] = make_int4(rs | (re << 16), lo + 16 * i, ad, pitch);
        }
        nu_tot += __builtin_amdgcn_readfirstlane(__shfl(inc, kWave - 1, kWave));
      }
      const int nu = min(nu_tot - pb, kEpiMaxUnits);

      // A unit's descriptor is read from LDS (all lanes the same address) and
      // made scalar with readfirstlane, so the unit loop branches and forms
      // the B slice's base address on the scalar unit; the read for the unit
      // refilled next is issued before the current unit's MFMAs.
      auto sdesc = [&](int4 dv) {
        return make_int4(__builtin_amdgcn_readfirstlane(dv.x), __builtin_amdgcn_readfirstlane(dv.y),
                         __builtin_amdgcn_readfirstlane(dv.z), __builtin_amdgcn_readfirstlane(dv.w));
      };
      auto rdesc = [&](int u) {   // u uniform; past the list: any entry (not used)
        return udesc[wave][min(u, kEpiMaxUnits - 1)];
      };
      u32x4_t ring[P][C::MR];
      const int rowb = r0 + wr * WR;                 // first row of this wave
      auto load_unit = [&](int slot, int4 d, bool ok) {   // d scalar
        const bool live = ok && d.z >= 0;
        // the unit's 16 columns are one block of B (bblk_off): 32 B per row
        const uint16_t* sb = (const uint16_t*)a.pv.base +
                             (live ? (long long)d.z * a.pv.slot_elems + a.pv.b_offset + bblk_off(0, jc0 + d.y, d_out) : 0);
        const int col = jc0 + d.y + kh;
        // columns past the adapter's rank read the zero block (d.w is the
        // rank rounded up to 8). (A pointer select here compiled into
        // divergent branches whose join waited for every load in flight: the
        // ring overlapped nothing.)
#pragma unroll
        for (int m = 0; m < C::MR; ++m) {
          const int row = min(rowb + m * 32 + l32, d_out - 1);
          // (nontemporal: a unit's B rows are read by this workgroup alone;
          // the verify pass's LoRA-on call took 3 us less, same bits)
          ring[slot][m] = ld_nt16(sel_addr(live && col < d.w, sb + (long long)row * 16 + kh, zeros));
        }
      };
      // v operands of a unit, one unit ahead (double buffer); the mask of
      // positions outside the run is applied only where the MFMA uses them
      u32x4_t vhi[2][C::MT], vlo[2][C::MT];
      auto load_v = [&](int b, int jc) {
#pragma unroll
        for (int n = 0; n < C::MT; ++n) {
          const int tl = min(wb + n * 32 + l32, BT - 1);
          vhi[b][n] = *(const u32x4_t*)&vsh[tl * VP + jc + kh];
          vlo[b][n] = *(const u32x4_t*)&vsl[tl * VP + jc + kh];
        }
      };
      int4 dcur[P];
#pragma unroll
      for (int u = 0; u < P; ++u) {
        dcur[u] = sdesc(rdesc(u));
        load_unit(u, dcur[u], u < nu);
      }
      load_v(0, dcur[0].y);
      for (int u0 = 0; u0 < nu; u0 += P) {          // uniform
#pragma unroll
        for (int u = 0; u < P; ++u) {
          const int U = u0 + u;
          const int4 d = dcur[u];
          const int4 dnext = rdesc(U + P);           // LDS read in flight during the MFMAs
          load_v((u + 1) & 1, dcur[(u + 1) % P].y);
          if (U < nu) {                              // uniform (scalar)
            const int rs = d.x & 0xffff, re = d.x >> 16;
            const int n_lo = (rs - wb) / 32, n_hi = (re - 1 - wb) / 32;
#pragma unroll
            for (int n = 0; n < C::MT; ++n) {
              if (n < n_lo || n > n_hi) continue;    // uniform
              const int tl = wb + n * 32 + l32;
              const bool in = tl >= rs && tl < re;
              const u32x4_t hiu = in ? vhi[u & 1][n] : zero_u32x4();
              const u32x4_t lou = in ? vlo[u & 1][n] : zero_u32x4();
#pragma unroll
              for (int m = 0; m < C::MR; ++m) {
                acc[m][n] = mfma32g(ring[u][m], hiu, acc[m][n]);
                acc[m][n] = mfma32g(ring[u][m], lou, acc[m][n]);
              }
            }
          }
          dcur[u] = sdesc(dnext);
          load_unit(u, dcur[u], U + P < nu);        // refill the slot P units ahead
        }
      }
      if (pb + kEpiMaxUnits >= nu_tot) break;       // uniform
      }
    }
  }

  // ---- store y (bf16, RNE), rows scattered through token_index ------------
  // A lane's accumulators are 16 d_out values of one position in runs of 4,
  // so a direct store would touch 32 rows of y with 16 bytes each per
  // instruction. They pass through a wave-private LDS tile [position][WR]
  // instead, and leave as 16-byte pieces with consecutive lanes covering one
  // row of y (whole 64-256 byte runs).
  constexpr int YP = WR * 2 + 16;                       // tile row pitch (bytes)
  constexpr int CPR = WR / 8;                           // 16-byte pieces per row
  static_assert(C::NW * WT * YP <= C::LDS_BYTES, "y tile fits the LDS");
  if (a.lora_on && !a.delta) __syncthreads();          // the expand's LDS reads are done
  uint16_t* __restrict__ y = (uint16_t*)a.y;
  if constexpr (kDeltaTile) {
    if (use_delta) {
      // the tile in fp32 [position][WR]; each lane then takes 8 rows of one
      // position, adds the dense term's 8 values (one 32-byte run of its row,
      // consecutive lanes covering the row), rounds once and stores 16 bytes.
      // The dense term requires d_out % 8 == 0, so every run is whole.
      constexpr int YP4 = WR * 4 + 16;
      char* yt4 = (char*)lds + wave * WT * YP4;
#pragma unroll
      for (int n = 0; n < C::MT; ++n)
#pragma unroll
        for (int m = 0; m < C::MR; ++m)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int rr = m * 32 + 8 * q + 4 * (lane / 32);
            *(f32x4_t*)(yt4 + (n * 32 + l32) * YP4 + rr * 4) =
                f32x4_t{acc[m][n][4 * q], acc[m][n][4 * q + 1], acc[m][n][4 * q + 2], acc[m][n][4 * q + 3]};
          }
      // (wave-private tile: the wave's own LDS writes are ordered before its reads)
      const int col = r0 + wr * WR + 8 * (lane % CPR);
#pragma unroll 2
      for (int tb = 0; tb < WT; tb += kWave / CPR) {
        const int tl = tb + lane / CPR;
        const int p = t0 + wt * WT + tl;
        if (p >= T || col >= d_out) continue;
        const float* dsrc = a.delta + (long long)p * d_out + col;
        const f32x4_t d0 = *(const f32x4_t*)dsrc, d1 = *(const f32x4_t*)(dsrc + 4);
        int row = a.sv.token_index ? a.sv.token_index[p] : p;
        row = min(max(row, 0), T - 1);
        const f32x4_t a0 = *(const f32x4_t*)(yt4 + tl * YP4 + (lane % CPR) * 32);
        const f32x4_t a1 = *(const f32x4_t*)(yt4 + tl * YP4 + (lane % CPR) * 32 + 16);
        u32x4_t v;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          v[i] = (uint32_t)f32_to_bf16_bits(a0[2 * i] + d0[2 * i]) |
                 ((uint32_t)f32_to_bf16_bits(a0[2 * i + 1] + d0[2 * i + 1]) << 16);
          v[2 + i] = (uint32_t)f32_to_bf16_bits(a1[2 * i] + d1[2 * i]) |
                     ((uint32_t)f32_to_bf16_bits(a1[2 * i + 1] + d1[2 * i + 1]) << 16);
        }
        *(u32x4_t*)(y + (long long)row * d_out + col) = v;
      }
      return;
    }
  }
  char* yt = (char*)lds + wave * WT * YP;
#pragma unroll
  for (int n = 0; n < C::MT; ++n)
#pragma unroll
    for (int m = 0; m < C::MR; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rr = m * 32 + 8 * q + 4 * (lane / 32);
        u32x2_t pk;
        pk.x = (uint32_t)f32_to_bf16_bits(acc[m][n][4 * q]) | ((uint32_t)f32_to_bf16_bits(acc[m][n][4 * q + 1]) << 16);
        pk.y = (uint32_t)f32_to_bf16_bits(acc[m][n][4 * q + 2]) | ((uint32_t)f32_to_bf16_bits(acc[m][n][4 * q + 3]) << 16);
        *(u32x2_t*)(yt + (n * 32 + l32) * YP + rr * 2) = pk;
      }
  // (wave-private tile: the wave's own LDS writes are ordered before its reads)
  const int col = r0 + wr * WR + 8 * (lane % CPR);
  const bool vec = (d_out & 7) == 0 && col + 8 <= d_out;
#pragma unroll 4
  for (int tb = 0; tb < WT; tb += kWave / CPR) {
    const int tl = tb + lane / CPR;
    const int p = t0 + wt * WT + tl;
    if (p >= T || col >= d_out) continue;
    int row = a.sv.token_index ? a.sv.token_index[p] : p;
    row = min(max(row, 0), T - 1);
    const u32x4_t v = *(const u32x4_t*)(yt + tl * YP + (lane % CPR) * 16);
    uint16_t* dst = y + (long long)row * d_out + col;
    if (vec) {
      *(u32x4_t*)dst = v;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (col + e < d_out) dst[e] = (uint16_t)(v[e / 2] >> (16 * (e & 1)));
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// d_in chunks of the shrink: enough workgroups for the GPU, at most
// kShrMaxSplit (the partials k_vfinal folds), each chunk at least one
// 512-wide group.
int choose_shrink_split_bf16(int d_in, int items) {
  const int groups = (d_in + 511) / 512;
  int ks = 1;
  while (ks < kShrMaxSplit && ks * 2 <= groups && items * ks < 1024) ks *= 2;
  return ks;
}

// Shapes of the MFMA shrink, by the batch's mean segment length (host
// bound): longer than 16 positions, 64 positions per pass (NRB = 4) and all
// of a segment's rank rows per item (NCB = 4: x is read once per position
// block); otherwise 16 positions (NRB = 1) and 16 rank rows per item
// (NCB = 1: a short segment of high rank spreads over several items).
// Measured on the prefill (4096 tokens, 64 segments, rank 64) and
// heterogeneous (256 tokens, ranks 8-64) batches: the prefill shrink took 30
// us with NCB = 4 and 4 d_in chunks against 43 with NCB = 1 in one chunk;
// the heterogeneous one 16.5 us with NCB = 1 in one chunk (more chunks or
// rank blocks were slower).
static bool shrink_long_segs(int T, int n_seg_bound) { return T > 16 * n_seg_bound; }

// items of the shrink: (block of 16 NRB positions, group of 16 NCB rank
// rows) per segment
int shrink_items_bound(int T, int n_seg_bound, int max_rank) {
  const int ncb = shrink_long_segs(T, n_seg_bound) ? 4 : 1;
  const int ng = (max_rank + 16 * ncb - 1) / (16 * ncb);
  const int pb = shrink_long_segs(T, n_seg_bound) ? 64 : 16;
  return ((n_seg_bound < kShrMaxSeg ? n_seg_bound : kShrMaxSeg) + (T + pb - 1) / pb) * (ng > 1 ? ng : 1);
}

// gorder (the XCD-grouped block order of k_gemm2) for launches of more than
// one block per CU on the HBM-bound tiles: measured on the fused gate|up
// projection at the verify batch (448 128x128 tiles over 28672 rows), where
// row tiles fastest left most row tiles' two position tiles in different
// rounds and read W twice.
template <int BR, int BT, int WR, int WT, int NB, int KB, int NX>
static void launch_g(const LinearArgs& a, hipStream_t st, bool grouped_order) {
  const int n_rt = (a.d_out + BR - 1) / BR, n_tt = (a.T + BT - 1) / BT;
  LinearArgs g = a;
  g.gorder = grouped_order && n_tt > 1 && n_rt % 8 == 0 && (long long)n_rt * n_tt > 256;
  if (BR == 256 && n_rt % 4 == 0 && n_tt % 2 == 0 && (long long)n_rt * n_tt <= 256) g.gorder = 2;
  g.wnt = n_tt <= 2;
  hipLaunchKernelGGL((k_gemm2<BR, BT, WR, WT, NB, KB, NX>), dim3(n_rt * n_tt),
                     dim3(GCfg<BR, BT, WR, WT, NB, KB, NX>::NT), 0, st, g);
}

// MLORA_FORCE_SHRINK=mfma keeps the MFMA shrink on short segments too.
static bool shrink_short_enabled() {
  const char* e = getenv("MLORA_FORCE_SHRINK");
  return !(e && strcmp(e, "mfma") == 0);
}

// The vector-ALU shrink for short segments: a segment count known on the
// host with at most two positions per segment on average (its items re-read
// an adapter's A for every kSsPos positions of a longer segment), ranks up
// to kSsMaxRank (a workgroup per kSsRows rank rows), one d_in chunk. Segments
// built on the device only bound their count by T, so they keep the MFMA
// shrink. Up to rank 32 it covers a fused gate|up pool of two rank-16
// slices at the verify batch, where the MFMA shrink and its fold took 16.2 +
// 5.1 us against 9.5 us for one rank-16 projection.
bool shrink_short(const LinearArgs& a) {
  return a.lora_on && a.ks == 1 && a.sv.n_seg_dev == nullptr && a.seg_grid > 0 && a.T <= 2 * a.seg_grid &&
         a.pv.max_rank <= kSsMaxRank && shrink_short_enabled();
}

void launch_shrink_bf16(const LinearArgs& a, hipStream_t st) {
  if (a.lora_on && a.seg_grid > 0) {
    // the MFMA shrink's shape follows the batch's mean segment length
    // (shrink_long_segs)
    const int nseg = a.seg_grid < kShrMaxSeg ? a.seg_grid : kShrMaxSeg;
    const bool long_segs = shrink_long_segs(a.T, a.seg_grid);
    const dim3 grid(shrink_items_bound(a.T, a.seg_grid, a.pv.max_rank), a.ks);
    const size_t lds = shrink_lds_bytes(a.seg_grid);
    if (shrink_short(a)) {
      // at most two positions per segment on average, one d_in chunk, ranks <= kSsMaxRank
      const dim3 gs((a.pv.max_rank + kSsRows - 1) / kSsRows, nseg + (a.T + kSsPos - 1) / kSsPos);
      hipLaunchKernelGGL(k_shrink_short, gs, dim3(256), lds, st, a);
      return;
    }
    if (long_segs) hipLaunchKernelGGL((k_shrink2<4, 4>), grid, dim3(256), lds, st, a);
    else hipLaunchKernelGGL((k_shrink2<1, 1>), grid, dim3(256), lds, st, a);
    if (a.ks > 1 && !a.delta) {   // (the dense term's expand folds the chunks itself)
      const int n4 = a.T * (a.r_ws / 4);
      hipLaunchKernelGGL(k_vfinal, dim3((n4 + 255) / 256), dim3(256), 0, st, a);
    }
  }
}

// Tile choice: large batches take 256x256 tiles (MFMA-bound); otherwise
// 128x128 tiles while they fill the GPU, else tiles that span 256 or 128
// positions with 64 W rows. A measured sweep of tiles and ring depths on the
// verify (256 tokens, 4096 -> 14336), heterogeneous (256 tokens,
// 5120 -> 5120) and prefill (4096 tokens) shapes, every choice giving the
// same bits: 128x128 tiles (3 W and 3 position slots) took the verify pass
// from 53 to 48 us without LoRA (4 + 4 slots, or 32-wide stages in rings of
// 6-9, were slower); the 256x256 tile runs 8 waves (two per SIMD, 128 rows x
// 64 positions each) on 64-wide stages in 2 + 2 slots: against 32-wide
// stages in 2 + 2 slots it took the q projection from 211 to 197 us with
// LoRA and 155 to 150 without, gate/up from 597 to 548 and 501 to 443, down
// from 573 to 504 and 495 to 411 (32-wide stages in rings of 3-6 slots were
// in between); the 64x128 tile stayed best on the 5120-wide layer (deeper
// W rings gained nothing there), its waves split by positions (64 rows x 32
// positions each): a wave then walks the segment runs of 32 positions, not
// 64, in units of 2 KB of B rather than 1 KB, and the heterogeneous batch's
// LoRA-on call dropped from 98 to 88 us. Later, with rotations sized by W,
// x and y: the 128x128 and 64x128 tiles in 8 waves (two per SIMD; waves of
// 64x32 and 32x32) beat their 4-wave forms on the verify batch (67.0-67.4
// against 70.6-71.3 us LoRA-on, 47.3 against 48.2-49.0 us off) and the
// heterogeneous one (82.6-82.9 against 84.7 us, 39.2 against 40.5 us): each
// CU then keeps twice the waves issuing loads; deeper rings or 2x2-wave
// shapes did not do better.
void launch_linear_bf16(const LinearArgs& a, hipStream_t st) {
  launch_shrink_bf16(a, st);
  if (a.lora_on && a.delta && a.seg_grid > 0)
    hipLaunchKernelGGL(k_expand_delta, dim3((a.d_out + kDxRows - 1) / kDxRows, a.T), dim3(kDxThreads), 0, st, a);
  auto tiles = [&](int br, int bt) {
    return (long long)((a.d_out + br - 1) / br) * ((a.T + bt - 1) / bt);
  };
  constexpr long long kFill = 192;   // tiles that keep most of the 256 CUs busy
  if (a.T > 128 && tiles(256, 256) >= kFill) launch_g<256, 256, 128, 64, 2, 64, 2>(a, st, false);
  else if (a.T > 64 && tiles(128, 128) >= kFill) launch_g<128, 128, 64, 32, 3, 64, 3>(a, st, true);
  else if (a.T > 128 && tiles(64, 256) >= kFill) launch_g<64, 256, 64, 64, 3, 64, 3>(a, st, true);
  else launch_g<64, 128, 32, 32, 4, 64, 4>(a, st, true);
}

}  // namespace mlora
