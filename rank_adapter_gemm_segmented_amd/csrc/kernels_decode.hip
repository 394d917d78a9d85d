// kernels_decode.hip -- bf16 multi-LoRA linear for small token counts (T <= 64).
//
// y_i = W x_i + scale_s * B_a (A_a x_i) ("Multi-LoRA Serving in Practice",
// section "Core Principle", displayed formula), per adapter segment
// ("InvisibleLoRA" abstract). At decode the layer is HBM-bound: W (and each
// touched adapter) must be streamed once, and with T <= 64 a CU that covered
// the whole of d_in would re-read all of x from L2 (4x the bytes of its W
// rows). So d_in is split into chunks across CUs, and the layer runs in two
// launches with no inter-workgroup synchronization:
//
//  k_stream  one-shot items (n-tile of 64 W rows, d_in chunk c). An item loads
//            its x chunk into LDS and its W rows straight into MFMA operand
//            registers, every load in flight at once, then runs
//            v_mfma_f32_16x16x32_bf16. The shrink v = A_a x is folded in per
//            segment: item (c, tile) takes segments tile, tile + n_tiles, ...
//            and multiplies their A rows (restricted to chunk c) against the
//            same x chunk in LDS. Outputs: fp32 partial tiles of W x and of
//            v, one slot per chunk (deterministic, no atomics).
//  k_finish  y = sum_c partial_c + scale_s * B_a (sum_c v_c), summed in chunk
//            order, the expand on the vector ALUs in fp32, one bf16 store.
//
// MFMA 16x16x32 bf16 lane layout: lane l holds row l%16, k-slots
// 8*(l/16)..+7 of each operand; result register v of lane l is row
// 4*(l/16)+v, column l%16.
#include "common.h"
#include "launch.h"

namespace mlora {

__device__ __forceinline__ f32x4_t mfma16d(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

constexpr int kDecThreads = 512;                   // 8 waves
constexpr int kDecWaves = kDecThreads / kWave;
constexpr int kDecRows = 64;                       // W rows per item (4 blocks of 16)
constexpr int kDecXPitch = kDecMaxKc + 8;          // LDS row pitch of the x chunk (bf16)
constexpr int kDecWSteps = kDecMaxKc / 2 / 32;     // 32-wide k-steps per wave (16)
constexpr int kDecWPre = 8;                        // W k-steps requested before the x barrier
constexpr int kDecASteps = kDecMaxKc / 8 / 32;     // shrink k-steps per wave per row block (4)

template <int TT>
struct DecSmem {
  uint16_t xs[TT * kDecXPitch];
  float red[4][kWave][4 * (TT / 16)];              // second-half partials of the W rows
};

// Partial tile layout (fragment-major): for chunk c, n-tile i, row block rb,
// token block tb: 256 floats ordered [lane][4].
__device__ __forceinline__ long long part_off(int c, int i, int rb, int tb, int n_tiles, int ntb) {
  return ((((long long)c * n_tiles + i) * 4 + rb) * ntb + tb) * 256;
}


// Eight FP8 e4m3 codes (OCP E4M3: bias 7, subnormals m/8 * 2^-6) -> eight
// bf16 values, exact: every e4m3 value has at most 4 significant bits and an
// exponent inside bf16's range. gfx950's scaled conversion turns two codes
// into two bf16 per instruction (scale 1; checked against the E4M3
// definition on all 256 codes).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI));
}
__device__ __forceinline__ u32x4_t e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  u32x4_t r;
  r.x = e4m3x2_to_bf16x2<false>(lo);
  r.y = e4m3x2_to_bf16x2<true>(lo);
  r.z = e4m3x2_to_bf16x2<false>(hi);
  r.w = e4m3x2_to_bf16x2<true>(hi);
  return r;
}

// W8: W holds FP8 e4m3 codes (one byte per element, a float32 scale per row
// applied by k_finish). A lane's 16-byte load then covers 16 columns, which
// serve two consecutive k-steps: lane group g = l / 16 of the step pair
// (2q, 2q + 1) starting at column C takes columns C + 16 g .. + 7 in step 2q
// and C + 16 g + 8 .. + 15 in step 2q + 1, and reads x at the same columns.
template <int TT, bool W8>
__global__ __launch_bounds__(kDecThreads) void k_stream_bf16(DecodeArgs a) {
  constexpr int NTB = TT / 16;
  constexpr int XP = kDecXPitch;
  constexpr int XCH = TT * (kDecMaxKc / 8) / kDecThreads;  // 16-byte x pieces per thread
  __shared__ __attribute__((aligned(16))) DecSmem<TT> sm;

  const int item = blockIdx.x;
  const int c = item / a.n_tiles;
  const int tile = item % a.n_tiles;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int l16 = lane % 16, kq = 8 * (lane / 16);
  const int T = a.T, d_in = a.d_in, d_out = a.d_out;
  const int k0 = c * a.kc;
  const int kc = min(a.kc, d_in - k0);          // this chunk's width (multiple of 8)
  const int nks = (kc + 31) / 32;
  const uint16_t* __restrict__ x = (const uint16_t*)a.x;
  const uint16_t* __restrict__ W = (const uint16_t*)a.W;
  const bool lora = a.lora_on != 0;

  // ---- 0. this item's shrink units -----------------------------------------
  // A unit is ur = a.unit_rows (4, 8 or 16) consecutive rank rows of one
  // segment: unit u = s * nq + q holds rows [q ur, (q + 1) ur) of segment s,
  // nq = ceil(max_rank / ur). Lane l of every wave holds unit tile + l * n_tiles
  // (at most 64 per item, which the host guarantees). The lane's segment
  // metadata loads go first in the queue, from clamped indices (without LoRA
  // they read the pool's zero block), so the waits for them never wait for the
  // x and W loads issued after them.
  // The device segment count, when there is one, is read the same way: the
  // offset vz is zero, but held in a vector register, so the load is a vector
  // load (ordered with the others) rather than a scalar one, whose wait would
  // come at once.
  int vz;
  asm volatile("v_mov_b32 %0, 0" : "=v"(vz));
  const int32_t* zi = (const int32_t*)a.pv.zeros;
  const bool nsd_on = lora && a.sv.n_seg_dev != nullptr;
  const int nsd = *((nsd_on ? a.sv.n_seg_dev : zi) + vz);
  const int ur = a.unit_rows;
  const int nq = (a.pv.max_rank + ur - 1) / ur;
  const int u_l = tile + lane * a.n_tiles;
  const int s_l = u_l / nq, j0_l = (u_l - s_l * nq) * ur;   // segment, first rank row
  const int si = lora ? min(s_l, max(a.sv.n_seg - 1, 0)) : 0;
  const int m_st0 = *(lora ? a.sv.seg_start + si : zi);
  const int m_st1 = *(lora ? a.sv.seg_start + si + 1 : zi);
  const int m_ad = *(lora ? a.sv.seg_adapter + si : zi);
  const int m_rk = *(lora ? a.sv.seg_rank + si : zi);
  const float m_sc = *(lora ? a.sv.seg_scale + si : (const float*)zi);

  // ---- 1. x chunk -> registers ---------------------------------------------
  // thread's pieces: token t_i = tid/128 + 4 i, 16-byte column tid % 128
  const int kc8 = kc / 8;
  const int xcol = tid % (kDecMaxKc / 8);
  const bool xcol_ok = xcol < kc8;
  const int xk = k0 + (xcol_ok ? xcol : 0) * 8;
  int xrow[XCH];
#pragma unroll
  for (int i = 0; i < XCH; ++i) xrow[i] = min(tid / (kDecMaxKc / 8) + (kDecThreads / (kDecMaxKc / 8)) * i, T - 1);
  if (a.sv.token_index) {  // uniform: gather rows of the sorted positions
#pragma unroll
    for (int i = 0; i < XCH; ++i) xrow[i] = min(max(a.sv.token_index[xrow[i]], 0), T - 1);
  }
  u32x4_t xr[XCH];
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int t = tid / (kDecMaxKc / 8) + (kDecThreads / (kDecMaxKc / 8)) * i;
    // absent tokens and columns past the chunk read the zero block (an
    // address select: a select on the loaded value would wait for it here)
    xr[i] = ld16(t < T && xcol_ok ? x + (long long)xrow[i] * d_in + xk : (const uint16_t*)a.pv.zeros);
  }

  // ---- 2. W rows -> MFMA A-operand registers --------------------------------
  // wave w: row block rb = w % 4, k-half kh = w / 4 of the chunk. Its first
  // kDecWPre k-steps are requested right behind the x loads, the rest inside
  // the MFMA loop, kDecWPre steps ahead of the step being multiplied: x's
  // requests lead every CU's queue, and HBM streams W while x lands (the
  // barrier below waits for LDS only, not for these loads). Requesting all of
  // the wave's W up front measured slower: x then lands later. Addresses past the chunk or d_out are clamped
  // into the row: their products meet zero x columns or land in discarded
  // rows; steps that belong to the other k-half read zeros. No select on a
  // loaded value.
  const int rb = wave & 3, kh = wave >> 2;
  const int nrow = tile * kDecRows + rb * 16 + l16;
  // (FP8: the first half ends on an even step, so no step pair straddles the halves)
  const int half_steps = W8 ? (((nks + 1) / 2 + 1) & ~1) : (nks + 1) / 2;
  const int ks_begin = kh ? half_steps : 0;
  const int ks_end = kh ? nks : half_steps;
  const uint16_t* wrow = W + (long long)min(nrow, d_out - 1) * d_in + k0;
  const uint8_t* wrow8 = (const uint8_t*)a.W + (long long)min(nrow, d_out - 1) * d_in + k0;
  u32x4_t wr[kDecWSteps];
  auto load_w = [&](int s) {
    // steps of the other k-half read the pool's zero block (address select)
    if constexpr (W8) {   // slot s holds step pair (2s, 2s + 1)
      const int k = (ks_begin + 2 * s) * 32 + 2 * kq;
      wr[s] = ld_nt16(ks_begin + 2 * s < ks_end ? (const void*)(wrow8 + min(k, kc - 16))
                                                : (const void*)((const uint16_t*)a.pv.zeros + kq));
    } else {
      const int k = (ks_begin + s) * 32 + kq;
      wr[s] = ld_nt16(ks_begin + s < ks_end ? wrow + min(k, kc - 8) : (const uint16_t*)a.pv.zeros + kq);
    }
  };
  // FP8: the 16 steps are 8 loads; half of them are requested ahead of the
  // x barrier, as for the bf16 weight (8 ahead: 16.7 us LoRA-on, 4: 16.2 us,
  // 2: 16.5 us on the decode batch)
  constexpr int kWLoads = W8 ? kDecWSteps / 2 : kDecWSteps;
  constexpr int kWPre = W8 ? kWLoads / 2 : kDecWPre;
#pragma unroll
  for (int s = 0; s < kWPre; ++s) load_w(s);
  // nothing below is hoisted between these loads (it would wait for the
  // metadata before the last of them are issued)
  __builtin_amdgcn_sched_barrier(0);

  // ---- 3. rows to shrink per unit -------------------------------------------
  // the segment's rank capped by the slot size (the registered rank is applied
  // by the position table, which k_finish reads), cut to the unit's rows
  const int nseg = !lora ? 0 : nsd_on ? min(max(nsd, 0), a.sv.n_seg) : a.sv.n_seg;
  const bool s_ok = s_l < nseg;
  const int ps_l = max(m_st0, 0), pe_l = min(m_st1, T);
  const bool live_l = s_ok && pe_l > ps_l && m_ad >= 0 && m_ad < a.pv.capacity && m_rk > 0;
  const int rr_l = live_l ? min(m_rk, a.pv.max_rank) : 0;
  const int rows_l = min(max(rr_l - j0_l, 0), ur);
  const unsigned long long umask = __ballot(rows_l > 0);   // wave-uniform

  // ---- 4. x registers -> LDS -----------------------------------------------
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int t = tid / (kDecMaxKc / 8) + (kDecThreads / (kDecMaxKc / 8)) * i;
    *(u32x4_t*)&sm.xs[t * XP + xcol * 8] = xr[i];
  }
  // registered rank of the lane's adapter, for the position table written by
  // wave 0 of the chunk-0 items, lanes of a segment's first unit (the others
  // read the zero block)
  const bool pos_item = lora && c == 0 && wave == 0;
  const bool pos_lane = s_l < nseg && j0_l == 0;
  const int reg_r = *(pos_item && pos_lane && live_l ? a.pv.rank + m_ad : zi);
  lds_barrier();

  // ---- 5. shrink units, visited in lane order -------------------------------
  // The A rows of the first two are requested now, so they stream in under the
  // W MFMAs. An absent row reads the pool's zero block; k past the chunk reads
  // a clamped in-row address whose product meets zero x in LDS.
  auto next_unit = [&](int i) {
    const unsigned long long rest = i >= kWave - 1 ? 0ull : umask & (~0ull << (i + 1));
    return rest ? (int)__builtin_ctzll(rest) : kWave;
  };
  u32x4_t ar[2][kDecASteps];
  auto load_a = [&](int i, u32x4_t* dst) {
    const int ii = i < kWave ? i : 0;
    const int rows = i < kWave ? __builtin_amdgcn_readlane(rows_l, ii) : 0;
    const int j0 = __builtin_amdgcn_readlane(j0_l, ii);
    const int ad = __builtin_amdgcn_readlane(m_ad, ii);
    const bool rok = l16 < rows;
    const uint16_t* arow = rok ? (const uint16_t*)a.pv.base + (long long)ad * a.pv.slot_elems +
                                     (long long)(j0 + l16) * d_in + k0
                               : (const uint16_t*)a.pv.zeros;
    const int klim = rok ? kc - 8 : kZeroBlockElems - 8;
#pragma unroll
    for (int st = 0; st < kDecASteps; ++st) {
      const int k = (wave + 8 * st) * 32 + kq;
      dst[st] = ld16(arow + min(k, klim));
    }
  };
  int bi = umask ? (int)__builtin_ctzll(umask) : kWave;   // unit in ar[0]
  int ni = next_unit(bi);                                 // unit in ar[1]
  // issued unconditionally (absent units read zeros): a branch here would
  // make the compiler's waits for the W loads below conservative
  load_a(bi, ar[0]);
  load_a(ni, ar[1]);

  // ---- 6. base MFMAs --------------------------------------------------------
  f32x4_t acc[NTB];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) acc[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kDecWSteps; ++s) {
    if constexpr (W8) {
      if ((s & 1) == 0 && s / 2 + kWPre < kWLoads) load_w(s / 2 + kWPre);
    } else {
      if (s + kDecWPre < kDecWSteps) load_w(s + kDecWPre);
    }
    // x columns past ks_end (past the chunk) are zero in LDS; k-steps past
    // the LDS chunk are clamped onto such columns
    int xc;
    u32x4_t wop;
    if constexpr (W8) {
      const int kp = min(ks_begin + (s & ~1), kDecMaxKc / 32 - 2);   // the step pair's first step
      xc = kp * 32 + 2 * kq + 8 * (s & 1);
      const u32x4_t raw = wr[s / 2];
      wop = (s & 1) ? e4m3x8_to_bf16x8(raw.z, raw.w) : e4m3x8_to_bf16x8(raw.x, raw.y);
    } else {
      xc = min(ks_begin + s, kDecMaxKc / 32 - 1) * 32 + kq;
      wop = wr[s];
    }
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      const u32x4_t xo = *(const u32x4_t*)&sm.xs[(tb * 16 + l16) * XP + xc];
      acc[tb] = mfma16d(wop, xo, acc[tb]);
    }
    __builtin_amdgcn_sched_barrier(0);   // keep each step's load next to its MFMAs
  }
  // fixed-order sum of the two k-halves, then one coalesced fragment store
  if (kh == 1) {
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
      for (int v = 0; v < 4; ++v) sm.red[rb][lane][tb * 4 + v] = acc[tb][v];
  }
  __syncthreads();
  if (kh == 0) {
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      f32x4_t o;
#pragma unroll
      for (int v = 0; v < 4; ++v) o[v] = acc[tb][v] + sm.red[rb][lane][tb * 4 + v];
      // (nontemporal: the finish kernel reads it once, from another XCD)
      __builtin_nontemporal_store(o, (f32x4_t*)(a.ypart + part_off(c, tile, rb, tb, a.n_tiles, NTB) + lane * 4));
    }
  }

  // ---- 7. position table for k_finish --------------------------------------
  // Every sorted position's entry {adapter or -1, rank, scale bits}: the rank
  // is the segment's capped by the registered one, so a lying rank never reads
  // past the registered adapter and an emptied slot drops out. The lane of a
  // segment's first unit writes the segment's positions.
  if (pos_item) {   // uniform
    const int r = live_l ? min(rr_l, reg_r) : 0;
    const int ad = r > 0 ? m_ad : -1;
    const int4 e = make_int4(ad, ad >= 0 ? r : 0, __float_as_int(ad >= 0 ? m_sc : 0.f), 0);
    if (pos_lane)
      for (int t = ps_l; t < pe_l; ++t) a.pos[t] = e;
  }

  // ---- 8. shrink units -------------------------------------------------------
  // Each wave writes its own k-slice of the unit straight to
  // v_part[c][wave][t][j] (k_finish sums the 8 * n_chunks slices in a fixed
  // order): no barrier after the W MFMAs.
  float* vp = a.v_part + ((long long)c * kDecWaves + wave) * T * a.r_ws;
  auto shrink_unit = [&](u32x4_t* cur) {
    const int rows = __builtin_amdgcn_readlane(rows_l, bi);
    const int j0 = __builtin_amdgcn_readlane(j0_l, bi);
    const int ps = __builtin_amdgcn_readlane(ps_l, bi), pe = __builtin_amdgcn_readlane(pe_l, bi);
    const int tb_lo = ps / 16, tb_hi = (pe - 1) / 16;
    f32x4_t vacc[NTB];
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) vacc[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < kDecASteps; ++st) {
      const int ks = wave + 8 * st;   // always < 32; operands past the chunk are zero
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        if (tb < tb_lo || tb > tb_hi) continue;
        const u32x4_t xo = *(const u32x4_t*)&sm.xs[(tb * 16 + l16) * XP + ks * 32 + kq];
        vacc[tb] = mfma16d(cur[st], xo, vacc[tb]);
      }
    }
    // refill this buffer with the unit after next
    const int n2 = next_unit(ni);
    if (n2 < kWave) load_a(n2, cur);
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      if (tb < tb_lo || tb > tb_hi) continue;
      const int t = tb * 16 + l16;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int jr = 4 * (lane / 16) + v;
        if (jr < rows && t >= ps && t < pe) __builtin_nontemporal_store(vacc[tb][v], vp + (long long)t * a.r_ws + j0 + jr);
      }
    }
    bi = ni;
    ni = n2;
  };
  while (bi < kWave) {   // uniform
    shrink_unit(ar[0]);
    if (bi >= kWave) break;
    shrink_unit(ar[1]);
  }
}

// ---------------------------------------------------------------------------
// finish: one workgroup per (n-tile, 16-token block); wave w = row block w.
// Every load that does not depend on the adapter id is issued first (chunk
// partials, v partials, the position table, token_index); the B rows follow
// once the lane's adapter is known.
// ---------------------------------------------------------------------------
constexpr int kFinUnroll = 8;

// SL: the pool holds fused adapters over stacked projections (expand only
// the tile's slice window; a template flag, so plain pools keep a loop that
// starts at column 0: a run-time start measured 1 us slower)
template <int TT, bool W8, bool SL>
__global__ __launch_bounds__(256) void k_finish_bf16(DecodeArgs a) {
  constexpr int NTB = TT / 16;
  constexpr int kPre = 2;                // B column groups of 8 prefetched (ranks <= 16)
  const int tile = blockIdx.x / NTB, tb = blockIdx.x % NTB;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int T = a.T, d_out = a.d_out;
  const int rb = wave;
  const bool lora = a.lora_on != 0;
  __shared__ float vs[16][kMaxRankWs + 4];
  __shared__ f32x4_t vgrp[4][256];

  const int t = tb * 16 + (lane % 16);   // this lane's token (sorted position)
  const int tc = min(t, T - 1);
  const int n = tile * kDecRows + rb * 16 + 4 * (lane / 16);
  int row = a.sv.token_index ? a.sv.token_index[tc] : tc;
  const int4 pe = lora ? a.pos[tc] : make_int4(-1, 0, 0, 0);

  // the chunk partials, all loads in flight (nontemporal, as they were
  // written: each is read once; measured 0.6 us faster per LoRA-on call on
  // the decode batch, same bits)
  const float* pbase = a.ypart + part_off(0, tile, rb, tb, a.n_tiles, NTB) + lane * 4;
  const long long cstride = (long long)a.n_tiles * 4 * NTB * 256;
  f32x4_t p[kFinUnroll];
#pragma unroll
  for (int u = 0; u < kFinUnroll; ++u)
    p[u] = __builtin_nontemporal_load((const f32x4_t*)(pbase + min(u, a.n_chunks - 1) * cstride));
  // FP8 weight: the row scales of the lane's 4 rows
  float wsc[4] = {1.f, 1.f, 1.f, 1.f};
  if constexpr (W8) {
#pragma unroll
    for (int v = 0; v < 4; ++v) wsc[v] = a.w_scale[min(n + v, d_out - 1)];
  }

  // v of the 16 tokens: sum of the stream kernel's slices [c][w]. A 16-byte
  // quad of one token is element e; G groups of threads each sum every G-th
  // slice of an element, then the groups are added in group order. The first
  // batch of slice loads is issued here, with the partials still in flight.
  // Rank quads summed and staged: all of them; for a fused pool only quads
  // [q0, q0 + nqv), the union over the block's 16 tokens of their windows in
  // this tile's slice, widened to multiples of 8 columns (the expand reads
  // v in groups of 8 from the window start rounded down to 8). Every wave
  // holds the same 16 tokens, so the union is the same in every wave.
  int q0 = 0, nqv = a.r_ws / 4;
  if constexpr (SL) {
    const int ad_ = pe.x, r_ = min(pe.y, a.pv.max_rank);
    const bool live_ = lora && ad_ >= 0 && ad_ < a.pv.capacity && r_ > 0 && t < T;
    int w0 = 0, w1 = r_;
    if (live_) slice_window(a.pv, tile * kDecRows, min(tile * kDecRows + kDecRows, d_out), r_, &w0, &w1);
    int lo = live_ ? (w0 & ~7) : 0x7fffffff, hi = live_ ? min(w1, r_) : 0;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      lo = min(lo, __shfl_xor(lo, off, kWave));
      hi = max(hi, __shfl_xor(hi, off, kWave));
    }
    q0 = hi > lo ? lo / 4 : 0;
    nqv = hi > lo ? round_up8(hi) / 4 - q0 : 1;
  }
  const int E = 16 * nqv;
  const int G = E >= 256 ? 1 : E >= 128 ? 2 : 4;
  const int nsl = a.n_chunks * kDecWaves;
  const long long vstride = (long long)T * a.r_ws;
  auto vptr = [&](int e0) {
    const int e = min(e0 + tid / G, E - 1);
    return a.v_part + (long long)min(tb * 16 + e / nqv, T - 1) * a.r_ws + 4 * (q0 + e % nqv);
  };
  f32x4_t vq[kFinUnroll];
  {
    // without LoRA every lane reads the pool's zero block (an address select
    // keeps the loads unconditional)
    const float* vp = vptr(0);
#pragma unroll
    for (int u = 0; u < kFinUnroll; ++u)
      vq[u] = *(const f32x4_t*)(lora ? vp + min(tid % G + u * G, nsl - 1) * vstride : (const float*)a.pv.zeros);
  }
  // the slice loads stay ahead of the B loads, which wait for the position
  // entry: the v sums below then wait for them alone
  __builtin_amdgcn_sched_barrier(0);


  // B rows of the lane's adapter (first 16 rank columns), as soon as the
  // position entry is in
  const int ad = pe.x, r = min(pe.y, a.pv.max_rank);
  const bool live = lora && ad >= 0 && ad < a.pv.capacity && r > 0 && t < T;
  const uint16_t* Bb = (const uint16_t*)(live ? a.pv.base : a.pv.zeros) +
                       (live ? (long long)ad * a.pv.slot_elems + a.pv.b_offset : 0);
  const int bld = live ? round_up8(r) : 0;
  // a fused adapter over stacked projections: only the tile's slice window
  // of rank columns can be nonzero in its rows (from column jb, a multiple of 8)
  int jb = 0, je = r;
  if constexpr (SL) {
    int w0 = 0, w1 = r;
    if (live) slice_window(a.pv, tile * kDecRows, min(tile * kDecRows + kDecRows, d_out), r, &w0, &w1);
    jb = w0 & ~7;
    je = min(w1, r);
  }
  u32x4_t b8[kPre][4];
#pragma unroll
  for (int g = 0; g < kPre; ++g)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      b8[g][v] = ld16(Bb + (live ? bblk_off(min(n + v, d_out - 1), min(jb + 8 * g, bld - 8), d_out) : 0));

  // chunk partials summed in chunk order
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < kFinUnroll; ++u)
    if (u < a.n_chunks) {
      acc[0] += p[u][0];
      acc[1] += p[u][1];
      acc[2] += p[u][2];
      acc[3] += p[u][3];
    }
  for (int c0 = kFinUnroll; c0 < a.n_chunks; c0 += kFinUnroll) {
#pragma unroll
    for (int u = 0; u < kFinUnroll; ++u)
      p[u] = __builtin_nontemporal_load((const f32x4_t*)(pbase + min(c0 + u, a.n_chunks - 1) * cstride));
#pragma unroll
    for (int u = 0; u < kFinUnroll; ++u)
      if (c0 + u < a.n_chunks) {
        acc[0] += p[u][0];
        acc[1] += p[u][1];
        acc[2] += p[u][2];
        acc[3] += p[u][3];
      }
  }

  if constexpr (W8) {
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] *= wsc[v];
  }

  if (lora) {
    for (int e0 = 0; e0 < E; e0 += 256 / G) {
      const int g = tid % G;
      const float* vp = vptr(e0);
      f32x4_t sum = f32x4_t{0.f, 0.f, 0.f, 0.f};
      for (int s0 = g; s0 < nsl; s0 += G * kFinUnroll) {
        if (e0 > 0 || s0 > g) {
#pragma unroll
          for (int u = 0; u < kFinUnroll; ++u) vq[u] = *(const f32x4_t*)(vp + min(s0 + u * G, nsl - 1) * vstride);
        }
#pragma unroll
        for (int u = 0; u < kFinUnroll; ++u)
          if (s0 + u * G < nsl) {
            sum[0] += vq[u][0];
            sum[1] += vq[u][1];
            sum[2] += vq[u][2];
            sum[3] += vq[u][3];
          }
      }
      vgrp[g][tid / G] = sum;
      lds_barrier();   // LDS only: the B loads stay in flight
      if (tid < 256 / G && e0 + tid < E) {
        f32x4_t tot = vgrp[0][tid];
        for (int gg = 1; gg < G; ++gg) {
          tot[0] += vgrp[gg][tid][0];
          tot[1] += vgrp[gg][tid][1];
          tot[2] += vgrp[gg][tid][2];
          tot[3] += vgrp[gg][tid][3];
        }
        const int ee = e0 + tid;
        *(f32x4_t*)&vs[ee / nqv][4 * (q0 + ee % nqv)] = tot;
      }
      lds_barrier();
    }
    if (live) {
      const float* vv = vs[lane % 16];
      float lsum[4] = {0.f, 0.f, 0.f, 0.f};
      for (int j0 = jb; j0 < je; j0 += 8) {
        u32x4_t bq[4];
        if (j0 - jb < 8 * kPre) {
#pragma unroll
          for (int v = 0; v < 4; ++v) bq[v] = b8[j0 - jb < 8 ? 0 : kPre - 1][v];
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v) bq[v] = ld16(Bb + bblk_off(min(n + v, d_out - 1), j0, d_out));
        }
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t wd = bq[v][e / 2];
            const float bv = bf16_bits_to_f32((uint16_t)((e & 1) ? (wd >> 16) : (wd & 0xffffu)));
            // columns j >= r of B are zero in the pool; v there is unused
            lsum[v] = fmaf(bv, j0 + e < r ? vv[j0 + e] : 0.f, lsum[v]);
          }
      }
      const float sc = __int_as_float(pe.z);
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] += sc * lsum[v];
    }
  }

  if (t >= T) return;
  row = min(max(row, 0), T - 1);
  uint16_t* yr = (uint16_t*)a.y + (long long)row * d_out;
  if (n + 3 < d_out && (d_out & 3) == 0) {
    u32x2_t pk;
    pk.x = (uint32_t)f32_to_bf16_bits(acc[0]) | ((uint32_t)f32_to_bf16_bits(acc[1]) << 16);
    pk.y = (uint32_t)f32_to_bf16_bits(acc[2]) | ((uint32_t)f32_to_bf16_bits(acc[3]) << 16);
    *(u32x2_t*)(yr + n) = pk;
  } else {
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (n + v < d_out) yr[n + v] = f32_to_bf16_bits(acc[v]);
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
bool decode_supported(int T, int n_seg_bound, int d_out, int max_rank) {
  // k_stream gives each item at most one wave's worth (64) of shrink units
  const long long n_tiles = (d_out + kDecRows - 1) / kDecRows;
  const long long units16 = (long long)n_seg_bound * ((max_rank + 15) / 16);
  return T >= 1 && T <= 64 && n_seg_bound <= kDecMaxSeg && units16 <= kWave * n_tiles;
}

// Rows per shrink unit: the smallest of 4, 8, 16 whose units (one per segment
// and row group) fit one per item of a chunk, so the A rows spread over as
// many items as possible; 16 when none does.
int decode_unit_rows(int n_seg_bound, int max_rank, int n_tiles) {
  for (int ur = 4; ur < 16; ur *= 2)
    if ((long long)n_seg_bound * ((max_rank + ur - 1) / ur) <= n_tiles) return ur;
  return 16;
}

// d_in chunk: a multiple of 64 (at most the LDS x chunk), small enough that
// n_tiles * n_chunks covers the 256 CUs.
void decode_plan(int d_in, int d_out, int* n_tiles, int* kc, int* n_chunks) {
  *n_tiles = (d_out + kDecRows - 1) / kDecRows;
  int chunks = (d_in + kDecMaxKc - 1) / kDecMaxKc;
  while (*n_tiles * chunks < 256 && d_in / (chunks + 1) >= 256) ++chunks;
  int k = (d_in + chunks - 1) / chunks;
  k = (k + 63) / 64 * 64;
  if (k > kDecMaxKc) k = kDecMaxKc;
  *kc = k;
  *n_chunks = (d_in + k - 1) / k;
}

template <int TT, bool W8>
static void launch_decode_tt(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((k_stream_bf16<TT, W8>), dim3(a.n_tiles * a.n_chunks), dim3(kDecThreads), 0, st, a);
  if (a.lora_on && a.pv.n_slices > 0)
    hipLaunchKernelGGL((k_finish_bf16<TT, W8, true>), dim3(a.n_tiles * (TT / 16)), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_finish_bf16<TT, W8, false>), dim3(a.n_tiles * (TT / 16)), dim3(256), 0, st, a);
}

void launch_decode_bf16(const DecodeArgs& a, hipStream_t st) {
  const bool w8 = a.w_scale != nullptr;
  if (a.T <= 16) w8 ? launch_decode_tt<16, true>(a, st) : launch_decode_tt<16, false>(a, st);
  else if (a.T <= 32) w8 ? launch_decode_tt<32, true>(a, st) : launch_decode_tt<32, false>(a, st);
  else w8 ? launch_decode_tt<64, true>(a, st) : launch_decode_tt<64, false>(a, st);
}

}  // namespace mlora
