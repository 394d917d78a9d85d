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
//            v_mfma_f32_16x16x32_bf16. The shrink v = A_a x is folded in as
//            extra rows: the touched adapters' A rows (restricted to chunk c)
//            are spread evenly over the items of chunk c and multiplied
//            against the same x chunk in LDS. Outputs: fp32 partial tiles of
//            W x and of v, one slot per chunk (deterministic, no atomics).
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
constexpr int kDecWPre = 8;                        // W k-steps requested before the MFMA loop
constexpr int kDecRowWin = 32;                     // shrink rows per item found by table lookup
constexpr int kDecASteps = kDecMaxKc / 8 / 32;     // shrink k-steps per wave per row block (4)

template <int TT>
struct DecSmem {
  uint16_t xs[TT * kDecXPitch];
  float red[4][kWave][4 * (TT / 16)];              // second-half partials of the W rows
  int pref[kDecMaxSeg + 1];                        // shrink-row prefix over segments
  int sad[kDecMaxSeg];                             // adapter of each segment (-1: none)
  int sps[kDecMaxSeg], spe[kDecMaxSeg];            // token range of each segment
  int rseg[kDecRowWin], rj[kDecRowWin];            // item's first shrink rows: segment, rank row
  int posseg[64];                                  // segment of each sorted position (-1: none)
};

// Partial tile layout (fragment-major): for chunk c, n-tile i, row block rb,
// token block tb: 256 floats ordered [lane][4].
__device__ __forceinline__ long long part_off(int c, int i, int rb, int tb, int n_tiles, int ntb) {
  return ((((long long)c * n_tiles + i) * 4 + rb) * ntb + tb) * 256;
}

// segment s holding shrink row q (pref is non-decreasing, pref[0] = 0 <= q)
__device__ __forceinline__ int seg_of_row(const int* pref, int nseg, int q) {
  int lo = 0, hi = nseg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pref[mid] <= q) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Loads below are unconditional from clamped addresses, with the value
// selected afterwards: branch-free code keeps the compiler's vmcnt waits exact,
// so MFMAs start on the first W k-step while later ones are still in flight.
__device__ __forceinline__ u32x4_t sel(bool keep, u32x4_t v) { return keep ? v : zero_u32x4(); }

template <int TT>
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

  // ---- 0. segment metadata: the last wave builds the segment table --------
  // Its loads go first in that wave's queue (branch-free, clamped indices), so
  // the wait for them does not wait for the x and W loads issued after them.
  constexpr int kMetaWave = kDecThreads / kWave - 1;
  const int nseg = lora ? min(seg_count(a.sv), kDecMaxSeg) : 0;
  int m_st[5] = {0, 0, 0, 0, 0}, m_ad[4] = {-1, -1, -1, -1}, m_r[4] = {0, 0, 0, 0};
  if (lora && wave == kMetaWave && nseg > 0) {   // wave-uniform branch
#pragma unroll
    for (int i = 0; i < 5; ++i) m_st[i] = a.sv.seg_start[min(lane * 4 + i, nseg)];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = min(lane * 4 + i, nseg - 1);
      m_ad[i] = a.sv.seg_adapter[s];
      m_r[i] = a.sv.seg_rank[s];
    }
  }

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
    xr[i] = sel(t < T && xcol_ok, ld16(x + (long long)xrow[i] * d_in + xk));
  }

  // ---- 3. segment table and shrink-row prefix (one wave, no block barrier) -
  if (lora && wave == kMetaWave) {
    // lane owns segments 4*lane .. 4*lane+3; rows to shrink per segment are its
    // rank capped by the slot size (the slot table is read by k_finish, which
    // drops emptied slots)
    int rr[4], tot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sg = lane * 4 + i;
      const int ps = max(m_st[i], 0), pe = min(m_st[i + 1], T);
      const bool ok = sg < nseg && pe > ps && m_ad[i] >= 0 && m_ad[i] < a.pv.capacity && m_r[i] > 0;
      rr[i] = ok ? min(m_r[i], a.pv.max_rank) : 0;
      tot += rr[i];
      if (sg < nseg) {
        sm.sad[sg] = ok ? m_ad[i] : -1;
        sm.sps[sg] = ps;
        sm.spe[sg] = pe;
      }
    }
    // inclusive wave scan of the lane totals
    int inc = tot;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int up = __shfl_up(inc, off, kWave);
      if (lane >= off) inc += up;
    }
    int run = inc - tot;
    int p0[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sg = lane * 4 + i;
      p0[i] = run;
      if (sg < nseg) sm.pref[sg] = run;
      run += rr[i];
    }
    if (lane == kWave - 1) sm.pref[nseg] = inc;   // total rows (nseg <= 256 = 4 * 64)
    // Direct lookup tables by scatter, so no lane needs a search later: the
    // segment and rank row of the item's first kDecRowWin shrink rows, and the
    // segment of every sorted position (item 0 writes the position table).
    const int rtot = __shfl(inc, kWave - 1, kWave);
    const int qb0 = (int)((long long)tile * rtot / a.n_tiles);
    const int qe0 = min((int)((long long)(tile + 1) * rtot / a.n_tiles), qb0 + kDecRowWin);
    if (lane < T) sm.posseg[lane] = -1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sg = lane * 4 + i;
      for (int q = max(p0[i], qb0); q < min(p0[i] + rr[i], qe0); ++q) {
        sm.rseg[q - qb0] = sg;
        sm.rj[q - qb0] = q - p0[i];
      }
      if (sg < nseg)
        for (int q = max(m_st[i], 0); q < min(m_st[i + 1], T); ++q) sm.posseg[q] = sg;
    }
  }

  // ---- 5. x registers -> LDS -----------------------------------------------
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int t = tid / (kDecMaxKc / 8) + (kDecThreads / (kDecMaxKc / 8)) * i;
    *(u32x4_t*)&sm.xs[t * XP + xcol * 8] = xr[i];
  }
  __syncthreads();

  // ---- 2. W rows -> MFMA A-operand registers --------------------------------
  // wave w: row block rb = w % 4, k-half kh = w / 4 of the chunk. The first
  // kDecWPre k-steps are requested now; the MFMA loop requests one more step
  // per step it consumes, so the MFMAs run while W streams in instead of
  // after the wave has finished issuing the whole chunk. W is requested only
  // once x is in LDS: x's misses would otherwise queue behind the W stream of
  // every CU. Addresses past the chunk or d_out are clamped into the row:
  // their products meet zero x columns or land in discarded rows; steps that
  // belong to the other k-half read zeros. No select on a loaded value.
  const int rb = wave & 3, kh = wave >> 2;
  const int nrow = tile * kDecRows + rb * 16 + l16;
  const int half_steps = (nks + 1) / 2;
  const int ks_begin = kh ? half_steps : 0;
  const int ks_end = kh ? nks : half_steps;
  const uint16_t* wrow = W + (long long)min(nrow, d_out - 1) * d_in + k0;
  u32x4_t wr[kDecWSteps];
  auto load_w = [&](int s) {
    // steps of the other k-half read the pool's zero block (address select)
    const int k = (ks_begin + s) * 32 + kq;
    wr[s] = ld_nt16(ks_begin + s < ks_end ? wrow + min(k, kc - 8) : (const uint16_t*)a.pv.zeros + kq);
  };
#pragma unroll
  for (int s = 0; s < kDecWPre; ++s) load_w(s);

  // ---- per-position table for k_finish ------------------------------------
  // One item resolves every sorted position's segment once (adapter checked
  // against the pool's slot table, rank, scale), so the finish kernel reads
  // one entry per token instead of walking the metadata. Its loads are issued
  // here and only waited for after the W MFMAs.
  const bool pos_writer = lora && blockIdx.x == 0 && tid < T;
  int pos_ad = -1, pos_r = 0, pos_s = 0;
  float pos_sc = 0.f;
  if (pos_writer) {
    const int sg = sm.posseg[tid];
    pos_s = sg >= 0 ? sg : 0;
    pos_ad = sg >= 0 ? sm.sad[sg] : -1;
    pos_r = a.pv.rank[pos_ad >= 0 ? pos_ad : 0];   // registered rank; used after the MFMAs
    pos_sc = a.sv.seg_scale[pos_s];
  }

  // ---- 4. shrink rows of this item: first two blocks of A rows -------------
  // (after the barrier: the segment table is in LDS; these loads overlap the
  // W MFMAs below)
  const int R = lora ? sm.pref[nseg] : 0;
  const int q_begin = (int)((long long)tile * R / a.n_tiles);
  const int q_end = (int)((long long)(tile + 1) * R / a.n_tiles);
  u32x4_t ar[2][kDecASteps];
  auto load_a = [&](int qb, u32x4_t* dst) {
    // no select on the loaded value (it would wait for the load right away):
    // an absent row reads the pool's zero block, and k past the chunk reads a
    // clamped in-row address whose product meets zero x in LDS
    const int q = qb + l16;
    const bool qok = q < q_end;
    const int qq = qok ? q : q_begin;
    int s, j;
    if (qb + 16 <= q_begin + kDecRowWin) {   // uniform: rows in the lookup window
      // (the entry is unset when the item has no rows: qok is false then)
      s = qok ? min(max(sm.rseg[qq - q_begin], 0), kDecMaxSeg - 1) : 0;
      j = sm.rj[qq - q_begin];
    } else {
      s = seg_of_row(sm.pref, nseg, qq);
      j = qq - sm.pref[s];
    }
    const int ad = qok ? sm.sad[s] : -1;
    const bool rok = qok && nseg > 0 && ad >= 0;
    const uint16_t* arow = rok ? (const uint16_t*)a.pv.base + (long long)ad * a.pv.slot_elems +
                                     (long long)j * d_in + k0
                               : (const uint16_t*)a.pv.zeros;
    const int klim = rok ? kc - 8 : kZeroBlockElems - 8;
#pragma unroll
    for (int st = 0; st < kDecASteps; ++st) {
      const int k = (wave + 8 * st) * 32 + kq;
      dst[st] = ld16(arow + min(k, klim));
    }
  };
  // issued unconditionally (rows past q_end read zeros): a branch here would
  // make the compiler's waits for the W loads below conservative
  load_a(q_begin, ar[0]);
  load_a(q_begin + 16, ar[1]);

  // output rows of shrink block qb held by this lane (qb + 4*(lane/16) + v):
  // segment, rank row, token range, and the token blocks the block covers.
  // Computed for the first block here, while the W loads are in flight.
  struct RowInfo { int os[4], oj[4], o0[4], o1[4], tb_lo, tb_hi; };
  auto row_info = [&](int qb) {
    RowInfo ri;
    int tlo = T, thi = 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int q = qb + 4 * (lane / 16) + v;
      ri.os[v] = -1;
      ri.oj[v] = 0;
      ri.o0[v] = 0;
      ri.o1[v] = 0;
      if (q < q_end) {
        int sg, jj;
        if (qb + 16 <= q_begin + kDecRowWin) {   // uniform: rows in the lookup window
          sg = sm.rseg[q - q_begin];
          jj = sm.rj[q - q_begin];
        } else {
          sg = seg_of_row(sm.pref, nseg, q);
          jj = q - sm.pref[sg];
        }
        ri.os[v] = sg;
        ri.oj[v] = jj;
        ri.o0[v] = sm.sps[sg];
        ri.o1[v] = sm.spe[sg];
        tlo = min(tlo, ri.o0[v]);
        thi = max(thi, ri.o1[v]);
      }
    }
    // wave-uniform range: lanes 0, 16, 32 and 48 hold the block's 16 rows
    tlo = min(tlo, __shfl_xor(tlo, 16, kWave));
    tlo = min(tlo, __shfl_xor(tlo, 32, kWave));
    thi = max(thi, __shfl_xor(thi, 16, kWave));
    thi = max(thi, __shfl_xor(thi, 32, kWave));
    ri.tb_lo = tlo / 16;
    ri.tb_hi = thi > tlo ? (thi - 1) / 16 : ri.tb_lo - 1;
    return ri;
  };
  RowInfo ri0 = row_info(q_begin);

  // ---- 6. base MFMAs --------------------------------------------------------
  f32x4_t acc[NTB];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) acc[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kDecWSteps; ++s) {
    if (s + kDecWPre < kDecWSteps) load_w(s + kDecWPre);
    // x columns past ks_end (past the chunk) are zero in LDS; k-steps past
    // the LDS chunk are clamped onto such columns
    const int ks = min(ks_begin + s, kDecMaxKc / 32 - 1);
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      const u32x4_t xo = *(const u32x4_t*)&sm.xs[(tb * 16 + l16) * XP + ks * 32 + kq];
      acc[tb] = mfma16d(wr[s], xo, acc[tb]);
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
      *(f32x4_t*)(a.ypart + part_off(c, tile, rb, tb, a.n_tiles, NTB) + lane * 4) = o;
    }
  }
  if (pos_writer) {
    const int r = pos_ad >= 0 ? min(sm.pref[pos_s + 1] - sm.pref[pos_s], pos_r) : 0;
    const int ad = r > 0 ? pos_ad : -1;
    a.pos[tid] = make_int4(ad, ad >= 0 ? r : 0, __float_as_int(ad >= 0 ? pos_sc : 0.f), 0);
  }
  if (q_begin >= q_end) return;   // uniform: no shrink rows in this item

  // ---- 7. shrink row blocks -------------------------------------------------
  // Each wave writes its own k-slice of the block straight to
  // v_part[c][wave][t][j] (k_finish sums the 8 * n_chunks slices in a fixed
  // order): no barrier after the W MFMAs.
  int buf = 0;
  for (int qb = q_begin; qb < q_end; qb += 16, buf ^= 1) {
    const RowInfo ri = qb == q_begin ? ri0 : row_info(qb);
    const int tb_lo = ri.tb_lo, tb_hi = ri.tb_hi;
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
        vacc[tb] = mfma16d(ar[buf][st], xo, vacc[tb]);
      }
    }
    if (qb + 32 < q_end) load_a(qb + 32, ar[buf]);   // refill this buffer two blocks ahead
    float* vp = a.v_part + ((long long)c * kDecWaves + wave) * T * a.r_ws;
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      if (tb < tb_lo || tb > tb_hi) continue;
      const int t = tb * 16 + l16;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (ri.os[v] >= 0 && t >= ri.o0[v] && t < ri.o1[v]) vp[(long long)t * a.r_ws + ri.oj[v]] = vacc[tb][v];
    }
  }
}

// ---------------------------------------------------------------------------
// finish: one workgroup per (n-tile, 16-token block); wave w = row block w.
// Every load that does not depend on the adapter id is issued first (chunk
// partials, v partials, the position table, token_index); the B rows follow
// once the lane's adapter is known.
// ---------------------------------------------------------------------------
constexpr int kFinUnroll = 8;

template <int TT>
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

  // the chunk partials, all loads in flight
  const float* pbase = a.ypart + part_off(0, tile, rb, tb, a.n_tiles, NTB) + lane * 4;
  const long long cstride = (long long)a.n_tiles * 4 * NTB * 256;
  f32x4_t p[kFinUnroll];
#pragma unroll
  for (int u = 0; u < kFinUnroll; ++u) p[u] = *(const f32x4_t*)(pbase + min(u, a.n_chunks - 1) * cstride);

  // B rows of the lane's adapter (first 16 rank columns), as soon as the
  // position entry is in
  const int ad = pe.x, r = min(pe.y, a.pv.max_rank);
  const bool live = lora && ad >= 0 && ad < a.pv.capacity && r > 0 && t < T;
  const uint16_t* Bb = (const uint16_t*)(live ? a.pv.base : a.pv.zeros) +
                       (live ? (long long)ad * a.pv.slot_elems + a.pv.b_offset : 0);
  const int bld = live ? round_up8(r) : 0;
  u32x4_t b8[kPre][4];
#pragma unroll
  for (int g = 0; g < kPre; ++g)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      b8[g][v] = ld16(Bb + (live ? (long long)min(n + v, d_out - 1) * bld + min(8 * g, bld - 8) : 0));

  // v of the 16 tokens: sum of the stream kernel's slices [c][w]. A 16-byte
  // quad of one token is element e; G groups of threads each sum every G-th
  // slice of an element, then the groups are added in group order. The first
  // batch of slice loads is issued here, with the partials still in flight.
  const int nq = a.r_ws / 4;
  const int E = 16 * nq;
  const int G = E >= 256 ? 1 : E >= 128 ? 2 : 4;
  const int nsl = a.n_chunks * kDecWaves;
  const long long vstride = (long long)T * a.r_ws;
  auto vptr = [&](int e0) {
    const int e = min(e0 + tid / G, E - 1);
    return a.v_part + (long long)min(tb * 16 + e / nq, T - 1) * a.r_ws + 4 * (e % nq);
  };
  f32x4_t vq[kFinUnroll];
  if (lora) {
    const float* vp = vptr(0);
#pragma unroll
    for (int u = 0; u < kFinUnroll; ++u) vq[u] = *(const f32x4_t*)(vp + min(tid % G + u * G, nsl - 1) * vstride);
  }

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
    for (int u = 0; u < kFinUnroll; ++u) p[u] = *(const f32x4_t*)(pbase + min(c0 + u, a.n_chunks - 1) * cstride);
#pragma unroll
    for (int u = 0; u < kFinUnroll; ++u)
      if (c0 + u < a.n_chunks) {
        acc[0] += p[u][0];
        acc[1] += p[u][1];
        acc[2] += p[u][2];
        acc[3] += p[u][3];
      }
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
      __syncthreads();
      if (tid < 256 / G && e0 + tid < E) {
        f32x4_t tot = vgrp[0][tid];
        for (int gg = 1; gg < G; ++gg) {
          tot[0] += vgrp[gg][tid][0];
          tot[1] += vgrp[gg][tid][1];
          tot[2] += vgrp[gg][tid][2];
          tot[3] += vgrp[gg][tid][3];
        }
        const int ee = e0 + tid;
        *(f32x4_t*)&vs[ee / nq][4 * (ee % nq)] = tot;
      }
      __syncthreads();
    }
    if (live) {
      const float* vv = vs[lane % 16];
      float lsum[4] = {0.f, 0.f, 0.f, 0.f};
      for (int j0 = 0; j0 < r; j0 += 8) {
        u32x4_t bq[4];
        if (j0 < 8 * kPre) {
#pragma unroll
          for (int v = 0; v < 4; ++v) bq[v] = b8[j0 / 8 == 0 ? 0 : kPre - 1][v];
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v) bq[v] = ld16(Bb + (long long)min(n + v, d_out - 1) * bld + j0);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t wd = bq[v][e / 2];
            const float bv = bf16_bits_to_f32((uint16_t)((e & 1) ? (wd >> 16) : (wd & 0xffffu)));
            // columns j >= r of the padded B row are zero; v there is unused
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
bool decode_supported(int T, int n_seg_bound) {
  return T >= 1 && T <= 64 && n_seg_bound <= kDecMaxSeg;
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

template <int TT>
static void launch_decode_tt(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_stream_bf16<TT>, dim3(a.n_tiles * a.n_chunks), dim3(kDecThreads), 0, st, a);
  hipLaunchKernelGGL(k_finish_bf16<TT>, dim3(a.n_tiles * (TT / 16)), dim3(256), 0, st, a);
}

void launch_decode_bf16(const DecodeArgs& a, hipStream_t st) {
  if (a.T <= 16) launch_decode_tt<16>(a, st);
  else if (a.T <= 32) launch_decode_tt<32>(a, st);
  else launch_decode_tt<64>(a, st);
}

}  // namespace mlora
