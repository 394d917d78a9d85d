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
constexpr int kDecRows = 64;                       // W rows per item (4 blocks of 16)
constexpr int kDecXPitch = kDecMaxKc + 8;          // LDS row pitch of the x chunk (bf16)
constexpr int kDecWSteps = kDecMaxKc / 2 / 32;     // 32-wide k-steps per wave (16)
constexpr int kDecASteps = kDecMaxKc / 8 / 32;     // shrink k-steps per wave per row block (4)

template <int TT>
struct DecSmem {
  uint16_t xs[TT * kDecXPitch];
  union {
    float red[4][kWave][4 * (TT / 16)];            // second-half partials of the W rows
    float vred[8][kWave][4];                       // shrink partials per wave
  } u;
  int pref[kDecMaxSeg + 1];                        // shrink-row prefix over segments
  int sad[kDecMaxSeg];                             // adapter of each segment (-1: none)
  int sps[kDecMaxSeg], spe[kDecMaxSeg];            // token range of each segment
  int rseg[16], rj[16];                            // current shrink row block: segment, rank row
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

  // ---- 2. W rows -> MFMA A-operand registers, every k-step at once ---------
  // wave w: row block rb = w % 4, k-half kh = w / 4 of the chunk
  const int rb = wave & 3, kh = wave >> 2;
  const int nrow = tile * kDecRows + rb * 16 + l16;
  const bool row_ok = nrow < d_out;
  const int half_steps = (nks + 1) / 2;
  const int ks_begin = kh ? half_steps : 0;
  const int ks_end = kh ? nks : half_steps;
  u32x4_t wr[kDecWSteps];
  {
    const uint16_t* wrow = W + (long long)(row_ok ? nrow : d_out - 1) * d_in + k0;
#pragma unroll
    for (int s = 0; s < kDecWSteps; ++s) {
      const int k = (ks_begin + s) * 32 + kq;
      const bool ok = row_ok && (ks_begin + s) < ks_end && k < kc;
      wr[s] = sel(ok, ld_nt16(wrow + (k < kc ? k : kc - 8)));
    }
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
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sg = lane * 4 + i;
      if (sg < nseg) sm.pref[sg] = run;
      run += rr[i];
    }
    if (lane == kWave - 1) sm.pref[nseg] = inc;   // total rows (nseg <= 256 = 4 * 64)
  }

  // ---- 5. x registers -> LDS -----------------------------------------------
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int t = tid / (kDecMaxKc / 8) + (kDecThreads / (kDecMaxKc / 8)) * i;
    *(u32x4_t*)&sm.xs[t * XP + xcol * 8] = xr[i];
  }
  __syncthreads();

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
    const int s = seg_of_row(sm.pref, nseg, qok ? q : q_begin);
    const int ad = sm.sad[s];
    const int j = (qok ? q : q_begin) - sm.pref[s];
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

  // ---- 6. base MFMAs --------------------------------------------------------
  f32x4_t acc[NTB];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) acc[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kDecWSteps; ++s) {
    const int ks = min(ks_begin + s, kDecMaxKc / 32 - 1);   // zero operands past ks_end
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      const u32x4_t xo = *(const u32x4_t*)&sm.xs[(tb * 16 + l16) * XP + ks * 32 + kq];
      acc[tb] = mfma16d(wr[s], xo, acc[tb]);
    }
  }
  // fixed-order sum of the two k-halves, then one coalesced fragment store
  if (kh == 1) {
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
      for (int v = 0; v < 4; ++v) sm.u.red[rb][lane][tb * 4 + v] = acc[tb][v];
  }
  __syncthreads();
  if (kh == 0) {
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      f32x4_t o;
#pragma unroll
      for (int v = 0; v < 4; ++v) o[v] = acc[tb][v] + sm.u.red[rb][lane][tb * 4 + v];
      *(f32x4_t*)(a.ypart + part_off(c, tile, rb, tb, a.n_tiles, NTB) + lane * 4) = o;
    }
  }
  if (q_begin >= q_end) return;   // uniform: no shrink rows in this item
  __syncthreads();                // red is reused as vred below

  // ---- 7. shrink row blocks -------------------------------------------------
  int buf = 0;
  for (int qb = q_begin; qb < q_end; qb += 16, buf ^= 1) {
    if (tid < 16) {   // row table of this block
      const int q = qb + tid;
      int s = -1, j = 0;
      if (q < q_end) {
        s = seg_of_row(sm.pref, nseg, q);
        j = q - sm.pref[s];
      }
      sm.rseg[tid] = s;
      sm.rj[tid] = j;
    }
    f32x4_t vacc[NTB];
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) vacc[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < kDecASteps; ++st) {
      const int ks = wave + 8 * st;   // always < 32; operands past the chunk are zero
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        const u32x4_t xo = *(const u32x4_t*)&sm.xs[(tb * 16 + l16) * XP + ks * 32 + kq];
        vacc[tb] = mfma16d(ar[buf][st], xo, vacc[tb]);
      }
    }
    if (qb + 32 < q_end) load_a(qb + 32, ar[buf]);   // refill this buffer two blocks ahead
    // reduce the 8 waves in a fixed order, one token block at a time
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
#pragma unroll
      for (int v = 0; v < 4; ++v) sm.u.vred[wave][lane][v] = vacc[tb][v];
      __syncthreads();
      if (tid < 256) {
        const int l = tid / 4, v = tid % 4;
        const int rr = 4 * (l / 16) + v;      // result row in the block = shrink row qb + rr
        const int t = tb * 16 + (l % 16);     // result column = sorted token position
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < 8; ++w) sum += sm.u.vred[w][l][v];
        const int s = sm.rseg[rr];
        if (s >= 0 && t >= sm.sps[s] && t < sm.spe[s])
          a.v_part[((long long)c * T + t) * a.r_ws + sm.rj[rr]] = sum;
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// finish: one workgroup per (n-tile, 16-token block); wave w = row block w.
// ---------------------------------------------------------------------------
constexpr int kFinUnroll = 8;

template <int TT>
__global__ __launch_bounds__(256) void k_finish_bf16(DecodeArgs a) {
  constexpr int NTB = TT / 16;
  const int tile = blockIdx.x / NTB, tb = blockIdx.x % NTB;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int T = a.T, d_out = a.d_out;
  const int rb = wave;
  __shared__ float vs[16][kMaxRankWs + 4];
  __shared__ int tseg[16], trank[16];
  __shared__ int sst[kDecMaxSeg + 1];

  // segment starts -> LDS (issued before the partial loads)
  const int S = a.lora_on ? min(seg_count(a.sv), kDecMaxSeg) : 0;
  for (int i = tid; i <= S && S > 0; i += 256) sst[i] = a.sv.seg_start[i];

  // the chunk partials, all loads in flight, summed in chunk order
  const float* pbase = a.ypart + part_off(0, tile, rb, tb, a.n_tiles, NTB) + lane * 4;
  const long long cstride = (long long)a.n_tiles * 4 * NTB * 256;
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < a.n_chunks; c0 += kFinUnroll) {
    f32x4_t p[kFinUnroll];
#pragma unroll
    for (int u = 0; u < kFinUnroll; ++u) {
      const int cc = min(c0 + u, a.n_chunks - 1);
      p[u] = *(const f32x4_t*)(pbase + cc * cstride);
    }
#pragma unroll
    for (int u = 0; u < kFinUnroll; ++u) {
      if (c0 + u < a.n_chunks) {
        acc[0] += p[u][0];
        acc[1] += p[u][1];
        acc[2] += p[u][2];
        acc[3] += p[u][3];
      }
    }
  }

  const int t = tb * 16 + (lane % 16);   // this lane's token (sorted position)
  const int n = tile * kDecRows + rb * 16 + 4 * (lane / 16);
  if (S > 0) {
    __syncthreads();
    if (tid < 16) {
      const int tt = tb * 16 + tid;
      int sg = -1, rk = 0;
      if (tt < T) {
        const int s = find_segment(sst, S, tt);
        if (sst[s] <= tt && tt < sst[s + 1]) {
          int r;
          if (seg_adapter_checked(a.sv, a.pv, s, &r) >= 0) { sg = s; rk = r; }
        }
      }
      tseg[tid] = sg;
      trank[tid] = rk;
    }
    __syncthreads();
    // stage scale * sum_c v_c for the 16 tokens
    for (int e = tid; e < 16 * a.r_ws; e += 256) {
      const int ti = e / a.r_ws, jj = e % a.r_ws;
      const int tt = tb * 16 + ti;
      const bool live = tseg[ti] >= 0 && jj < trank[ti];
      const float* vp = a.v_part + (long long)min(tt, T - 1) * a.r_ws + jj;
      const long long vstride = (long long)T * a.r_ws;
      float sum = 0.f;
      for (int c0 = 0; c0 < a.n_chunks; c0 += kFinUnroll) {
        float q[kFinUnroll];
#pragma unroll
        for (int u = 0; u < kFinUnroll; ++u) q[u] = vp[min(c0 + u, a.n_chunks - 1) * vstride];
#pragma unroll
        for (int u = 0; u < kFinUnroll; ++u)
          if (c0 + u < a.n_chunks) sum += q[u];
      }
      vs[ti][jj] = live ? sum * a.sv.seg_scale[tseg[ti]] : 0.f;
    }
    __syncthreads();
    const int sg = tseg[lane % 16];
    if (sg >= 0 && t < T) {
      const int r = trank[lane % 16];
      const int ad = a.sv.seg_adapter[sg];
      const int bld = round_up8(r);
      const uint16_t* Bb = (const uint16_t*)a.pv.base + (long long)ad * a.pv.slot_elems + a.pv.b_offset;
      const float* vv = vs[lane % 16];
      float lsum[4] = {0.f, 0.f, 0.f, 0.f};
      for (int j0 = 0; j0 < r; j0 += 8) {
        u32x4_t b8[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) b8[v] = ld16(Bb + (long long)min(n + v, d_out - 1) * bld + j0);
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t wd = b8[v][e / 2];
            const float bv = bf16_bits_to_f32((uint16_t)((e & 1) ? (wd >> 16) : (wd & 0xffffu)));
            lsum[v] = fmaf(bv, vv[j0 + e], lsum[v]);   // vv[j >= r] is 0
          }
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] += lsum[v];
    }
  }

  if (t >= T) return;
  int row = a.sv.token_index ? a.sv.token_index[t] : t;
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
