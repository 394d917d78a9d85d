// kernels_bf16.hip -- bf16 multi-LoRA linear on gfx950 MFMA.
//
// y_i = W x_i + scale_s * B_a (A_a x_i): the LoRA forward of "Multi-LoRA
// Serving in Practice", section "Core Principle" (displayed formula), with the
// batch partitioned into per-adapter segments ("InvisibleLoRA" abstract).
//
// Two launches:
//   k_shrink_bf16  v = A_a x over each segment, fp32, split over d_in chunks
//                  into deterministic partials (no atomics);
//   k_gemm_bf16    base W x on v_mfma_f32_16x16x32_bf16 with W streamed once
//                  from HBM straight into MFMA operand registers and x staged
//                  in LDS; the epilogue adds scale * B_a v on the same MFMA
//                  accumulators (v split into a bf16 high and low part so the
//                  fp32 intermediate keeps ~16 mantissa bits) and stores y once.
//
// MFMA operand layout used throughout (16x16x32 bf16, wave64): lane l supplies
// row (l % 16) and k-slots 8*(l/16) .. 8*(l/16)+7 of each operand; the result
// element for lane l, register v is row 4*(l/16)+v, column l % 16.
#include "common.h"
#include "launch.h"

namespace mlora {

__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Shrink: v_part[c][p][j] = sum_{k in chunk c} A_a[j,k] x[row(p),k]
// grid (segments, d_in chunks), 4 waves; each wave takes every 4th 32-wide
// k-step of the chunk, waves are summed in a fixed order through LDS.
// MFMA rows = sorted positions (16 per block), columns = rank index j.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_shrink_bf16(LinearArgs a) {
  const int s = blockIdx.x, c = blockIdx.y;
  const SegView& sv = a.sv;
  const int S = seg_count(sv);
  if (s >= S) return;
  const int ps = max(sv.seg_start[s], 0);
  const int pe = min(sv.seg_start[s + 1], a.T);
  if (pe <= ps) return;
  int r;
  const int ad = seg_adapter_checked(sv, a.pv, s, &r);
  if (ad < 0) return;

  const uint16_t* __restrict__ x = (const uint16_t*)a.x;
  const uint16_t* __restrict__ Aa = (const uint16_t*)a.pv.base + (long long)ad * a.pv.slot_elems;
  const int d_in = a.d_in;
  const int nks = (d_in + 31) / 32;
  const int kb = (int)((long long)c * nks / a.ks);
  const int ke = (int)((long long)(c + 1) * nks / a.ks);

  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int l16 = lane % 16, kq = 8 * (lane / 16);
  __shared__ float red[4][kWave][17];

  for (int pb = ps; pb < pe; pb += 64) {
    // batch rows of this wave's four 16-position blocks (fixed over k)
    const uint16_t* xrow[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int p = pb + rb * 16 + l16;
      xrow[rb] = nullptr;
      if (p < pe) {
        int row = sv.token_index ? sv.token_index[p] : p;
        row = min(max(row, 0), a.T - 1);
        xrow[rb] = x + (long long)row * d_in;
      }
    }
    for (int jg = 0; jg < r; jg += 64) {
      f32x4_t acc[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

      for (int ksi = kb + wave; ksi < ke; ksi += 4) {
        const int k = ksi * 32 + kq;
        const bool kv = k < d_in;
        u32x4_t xo[4], ao[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) xo[rb] = (kv && xrow[rb]) ? ld16(xrow[rb] + k) : zero_u32x4();
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const int j = jg + cb * 16 + l16;
          ao[cb] = (kv && j < r) ? ld16(Aa + (long long)j * d_in + k) : zero_u32x4();
        }
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          if (pb + rb * 16 >= pe) continue;  // wave-uniform
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            if (jg + cb * 16 >= r) continue;  // wave-uniform
            acc[rb][cb] = mfma16(xo[rb], ao[cb], acc[rb][cb]);
          }
        }
      }
      // fixed-order sum of the four waves, one 16-position block at a time
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        if (pb + rb * 16 >= pe) break;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int v = 0; v < 4; ++v) red[wave][lane][cb * 4 + v] = acc[rb][cb][v];
        __syncthreads();
        for (int e = threadIdx.x; e < kWave * 16; e += 256) {
          const int l = e / 16, q = e % 16, cb = q / 4, v = q % 4;
          const int p = pb + rb * 16 + 4 * (l / 16) + v;
          const int j = jg + cb * 16 + (l % 16);
          const float sum = ((red[0][l][q] + red[1][l][q]) + red[2][l][q]) + red[3][l][q];
          if (p < pe && j < r) a.v_part[((long long)c * a.T + p) * a.r_ws + j] = sum;
        }
        __syncthreads();
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Base GEMM + fused expand.
// Tile: 64 rows of W (4 waves x 16) x TT sorted positions. W rows go straight
// from HBM into MFMA A-operand registers (each W byte is read once overall);
// x rows (gathered through token_index) are staged in LDS, double-buffered.
// ---------------------------------------------------------------------------
constexpr int kKB = 64;            // k per pipeline stage (two MFMA k-steps)
constexpr int kXPitch = kKB + 8;   // LDS row pitch of the x stage, in bf16

template <int TT>
struct GemmSmem {
  union {
    uint16_t xs[2][TT * kXPitch];
    float vs[TT * 36];             // epilogue: scale * v for 32 rank columns
  } u;
  int pseg[TT];
  int prank[TT];
  float pscale[TT];
};

template <int TT>
__global__ __launch_bounds__(256) void k_gemm_bf16(LinearArgs a) {
  constexpr int NTB = TT / 16;
  constexpr int NCH = (TT * (kKB / 8) + 255) / 256;  // 16-byte x chunks per thread per stage
  __shared__ __attribute__((aligned(16))) GemmSmem<TT> sm;

  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int l16 = lane % 16, kq = 8 * (lane / 16);
  const int n0 = blockIdx.x * 64 + wave * 16;
  const int p0 = blockIdx.y * TT;
  const int T = a.T, d_in = a.d_in, d_out = a.d_out;
  const uint16_t* __restrict__ x = (const uint16_t*)a.x;
  const uint16_t* __restrict__ W = (const uint16_t*)a.W;

  const int nrow = n0 + l16;
  const bool row_ok = nrow < d_out;
  const uint16_t* wrow = W + (long long)(row_ok ? nrow : 0) * d_in;

  // x chunk assignment: chunk = tid + 256*i -> tile row chunk/8, 16-byte column chunk%8
  const uint16_t* xsrc[NCH];
  int xdst[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int ch = threadIdx.x + 256 * i;
    const int tr = ch / 8, cc = ch % 8;
    xsrc[i] = nullptr;
    xdst[i] = -1;
    if (tr < TT) {
      xdst[i] = tr * kXPitch + cc * 8;
      const int p = p0 + tr;
      if (p < T) {
        int row = a.sv.token_index ? a.sv.token_index[p] : p;
        row = min(max(row, 0), T - 1);
        xsrc[i] = x + (long long)row * d_in + cc * 8;
      }
    }
  }

  f32x4_t acc[NTB];
#pragma unroll
  for (int i = 0; i < NTB; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nst = (d_in + kKB - 1) / kKB;
  u32x4_t xr[NCH];
  auto load_x = [&](int st) {
    const int kb = st * kKB;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int k = kb + (threadIdx.x + 256 * i) % 8 * 8;
      xr[i] = (xsrc[i] && k < d_in) ? ld16(xsrc[i] + kb) : zero_u32x4();
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NCH; ++i)
      if (xdst[i] >= 0) *(u32x4_t*)&sm.u.xs[buf][xdst[i]] = xr[i];
  };
  auto load_w = [&](int st, u32x4_t* w) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int k = st * kKB + kk * 32 + kq;
      w[kk] = (row_ok && k < d_in) ? ld_nt16(wrow + k) : zero_u32x4();
    }
  };

  u32x4_t wc[2], wn[2];
  load_x(0);
  load_w(0, wc);
  store_x(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const bool more = st + 1 < nst;
    if (more) {
      load_w(st + 1, wn);
      load_x(st + 1);
    }
    const uint16_t* xb = sm.u.xs[st & 1];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        const u32x4_t xo = *(const u32x4_t*)&xb[(tb * 16 + l16) * kXPitch + kk * 32 + kq];
        acc[tb] = mfma16(wc[kk], xo, acc[tb]);
      }
    }
    if (more) store_x((st + 1) & 1);
    __syncthreads();
    wc[0] = wn[0];
    wc[1] = wn[1];
  }

  if (a.lora_on) {
    // per-position segment info
    const SegView& sv = a.sv;
    const int S = seg_count(sv);
    for (int t = threadIdx.x; t < TT; t += 256) {
      const int p = p0 + t;
      int sg = -1, rk = 0;
      float sc = 0.f;
      if (p < T && S > 0) {
        const int s = find_segment(sv.seg_start, S, p);
        if (sv.seg_start[s] <= p && p < sv.seg_start[s + 1]) {
          int r;
          if (seg_adapter_checked(sv, a.pv, s, &r) >= 0) {
            sg = s;
            rk = r;
            sc = sv.seg_scale[s];
          }
        }
      }
      sm.pseg[t] = sg;
      sm.prank[t] = rk;
      sm.pscale[t] = sc;
    }
    __syncthreads();
    for (int jc = 0; jc < a.r_ws; jc += 32) {
      // stage scale * sum_c v_part[c][p][jc..jc+31]
      for (int e = threadIdx.x; e < TT * 32; e += 256) {
        const int t = e / 32, jj = e % 32, j = jc + jj;
        float val = 0.f;
        if (sm.pseg[t] >= 0 && j < sm.prank[t]) {
          const long long base = (long long)(p0 + t) * a.r_ws + j;
          float sum = 0.f;
          for (int c = 0; c < a.ks; ++c) sum += a.v_part[(long long)c * T * a.r_ws + base];
          val = sum * sm.pscale[t];
        }
        sm.u.vs[t * 36 + jj] = val;
      }
      __syncthreads();
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        const int tb0 = tb * 16;
        if (p0 + tb0 >= T) break;
        int t = tb0;
        const int tend = min(tb0 + 16, T - p0);
        while (t < tend) {  // runs of equal segment (wave-uniform)
          const int sg = sm.pseg[t];
          int u = t + 1;
          while (u < tend && sm.pseg[u] == sg) ++u;
          if (sg >= 0 && jc < sm.prank[t]) {
            const int r = sm.prank[t];
            const int ad = sv.seg_adapter[sg];
            const uint16_t* Bb = (const uint16_t*)a.pv.base + (long long)ad * a.pv.slot_elems +
                                 a.pv.b_offset;
            const int bld = round_up8(r);
            const int j = jc + kq;
            const u32x4_t bop = (row_ok && j < r) ? ld16(Bb + (long long)nrow * bld + j) : zero_u32x4();
            const int tl = tb0 + l16;
            float vv[8], vl[8];
            const bool in = tl >= t && tl < u;
#pragma unroll
            for (int e = 0; e < 8; ++e) vv[e] = in ? sm.u.vs[tl * 36 + kq + e] : 0.f;
            const bf16x8_t hi = pack_bf16x8(vv);
            const u32x4_t hiu = __builtin_bit_cast(u32x4_t, hi);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const uint16_t hb = (uint16_t)((e & 1) ? (hiu[e / 2] >> 16) : (hiu[e / 2] & 0xffffu));
              vl[e] = vv[e] - bf16_bits_to_f32(hb);
            }
            const bf16x8_t lo = pack_bf16x8(vl);
            acc[tb] = mfma16(bop, hiu, acc[tb]);
            acc[tb] = mfma16(bop, __builtin_bit_cast(u32x4_t, lo), acc[tb]);
          }
          t = u;
        }
      }
      __syncthreads();
    }
  }

  // store y (bf16, RNE), rows scattered through token_index
  uint16_t* __restrict__ y = (uint16_t*)a.y;
  const int nb = n0 + 4 * (lane / 16);
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    const int p = p0 + tb * 16 + l16;
    if (p >= T) continue;
    int row = a.sv.token_index ? a.sv.token_index[p] : p;
    row = min(max(row, 0), T - 1);
    uint16_t* yr = y + (long long)row * d_out;
    if (nb + 3 < d_out && (d_out & 3) == 0) {
      u32x2_t pk;
      pk.x = (uint32_t)f32_to_bf16_bits(acc[tb][0]) | ((uint32_t)f32_to_bf16_bits(acc[tb][1]) << 16);
      pk.y = (uint32_t)f32_to_bf16_bits(acc[tb][2]) | ((uint32_t)f32_to_bf16_bits(acc[tb][3]) << 16);
      *(u32x2_t*)(yr + nb) = pk;
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (nb + v < d_out) yr[nb + v] = f32_to_bf16_bits(acc[tb][v]);
    }
  }
}

int choose_shrink_split_bf16(int d_in, int seg_grid) {
  const int nks = (d_in + 31) / 32;
  int ks = 1;
  while (ks < kMaxShrinkSplit && seg_grid * ks < 512 && nks / (ks * 2) >= 8) ks *= 2;
  return ks;
}

template <int TT>
static void launch_gemm(const LinearArgs& a, hipStream_t st) {
  dim3 grid((a.d_out + 63) / 64, (a.T + TT - 1) / TT);
  hipLaunchKernelGGL(k_gemm_bf16<TT>, grid, dim3(256), 0, st, a);
}

void launch_linear_bf16(const LinearArgs& a, hipStream_t st) {
  if (a.lora_on && a.seg_grid > 0)
    hipLaunchKernelGGL(k_shrink_bf16, dim3(a.seg_grid, a.ks), dim3(256), 0, st, a);
  if (a.T <= 16) launch_gemm<16>(a, st);
  else if (a.T <= 32) launch_gemm<32>(a, st);
  else if (a.T <= 64) launch_gemm<64>(a, st);
  else launch_gemm<128>(a, st);
}

}  // namespace mlora
