// kernels_gemv.hip -- bf16 multi-LoRA linear for small token counts as a
// full-d_in GEMV on gfx950: one launch for the base product and the expand.
//
// y_i = W x_i + scale_s * B_a (A_a x_i) ("Multi-LoRA Serving in Practice",
// section "Core Principle", displayed formula), per adapter segment
// ("InvisibleLoRA" abstract). LoRA-on, the shrink runs first (k_shrink2 with
// one d_in chunk writes scale * v per sorted position and the position table);
// this kernel then adds the expand in its epilogue, so y is written once.
//
// k_gemv: one workgroup of 8 waves per 16 W rows over the whole of d_in.
// Wave w takes k-steps w, w + 8, w + 16, ... of 32 columns; each k-step loads
// the 16 W rows' 32 columns and the tile's tokens' 32 columns of x straight
// into v_mfma_f32_16x16x32_bf16 operand registers (no LDS), with a ring of
// 6 or 8 k-steps of loads in flight. The eight waves' partial sums meet in
// LDS and are added in wave order (deterministic). The position table, the
// scale * v rows and the first B rows of the expand are requested before the
// k-loop, so they land while W streams.
//
// MFMA 16x16x32 bf16 layout: lane l supplies row l%16 and k-slots
// 8*(l/16)..+7 of each operand; result register v of lane l is row
// 4*(l/16)+v, column l%16. Rows are W rows (output features), columns are
// tokens, so a lane ends with 4 consecutive features of one token.
#include "common.h"
#include "launch.h"

namespace mlora {

namespace {

constexpr int kGvThreads = 512;            // 8 waves
constexpr int kGvWaves = kGvThreads / kWave;
constexpr int kGvRows = 16;                // W rows per workgroup
constexpr int kGvPre = 2;                  // 8-wide rank groups of B and v requested early

__device__ __forceinline__ f32x4_t mfma16v(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

template <int TT>
__global__ __launch_bounds__(kGvThreads) void k_gemv_bf16(LinearArgs a) {
  constexpr int NTB = TT / 16;
  // k-steps of loads in flight per wave (5 16-byte loads per step at 64
  // tokens: the ring then takes 120 of the 256 registers a lane has)
  constexpr int kGvRing = TT == 64 ? 6 : 8;
  __shared__ float red[kGvWaves][NTB][kWave][4];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int l16 = lane % 16, kq = 8 * (lane / 16);
  const int T = a.T, d_in = a.d_in, d_out = a.d_out;
  const int n0 = blockIdx.x * kGvRows;
  const uint16_t* __restrict__ W = (const uint16_t*)a.W;
  const uint16_t* __restrict__ x = (const uint16_t*)a.x;
  const uint16_t* zeros = (const uint16_t*)a.pv.zeros;
  const bool lora = a.lora_on != 0;

  // ---- epilogue operands first (waves 0 .. NTB-1: token block = wave) ------
  // lane: sorted position p = 16 wave + l16, rows n0 + 4 (l / 16) + 0..3
  const bool epi = wave < NTB;
  const int p = 16 * (epi ? wave : 0) + l16;
  const bool p_ok = epi && p < T;
  int4 pi = make_int4(0, -1, 0, 0);
  if (lora && p_ok) pi = a.pos_info[p];
  const int nb = n0 + 4 * (lane / 16);      // first of the lane's 4 rows
  // B rows and scale * v of the first kGvPre rank groups (absent: zero block)
  u32x4_t bq[kGvPre][4];
  f32x4_t vq[kGvPre][2];
  const int ad = pi.y, rk = (ad >= 0 && ad < a.pv.capacity) ? min(pi.z, a.pv.max_rank) : 0;
  const uint16_t* brow0 = rk > 0 ? (const uint16_t*)a.pv.base + (long long)ad * a.pv.slot_elems + a.pv.b_offset
                                 : zeros;
  const float* vrow = a.v_fin + (long long)min(p, max(T - 1, 0)) * a.r_ws;
#pragma unroll
  for (int g = 0; g < kGvPre; ++g) {
    const bool on = 8 * g < rk;
#pragma unroll
    for (int v = 0; v < 4; ++v)
      bq[g][v] = ld16(on ? brow0 + bblk_off(min(nb + v, d_out - 1), 8 * g, d_out) : zeros);
    vq[g][0] = on ? *(const f32x4_t*)(vrow + 8 * g) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    vq[g][1] = on ? *(const f32x4_t*)(vrow + 8 * g + 4) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // ---- base product: ring of kGvRing k-steps per wave -----------------------
  const uint16_t* wrow = W + (long long)min(n0 + l16, d_out - 1) * d_in;
  const uint16_t* xrow[NTB];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    const int q = min(16 * tb + l16, T - 1);
    int row = a.sv.token_index ? a.sv.token_index[q] : q;
    row = min(max(row, 0), T - 1);
    xrow[tb] = x + (long long)row * d_in;
  }
  const int nks = (d_in + 31) / 32;
  const int steps = (nks + kGvWaves - 1) / kGvWaves;             // per wave, uniform
  const int iters = (steps + kGvRing - 1) / kGvRing;
  u32x4_t wq[kGvRing], xq[kGvRing][NTB];
  // step i of this wave is k-step wave + 8 i; past d_in every load reads the
  // zero block (an address select: each load is unconditional, so the
  // compiler's waits in the ring stay exact)
  auto load = [&](int i, int slot) {
    const int k = (wave + kGvWaves * i) * 32 + kq;
    const bool ok = k < d_in;
    wq[slot] = ld_nt16(ok ? wrow + k : zeros);
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) xq[slot][tb] = ld16(ok ? xrow[tb] + k : zeros);
  };
#pragma unroll
  for (int s = 0; s < kGvRing; ++s) load(s, s);
  f32x4_t acc[NTB];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) acc[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < kGvRing; ++s) {
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) acc[tb] = mfma16v(wq[s], xq[s][tb], acc[tb]);
      load((it + 1) * kGvRing + s, s);
    }
  }

  // ---- fixed-order sum of the waves -----------------------------------------
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) *(f32x4_t*)red[wave][tb][lane] = acc[tb];
  __syncthreads();
  if (!epi) return;
  f32x4_t y = *(const f32x4_t*)red[0][wave][lane];
#pragma unroll
  for (int w = 1; w < kGvWaves; ++w) {
    const f32x4_t o = *(const f32x4_t*)red[w][wave][lane];
#pragma unroll
    for (int v = 0; v < 4; ++v) y[v] += o[v];
  }

  // ---- expand: y += B_a (scale v), 8 rank entries at a time -----------------
  if (lora && rk > 0) {
    f32x4_t e = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto group = [&](const u32x4_t* b, const f32x4_t* vv) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          s += bf16_bits_to_f32((uint16_t)(b[v][j >> 1] >> (16 * (j & 1)))) * vv[j >> 2][j & 3];
        e[v] += s;
      }
    };
#pragma unroll
    for (int g = 0; g < kGvPre; ++g) group(bq[g], vq[g]);
    for (int g = kGvPre; 8 * g < rk; ++g) {
      u32x4_t b[4];
      f32x4_t vv[2];
#pragma unroll
      for (int v = 0; v < 4; ++v) b[v] = ld16(brow0 + bblk_off(min(nb + v, d_out - 1), 8 * g, d_out));
      vv[0] = *(const f32x4_t*)(vrow + 8 * g);
      vv[1] = *(const f32x4_t*)(vrow + 8 * g + 4);
      group(b, vv);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) y[v] += e[v];
  }

  // ---- store: 4 consecutive features of one token, rounded once -----------
  if (!p_ok) return;
  int row = a.sv.token_index ? a.sv.token_index[p] : p;
  row = min(max(row, 0), T - 1);
  uint16_t* dst = (uint16_t*)a.y + (long long)row * d_out + nb;
  if (nb + 4 <= d_out && (d_out & 3) == 0) {
    u32x2_t pk;
    pk.x = (uint32_t)f32_to_bf16_bits(y[0]) | ((uint32_t)f32_to_bf16_bits(y[1]) << 16);
    pk.y = (uint32_t)f32_to_bf16_bits(y[2]) | ((uint32_t)f32_to_bf16_bits(y[3]) << 16);
    *(u32x2_t*)dst = pk;
  } else {
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (nb + v < d_out) dst[v] = f32_to_bf16_bits(y[v]);
  }
}

}  // namespace

void launch_gemv_bf16(const LinearArgs& a, hipStream_t st) {
  const dim3 grid((a.d_out + kGvRows - 1) / kGvRows);
  if (a.T <= 16) hipLaunchKernelGGL(k_gemv_bf16<16>, grid, dim3(kGvThreads), 0, st, a);
  else if (a.T <= 32) hipLaunchKernelGGL(k_gemv_bf16<32>, grid, dim3(kGvThreads), 0, st, a);
  else hipLaunchKernelGGL(k_gemv_bf16<64>, grid, dim3(kGvThreads), 0, st, a);
}

}  // namespace mlora
