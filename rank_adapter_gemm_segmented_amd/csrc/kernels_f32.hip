// kernels_f32.hip -- fp32 multi-LoRA linear on the gfx950 vector ALUs.
//
// Same layer as the bf16 path (the LoRA forward of "Multi-LoRA Serving in
// Practice", section "Core Principle", per adapter segment), computed and
// stored in fp32. It serves small fp32 layers; the large configurations are
// bf16 and run on MFMA.
#include "common.h"
#include "launch.h"

namespace mlora {

// v_part[0][p][j] = sum_k A_a[j,k] x[row(p),k]; one workgroup per segment.
// Wave w takes positions ps + w, ps + w + 4, ...; for a position, groups of
// kF32Rows rank rows are read together (every load of the group in flight),
// the 64 lanes splitting d_in (16-byte loads, lane l at k = 4l + 256 i); each
// row's partial sums are added across the wave with xor shuffles (a fixed
// order).
constexpr int kF32Rows = 8;

__global__ __launch_bounds__(256) void k_shrink_f32(LinearArgs a) {
  const int s = blockIdx.x;
  const SegView& sv = a.sv;
  const int S = seg_count(sv);
  if (s >= S) return;
  const int ps = max(sv.seg_start[s], 0);
  const int pe = min(sv.seg_start[s + 1], a.T);
  if (pe <= ps) return;
  int r;
  const int ad = seg_adapter_checked(sv, a.pv, s, &r);
  if (ad < 0) return;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const float* __restrict__ x = (const float*)a.x;
  const float* __restrict__ Aa = (const float*)a.pv.base + (long long)ad * a.pv.slot_elems;
  const int d_in = a.d_in;   // a multiple of 4
  for (int p = ps + wave; p < pe; p += 4) {
    int row = sv.token_index ? sv.token_index[p] : p;
    row = min(max(row, 0), a.T - 1);
    const float* xr = x + (long long)row * d_in;
    for (int j0 = 0; j0 < r; j0 += kF32Rows) {
      float acc[kF32Rows];
#pragma unroll
      for (int i = 0; i < kF32Rows; ++i) acc[i] = 0.f;
      for (int k = 4 * lane; k < d_in; k += 4 * kWave) {
        const f32x4_t xv = *(const f32x4_t*)(xr + k);
        f32x4_t av[kF32Rows];
#pragma unroll
        for (int i = 0; i < kF32Rows; ++i) av[i] = *(const f32x4_t*)(Aa + (long long)min(j0 + i, r - 1) * d_in + k);
#pragma unroll
        for (int i = 0; i < kF32Rows; ++i)
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[i] = fmaf(av[i][c], xv[c], acc[i]);
      }
#pragma unroll
      for (int i = 0; i < kF32Rows; ++i) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) acc[i] += __shfl_xor(acc[i], off, kWave);
      }
      if (lane < kF32Rows && j0 + lane < r) {
        float v = acc[0];
#pragma unroll
        for (int i = 1; i < kF32Rows; ++i) v = lane == i ? acc[i] : v;
        a.v_part[(long long)p * a.r_ws + j0 + lane] = v;
      }
    }
  }
}

// Tile: 64 output features x 16 sorted positions; thread (tx, ty) owns feature
// n0+tx for positions 4*ty .. 4*ty+3. d_in is walked in chunks of kF32KB with
// the next chunk's loads in flight in registers while the current one is
// multiplied from LDS.
constexpr int kF32KB = 64;

__global__ __launch_bounds__(256) void k_gemm_f32(LinearArgs a) {
  __shared__ float Ws[64][kF32KB + 1];
  __shared__ float Xs[16][kF32KB + 1];
  const int tid = threadIdx.x;
  const int tx = tid % 64, ty = tid / 64;
  const int n0 = blockIdx.x * 64, p0 = blockIdx.y * 16;
  const int T = a.T, d_in = a.d_in, d_out = a.d_out;
  const float* __restrict__ x = (const float*)a.x;
  const float* __restrict__ W = (const float*)a.W;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};

  // loader: W chunk 64 x 64 = 1024 float4 (4 per thread), x chunk 16 x 64 =
  // 256 float4 (1 per thread); absent rows or columns load zeros
  const float* wsrc[4];
  int wr_[4], wc_[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = tid + 256 * i;
    wr_[i] = q / (kF32KB / 4);
    wc_[i] = 4 * (q % (kF32KB / 4));
    wsrc[i] = W + (long long)min(n0 + wr_[i], d_out - 1) * d_in + wc_[i];
  }
  const int xr_ = tid / (kF32KB / 4), xc_ = 4 * (tid % (kF32KB / 4));
  int xrow = min(p0 + xr_, T - 1);
  if (a.sv.token_index) xrow = min(max(a.sv.token_index[xrow], 0), T - 1);
  const float* xsrc = x + (long long)xrow * d_in + xc_;
  f32x4_t wreg[4], xreg;
  auto load = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = n0 + wr_[i] < d_out && kb + wc_[i] < d_in;
      wreg[i] = ok ? *(const f32x4_t*)(wsrc[i] + kb) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const bool ok = p0 + xr_ < T && kb + xc_ < d_in;
    xreg = ok ? *(const f32x4_t*)(xsrc + kb) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  };
  load(0);
  for (int kb = 0; kb < d_in; kb += kF32KB) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) Ws[wr_[i]][wc_[i] + c] = wreg[i][c];
#pragma unroll
    for (int c = 0; c < 4; ++c) Xs[xr_][xc_ + c] = xreg[c];
    __syncthreads();
    if (kb + kF32KB < d_in) load(kb + kF32KB);   // uniform
#pragma unroll 16
    for (int kk = 0; kk < kF32KB; ++kk) {
      const float w = Ws[tx][kk];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = fmaf(w, Xs[ty * 4 + q][kk], acc[q]);
    }
    __syncthreads();
  }

  const int n = n0 + tx;
  if (n >= d_out) return;
  const SegView& sv = a.sv;
  const int S = a.lora_on ? seg_count(sv) : 0;
  float* __restrict__ y = (float*)a.y;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int p = p0 + ty * 4 + q;
    if (p >= T) continue;
    float val = acc[q];
    if (S > 0) {
      const int s = find_segment(sv.seg_start, S, p);
      int r;
      const int ad = (sv.seg_start[s] <= p && p < sv.seg_start[s + 1])
                         ? seg_adapter_checked(sv, a.pv, s, &r) : -1;
      if (ad >= 0) {
        const float* Bb = (const float*)a.pv.base + (long long)ad * a.pv.slot_elems + a.pv.b_offset;
        const float* bn = Bb + (long long)n * round_up8(r);
        const float* vp = a.v_part + (long long)p * a.r_ws;
        float lora = 0.f;
        for (int j = 0; j < r; ++j) lora = fmaf(bn[j], vp[j], lora);
        val = fmaf(sv.seg_scale[s], lora, val);
      }
    }
    int row = sv.token_index ? sv.token_index[p] : p;
    row = min(max(row, 0), T - 1);
    y[(long long)row * d_out + n] = val;
  }
}

void launch_linear_f32(const LinearArgs& a, hipStream_t st) {
  if (a.lora_on && a.seg_grid > 0)
    hipLaunchKernelGGL(k_shrink_f32, dim3(a.seg_grid), dim3(256), 0, st, a);
  dim3 grid((a.d_out + 63) / 64, (a.T + 15) / 16);
  hipLaunchKernelGGL(k_gemm_f32, grid, dim3(256), 0, st, a);
}

}  // namespace mlora
