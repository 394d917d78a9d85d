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
  const float* __restrict__ x = (const float*)a.x;
  const float* __restrict__ Aa = (const float*)a.pv.base + (long long)ad * a.pv.slot_elems;
  const int d_in = a.d_in;
  const int npairs = (pe - ps) * r;
  for (int e = threadIdx.x; e < npairs; e += blockDim.x) {
    const int p = ps + e / r, j = e % r;
    int row = sv.token_index ? sv.token_index[p] : p;
    row = min(max(row, 0), a.T - 1);
    const float* xr = x + (long long)row * d_in;
    const float* aj = Aa + (long long)j * d_in;
    float acc = 0.f;
    for (int k = 0; k < d_in; ++k) acc = fmaf(aj[k], xr[k], acc);
    a.v_part[(long long)p * a.r_ws + j] = acc;
  }
}

// Tile: 64 output features x 16 sorted positions; thread (tx, ty) owns feature
// n0+tx for positions 4*ty .. 4*ty+3.
constexpr int kF32KB = 32;

__global__ __launch_bounds__(256) void k_gemm_f32(LinearArgs a) {
  __shared__ float Ws[64][kF32KB + 1];
  __shared__ float Xs[16][kF32KB + 1];
  const int tx = threadIdx.x % 64, ty = threadIdx.x / 64;
  const int n0 = blockIdx.x * 64, p0 = blockIdx.y * 16;
  const int T = a.T, d_in = a.d_in, d_out = a.d_out;
  const float* __restrict__ x = (const float*)a.x;
  const float* __restrict__ W = (const float*)a.W;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};

  for (int kb = 0; kb < d_in; kb += kF32KB) {
    for (int e = threadIdx.x; e < 64 * kF32KB; e += 256) {
      const int r = e / kF32KB, kk = e % kF32KB;
      const int n = n0 + r, k = kb + kk;
      Ws[r][kk] = (n < d_out && k < d_in) ? W[(long long)n * d_in + k] : 0.f;
    }
    for (int e = threadIdx.x; e < 16 * kF32KB; e += 256) {
      const int t = e / kF32KB, kk = e % kF32KB;
      const int p = p0 + t, k = kb + kk;
      float v = 0.f;
      if (p < T && k < d_in) {
        int row = a.sv.token_index ? a.sv.token_index[p] : p;
        row = min(max(row, 0), T - 1);
        v = x[(long long)row * d_in + k];
      }
      Xs[t][kk] = v;
    }
    __syncthreads();
#pragma unroll 8
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
