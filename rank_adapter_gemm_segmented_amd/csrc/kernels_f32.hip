// kernels_f32.hip -- fp32 multi-LoRA linear on the gfx950 vector ALUs.
//
// Same layer as the bf16 path (the LoRA forward of "Multi-LoRA Serving in
// Practice", section "Core Principle", per adapter segment), computed and
// stored in fp32. It serves small fp32 layers; the large configurations are
// bf16 and run on MFMA.
#include "common.h"
#include "launch.h"

namespace mlora {

// v_part[0][p][j] = sum_k A_a[j,k] x[row(p),k]; one workgroup per segment,
// which also writes its positions' entries of the position table.
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
  // the position table: {segment, adapter or -1, rank, scale bits}
  for (int p = ps + (int)threadIdx.x; p < pe; p += 256)
    a.pos_info[p] = make_int4(s, ad, ad >= 0 ? r : 0, __float_as_int(ad >= 0 ? sv.seg_scale[s] : 0.f));
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

// Tile: 16 output features x 16 sorted positions, one output per thread
// (tx = feature, ty = position), so a small layer spreads over many
// workgroups: the 256-wide layer of 16 tokens runs 16 of them (64-feature
// tiles ran 4, each issuing ~5000 LDS reads per wave: 10 us). d_in is walked
// in chunks of kF32KB columns with the next chunk's loads in flight in
// registers while the current one is multiplied from LDS; the chunk is wide
// (4 W and 4 x loads of 16 bytes per thread, all in flight at once), so a
// small layer loads everything in one round trip.
constexpr int kF32KB = 256;
constexpr int kF32Feat = 16;

__global__ __launch_bounds__(256) void k_gemm_f32(LinearArgs a) {
  __shared__ float Ws[kF32Feat][kF32KB + 1];
  __shared__ float Xs[16][kF32KB + 1];
  const int tid = threadIdx.x;
  const int tx = tid % kF32Feat, ty = tid / kF32Feat;
  const int n0 = blockIdx.x * kF32Feat, p0 = blockIdx.y * 16;
  const int T = a.T, d_in = a.d_in, d_out = a.d_out;
  const float* __restrict__ x = (const float*)a.x;
  const float* __restrict__ W = (const float*)a.W;
  float acc = 0.f;
  // loader: W chunk 16 x 256 and x chunk 16 x 256, 1024 float4 each (4 per
  // thread); absent rows or columns load zeros
  constexpr int N4 = 16 * kF32KB / 4 / 256;
  const float* wsrc[N4];
  const float* xsrc[N4];
  int lr_[N4], lc_[N4];
#pragma unroll
  for (int i = 0; i < N4; ++i) {
    const int q = tid + 256 * i;
    lr_[i] = q / (kF32KB / 4);
    lc_[i] = 4 * (q % (kF32KB / 4));
    wsrc[i] = W + (long long)min(n0 + lr_[i], d_out - 1) * d_in + lc_[i];
    int xrow = min(p0 + lr_[i], T - 1);
    if (a.sv.token_index) xrow = min(max(a.sv.token_index[xrow], 0), T - 1);
    xsrc[i] = x + (long long)xrow * d_in + lc_[i];
  }
  // this position's adapter entry, requested with the first chunk (the
  // epilogue's B and v loads then need no further round trip)
  const int p = p0 + ty;
  const int4 pe4 = a.lora_on ? a.pos_info[min(p, T - 1)] : make_int4(0, -1, 0, 0);
  f32x4_t wreg[N4], xreg[N4];
  auto load = [&](int kb) {
#pragma unroll
    for (int i = 0; i < N4; ++i) {
      const bool wok = n0 + lr_[i] < d_out && kb + lc_[i] < d_in;
      wreg[i] = wok ? *(const f32x4_t*)(wsrc[i] + kb) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      const bool xok = p0 + lr_[i] < T && kb + lc_[i] < d_in;
      xreg[i] = xok ? *(const f32x4_t*)(xsrc[i] + kb) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };
  load(0);
  for (int kb = 0; kb < d_in; kb += kF32KB) {
#pragma unroll
    for (int i = 0; i < N4; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        Ws[lr_[i]][lc_[i] + c] = wreg[i][c];
        Xs[lr_[i]][lc_[i] + c] = xreg[i][c];
      }
    __syncthreads();
    if (kb + kF32KB < d_in) load(kb + kF32KB);   // uniform
#pragma unroll 16
    for (int kk = 0; kk < kF32KB; ++kk) acc = fmaf(Ws[tx][kk], Xs[ty][kk], acc);
    __syncthreads();
  }
  const int n = n0 + tx;
  if (n >= d_out || p >= T) return;
  const SegView& sv = a.sv;
  float val = acc;
  const int ad = pe4.y, r = min(pe4.z, a.pv.max_rank);
  if (a.lora_on && ad >= 0 && ad < a.pv.capacity && r > 0) {
    const float* Bb = (const float*)a.pv.base + (long long)ad * a.pv.slot_elems + a.pv.b_offset;
    const float* bn = Bb + (long long)n * round_up8(r);
    const float* vp = a.v_part + (long long)p * a.r_ws;
    float lora = 0.f;
    for (int j = 0; j < r; ++j) lora = fmaf(bn[j], vp[j], lora);
    val = fmaf(__int_as_float(pe4.w), lora, val);
  }
  int row = sv.token_index ? sv.token_index[p] : p;
  row = min(max(row, 0), T - 1);
  ((float*)a.y)[(long long)row * d_out + n] = val;
}

void launch_linear_f32(const LinearArgs& a, hipStream_t st) {
  if (a.lora_on && a.seg_grid > 0)
    hipLaunchKernelGGL(k_shrink_f32, dim3(a.seg_grid), dim3(256), 0, st, a);
  dim3 grid((a.d_out + kF32Feat - 1) / kF32Feat, (a.T + 15) / 16);
  hipLaunchKernelGGL(k_gemm_f32, grid, dim3(256), 0, st, a);
}

}  // namespace mlora
