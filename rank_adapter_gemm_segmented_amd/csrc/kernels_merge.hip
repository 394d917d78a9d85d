// kernels_merge.hip -- merge (or unmerge) one adapter into a base weight on gfx950:
//
//     W_out = W_in + c * B_a A_a        (W [d_out, d_in], A_a [r, d_in], B_a [d_out, r])
//
// The "LoRA Inference" glossary (first paragraph) merges an adapter into the
// frozen weights, W = W0 + dW; the update of one adapter is the low-rank term
// of the "Multi-LoRA Serving in Practice" LoRA forward (section "Core
// Principle", displayed formula), so dW = c B A. c < 0 unmerges.
//
// bf16 (k_merge_bf16): one workgroup of 4 waves per 64-row x 128-column tile
// of W, 4 waves per SIMD resident. The kernel streams W once in and once out
// (HBM bound); dW is a K = rank contraction on v_mfma_f32_32x32x16_bf16:
//  1. each thread requests its four 16-byte pieces of the W tile first;
//  2. per rank chunk of 64: the A chunk [64 rank rows x 128 columns] is
//     loaded coalesced and stored to LDS as loaded (zero past the rank). An
//     MFMA operand (8 rank entries of one column) is gathered with 2-byte LDS
//     reads; a transposed store of 2-byte pieces measured slower, since its
//     lanes fall on few banks. The B rows of the tile's 64 W rows are loaded
//     straight into MFMA operand registers (8 consecutive rank entries are
//     one 16-byte load: a bf16 pool stores B in blocks of 16 rank columns,
//     zero past the rank; an fp32 pool in rows zero-padded to a multiple of 8).
//     Wave w multiplies columns 32w..32w+31 (MFMA rows) against the tile's
//     two 32-row blocks (MFMA columns);
//  3. c * dW (fp32) goes to an LDS tile [64][128]; each thread adds it to its
//     W pieces in fp32, rounds once (RNE) and stores 16 bytes. W is read
//     and written once, so both streams bypass the cache's keep policy
//     (nontemporal loads and stores): 2-8% faster than cached stores.
// MFMA 32x32x16 bf16 layout: lane l supplies row l%32 and k-slots
// 8*(l/32)..+7 of each operand; result register v of lane l is row
// 8*(v/4)+4*(l/32)+v%4, column l%32.
//
// fp32 (k_merge_f32): one thread per 4 consecutive columns of one row, rank
// loop on VALU.
//
// W_out may be W_in (in place): every 16-byte piece of W is read and written
// by the same thread only.
#include "common.h"
#include "launch.h"

namespace mlora {

namespace {

constexpr int kMgRows = 64;                  // W rows per tile
constexpr int kMgCols = 128;                 // W columns per tile
constexpr int kMgRc = 64;                    // rank rows per chunk
constexpr int kMgAsPitch = kMgCols + 8;      // bf16 per staged A row (272 bytes)
constexpr int kMgDPitch = kMgCols + 4;       // floats per delta-tile row
constexpr int kMgAsBytes = kMgRc * kMgAsPitch * 2;
constexpr int kMgDBytes = kMgRows * kMgDPitch * 4;
constexpr int kMgLds = kMgAsBytes > kMgDBytes ? kMgAsBytes : kMgDBytes;

__device__ __forceinline__ f32x16_t mfma32m(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_merge_bf16(MergeArgs a) {
  __shared__ __align__(16) char lds[kMgLds];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k0 = blockIdx.x * kMgCols, n0 = blockIdx.y * kMgRows;
  const int d_in = a.d_in, d_out = a.d_out, rank = a.rank, pitch = a.pitch;
  const uint16_t* Win = (const uint16_t*)a.W_in;   // may alias W_out: each piece has one owner thread
  const uint16_t* __restrict__ A = (const uint16_t*)a.A;
  const uint16_t* __restrict__ B = (const uint16_t*)a.B;

  // 1. the W tile: piece i of thread t is row (t + 256 i) / 16, columns 8 * ((t + 256 i) % 16)..+7
  u32x4_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + 256 * i;
    const int n = n0 + (idx >> 4), col = k0 + 8 * (idx & 15);
    w[i] = (n < d_out && col < d_in) ? ld_nt16(Win + (long long)n * d_in + col) : zero_u32x4();
  }

  // 2. dW on MFMA, rank chunk by rank chunk
  f32x16_t acc[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[nb][v] = 0.f;
  uint16_t* As = (uint16_t*)lds;
  // B rows of this lane's two MFMA columns; rows past d_out are clamped (their results are dropped)
  const int nrow0 = min(n0 + (lane & 31), d_out - 1);
  const int nrow1 = min(n0 + 32 + (lane & 31), d_out - 1);
  for (int jc = 0; jc < rank; jc += kMgRc) {
    const int kr = min(kMgRc, rank - jc);      // rank rows in this chunk
    u32x4_t av[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      const int j = idx >> 4;
      const int col = min(k0 + 8 * (idx & 15), d_in - 8);   // columns past d_in are dropped
      av[i] = j < kr ? ld16(A + (long long)(jc + j) * d_in + col) : zero_u32x4();
    }
    if (jc) __syncthreads();                   // the previous chunk's LDS reads are done
    // rows of the chunk as loaded (16-byte stores, no bank conflicts); only the
    // rank rows the MFMAs read (zero from kr up to the next multiple of 16)
    const int kr16 = (kr + 15) & ~15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      if (16 * i >= kr16) break;               // rows 16 i .. 16 i + 15 of the chunk
      *(u32x4_t*)(As + (idx >> 4) * kMgAsPitch + 8 * (idx & 15)) = av[i];
    }
    // B operands after the A registers are free (they are L2 hits: every column tile reads them)
    u32x4_t bv[4][2];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int jj = jc + 16 * s + 8 * (lane >> 5);
      const bool on = 16 * s < kr && jj < pitch;
      bv[s][0] = on ? ld16(B + bblk_off(nrow0, jj, d_out)) : zero_u32x4();
      bv[s][1] = on ? ld16(B + bblk_off(nrow1, jj, d_out)) : zero_u32x4();
    }
    __syncthreads();
    const int mcol = 32 * wave + (lane & 31);  // this lane's MFMA row: a W column of the tile
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (16 * s >= kr) break;
      // 8 consecutive rank entries of one column: 2-byte LDS reads down the column
      const uint16_t* col = As + (16 * s + 8 * (lane >> 5)) * kMgAsPitch + mcol;
      u32x4_t am;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        am[e] = (uint32_t)col[(2 * e) * kMgAsPitch] | ((uint32_t)col[(2 * e + 1) * kMgAsPitch] << 16);
      acc[0] = mfma32m(am, bv[s][0], acc[0]);
      acc[1] = mfma32m(am, bv[s][1], acc[1]);
    }
  }

  // 3. c * dW through LDS, added to the W pieces, one rounding
  __syncthreads();                             // every wave's A reads are done
  float* D = (float*)lds;
  const float c = a.scale;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4_t d;
#pragma unroll
      for (int e = 0; e < 4; ++e) d[e] = c * acc[nb][4 * q + e];
      *(f32x4_t*)(D + (32 * nb + (lane & 31)) * kMgDPitch + 32 * wave + 8 * q + 4 * (lane >> 5)) = d;
    }
  __syncthreads();
  uint16_t* Wout = (uint16_t*)a.W_out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + 256 * i;
    const int row = idx >> 4, c8 = idx & 15;
    const int n = n0 + row, col = k0 + 8 * c8;
    if (n >= d_out || col >= d_in) continue;
    const f32x4_t d0 = *(const f32x4_t*)(D + row * kMgDPitch + 8 * c8);
    const f32x4_t d1 = *(const f32x4_t*)(D + row * kMgDPitch + 8 * c8 + 4);
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float we = bf16_bits_to_f32((uint16_t)(w[i][e >> 1] >> (16 * (e & 1))));
      o[e] = we + (e < 4 ? d0[e] : d1[e - 4]);
    }
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, pack_bf16x8(o)),
                                (u32x4_t*)(Wout + (long long)n * d_in + col));
  }
}

__global__ __launch_bounds__(256) void k_merge_f32(MergeArgs a) {
  const int n = blockIdx.x;
  const int k = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (k >= a.d_in) return;
  const float* __restrict__ A = (const float*)a.A;
  const float* __restrict__ Bn = (const float*)a.B + (long long)n * a.pitch;
  const f32x4_t w = *(const f32x4_t*)((const float*)a.W_in + (long long)n * a.d_in + k);
  f32x4_t d = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < a.rank; ++j) {
    const float b = Bn[j];
    const f32x4_t av = *(const f32x4_t*)(A + (long long)j * a.d_in + k);
#pragma unroll
    for (int e = 0; e < 4; ++e) d[e] = fmaf(b, av[e], d[e]);
  }
  f32x4_t o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = w[e] + a.scale * d[e];
  *(f32x4_t*)((float*)a.W_out + (long long)n * a.d_in + k) = o;
}

}  // namespace

void launch_merge(const MergeArgs& a, bool bf16, hipStream_t st) {
  if (bf16) {
    const dim3 grid((a.d_in + kMgCols - 1) / kMgCols, (a.d_out + kMgRows - 1) / kMgRows);
    hipLaunchKernelGGL(k_merge_bf16, grid, dim3(256), 0, st, a);
  } else {
    const dim3 grid(a.d_out, (a.d_in / 4 + 255) / 256);
    hipLaunchKernelGGL(k_merge_f32, grid, dim3(256), 0, st, a);
  }
}

}  // namespace mlora
