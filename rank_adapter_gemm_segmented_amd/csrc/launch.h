// launch.h -- host-side launchers of the gfx950 kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mlora.h"
#include "common.h"

namespace mlora {

// Arguments of one layer call after host validation.
struct LinearArgs {
  const void* x;
  const void* W;
  void* y;
  int T, d_in, d_out;
  int lora_on;
  SegView sv;
  PoolView pv;
  float* v_part;   // workspace: shrink partials [ks][T][r_ws] fp32
  float* v_fin;    // workspace: scale * v per sorted position [T][r_ws] fp32
  int4* pos_info;  // workspace: per sorted position {segment, adapter, rank, scale bits}
  int r_ws;        // row pitch of v_part (max_rank rounded up to 16)
  int ks;          // number of d_in chunks of the shrink (1..kMaxShrinkSplit)
  int seg_grid;    // number of segments to cover (upper bound)
  float* delta;    // workspace: dense adapter term [T][d_out] fp32 (k_expand_delta), or null
  int gorder;      // tiled GEMM block order (set by its launcher): 0 row tiles fastest,
                   // 1 XCD-grouped (row tiles per XCD, their position tiles adjacent),
                   // 2 one round in 2-D blocks per XCD (n_rt / 4 x n_tt / 2 tiles)
  int wnt;         // tiled GEMM: stage W rows by nontemporal loads (set by its launcher)
};

constexpr int kMaxShrinkSplit = 16;
constexpr int kMaxRankWs = 256;   // largest v row pitch (max_rank rounded up to 16)
constexpr int kDxMaxRank = 64;    // largest rank of the dense-term expand (k_expand_delta)
constexpr int kDxMaxT = 512;      // most tokens of a call whose workspace holds the dense term
constexpr size_t kDxMaxBytes = 16u << 20;   // and at most this many bytes of it

// Small-T (decode) path: split-K streaming kernel + finishing kernel.
constexpr int kDecMaxKc = 1024;   // largest d_in chunk per item
constexpr int kDecMaxSeg = 256;   // most segments the decode path handles

struct DecodeArgs {
  const void* x;
  const void* W;
  void* y;
  int T, d_in, d_out;
  int lora_on;
  SegView sv;
  PoolView pv;
  float* ypart;    // workspace: partial tiles [n_chunks][n_tiles][4][T/16 blocks][256]
  float* v_part;   // workspace: shrink partials [n_chunks][8 waves][T][r_ws]
  int4* pos;       // workspace: per sorted position {adapter or -1, rank, scale bits, 0} [T]
  int r_ws;
  int n_tiles;     // ceil(d_out / 64)
  int kc;          // d_in chunk width (multiple of 64)
  int n_chunks;    // ceil(d_in / kc)
  int unit_rows;   // rank rows per shrink unit (4, 8 or 16)
  const float* w_scale;   // FP8 weight: float32 scale per W row (W holds e4m3 codes); null: bf16 W
};

// Merge of one adapter into a base weight: W_out = W_in + scale * B A.
struct MergeArgs {
  const void* W_in;
  void* W_out;     // == W_in (in place) or disjoint
  const void* A;   // slot A [rank, d_in]
  const void* B;   // slot B: bf16 blocks of 16 rank columns (bblk_off); fp32 [d_out, pitch]; zero past the rank
  int d_in, d_out, rank, pitch;   // pitch: the rank rounded up to 8
  float scale;
};

// merge kernels (kernels_merge.hip)
void launch_merge(const MergeArgs& a, bool bf16, hipStream_t st);

// metadata kernels (kernels_meta.hip)
void launch_token_map(const int32_t* seg_start, const int32_t* seg_adapter, int T, int S,
                      int32_t* token_seg, int32_t* token_adapter, hipStream_t st);
size_t build_segments_lds_bytes(int T);
void launch_build_segments(const int32_t* token_adapter, const float* adapter_scale, int T,
                           const PoolView& pv, int32_t* token_index, int32_t* seg_start,
                           int32_t* seg_adapter, int32_t* seg_rank, float* seg_scale,
                           int32_t* n_seg_out, hipStream_t st);
void launch_validate(const int32_t* seg_start, const int32_t* seg_adapter, const int32_t* seg_rank,
                     const int32_t* token_index, int T, int S, const PoolView& pv, int32_t* counts,
                     int32_t* result, hipStream_t st);
void launch_fill_u32(void* p, size_t n_words, uint32_t v, hipStream_t st);
void launch_set_slot_rank(int32_t* table, int id, int rank, hipStream_t st);

// bf16 path for larger token counts (kernels_gemm.hip); the shrink alone
// (k_shrink_short, or k_shrink2 and k_vfinal when ks > 1) writes pos_info
// and v_fin
void launch_linear_bf16(const LinearArgs& a, hipStream_t st);
void launch_shrink_bf16(const LinearArgs& a, hipStream_t st);

// full-d_in GEMV with the expand for T <= 64 (kernels_gemv.hip); LoRA-on
// needs launch_shrink_bf16 first
void launch_gemv_bf16(const LinearArgs& a, hipStream_t st);
int choose_shrink_split_bf16(int d_in, int items);
int shrink_items_bound(int T, int n_seg_bound, int max_rank);
// true when the shrink of this call is k_shrink_short (else k_shrink2)
bool shrink_short(const LinearArgs& a);

// decode path (kernels_decode.hip)
bool decode_supported(int T, int n_seg_bound, int d_out, int max_rank);
int decode_unit_rows(int n_seg_bound, int max_rank, int n_tiles);
void decode_plan(int d_in, int d_out, int* n_tiles, int* kc, int* n_chunks);
void launch_decode_bf16(const DecodeArgs& a, hipStream_t st);

// fp32 path (kernels_f32.hip)
void launch_linear_f32(const LinearArgs& a, hipStream_t st);

}  // namespace mlora
