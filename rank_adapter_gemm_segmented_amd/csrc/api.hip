// api.hip -- the exported C ABI (include/mlora.h): adapter pool, workspace,
// host-side validation and kernel dispatch, plus the device scratch array of
// the entry point that allocates nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/mlora.h"
#include "launch.h"

using namespace mlora;

struct mlora_pool_s {
  void* base = nullptr;
  size_t bytes = 0;
  int d_in = 0, d_out = 0, dtype = 0, max_rank = 0, capacity = 0;
  size_t elem = 0;
  long long slot_elems = 0;  // elements per slot (multiple of 128)
  long long b_offset = 0;    // elements from slot start to B
  int32_t* dev_rank = nullptr;
  void* zeros = nullptr;     // kZeroBytes of zeros, never written after creation
  std::vector<int> host_rank;
  // 0: no adapter registered yet; 1: plain adapters; 2: fused adapters over
  // stacked projections (the pool keeps the row slicing of its first one)
  int kind = 0;
  int n_slices = 0;          // row slicing of a fused pool (0: none)
  int slice_end[MLORA_MAX_SLICES] = {};
  bool slice_uniform = true; // every fused adapter so far has equal slice ranks
};

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kZeroBytes = 4096;   // zero block at the end of the pool arena

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

size_t elem_size(int dtype) { return dtype == MLORA_F32 ? 4 : dtype == MLORA_BF16 ? 2 : 0; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Slot geometry: A [max_rank, d_in] then B. bf16 pools store B in blocks of
// 16 rank columns ([round_up16(max_rank) / 16][d_out][16], see bblk_off);
// fp32 pools as rows of round_up8(rank) columns ([d_out][round_up8(max_rank)]).
void slot_geometry(int d_in, int d_out, int max_rank, int dtype, long long* slot_elems, long long* b_off) {
  const long long a_elems = (long long)max_rank * d_in;
  const long long b_elems = (long long)d_out * (dtype == MLORA_BF16 ? (max_rank + 15) & ~15 : (max_rank + 7) & ~7);
  *b_off = (a_elems + 127) / 128 * 128;
  *slot_elems = (*b_off + b_elems + 127) / 128 * 128;
}

bool shape_ok(int d_in, int d_out, int dtype, int max_rank, int capacity) {
  if (elem_size(dtype) == 0) return false;
  if (d_in < 1 || d_in > MLORA_MAX_DIM || d_out < 1 || d_out > MLORA_MAX_DIM) return false;
  if (d_in % (dtype == MLORA_F32 ? 4 : 8) != 0) return false;
  if (max_rank < 1 || max_rank > MLORA_MAX_RANK) return false;
  if (capacity < 1 || capacity > (1 << 20)) return false;
  return true;
}

// Workspace layout for up to T tokens.
struct WsLayout {
  size_t err, token_index, seg_start, seg_adapter, seg_rank, seg_scale, n_seg, counts, v_part,
      ypart, pos_info, v_fin, delta, total;
};

int r_ws_of(int max_rank) { return (max_rank + 15) / 16 * 16; }

// Bytes of the dense adapter term [T][d_out] fp32 of k_expand_delta: bf16
// pools, up to kDxMaxT tokens and kDxMaxBytes, otherwise none.
size_t delta_bytes(const mlora_pool_s* p, int T) {
  if (p->dtype != MLORA_BF16 || T > kDxMaxT) return 0;
  const size_t b = (size_t)T * p->d_out * 4;
  return b <= kDxMaxBytes ? b : 0;
}

// the largest token count up to max_tokens that still has a dense-term region
int delta_tokens_max(const mlora_pool_s* p, int max_tokens) {
  if (p->dtype != MLORA_BF16) return 0;
  const long long by_bytes = (long long)(kDxMaxBytes / ((size_t)p->d_out * 4));
  long long t = max_tokens < kDxMaxT ? max_tokens : kDxMaxT;
  return (int)(t < by_bytes ? t : by_bytes);
}

WsLayout ws_layout(const mlora_pool_s* p, int T) {
  WsLayout L;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, kAlign); return at; };
  const size_t t1 = (size_t)T + 2;
  L.err = take(16);
  L.token_index = take(t1 * 4);
  L.seg_start = take(t1 * 4);
  L.seg_adapter = take(t1 * 4);
  L.seg_rank = take(t1 * 4);
  L.seg_scale = take(t1 * 4);
  L.n_seg = take(16);
  L.counts = take(t1 * 4);
  int n_tiles = 0, kc = 0, n_chunks = 0;
  decode_plan(p->d_in, p->d_out, &n_tiles, &kc, &n_chunks);
  // shrink partial slices: split-K of the large-T path (at most
  // kMaxShrinkSplit), and at T <= 64 also 8 waves per d_in chunk of the
  // decode stream
  const int dec_splits = n_chunks * 8;
  const int splits = T <= 64 && dec_splits > kMaxShrinkSplit ? dec_splits : kMaxShrinkSplit;
  L.v_part = take((size_t)splits * T * r_ws_of(p->max_rank) * 4);
  // decode partial tiles, only for token counts the decode path takes
  const size_t tt = T <= 16 ? 16 : T <= 32 ? 32 : 64;
  L.ypart = take(p->dtype == MLORA_BF16 && T <= 64 ? (size_t)n_chunks * n_tiles * 64 * tt * 4 : 0);
  L.pos_info = take((size_t)T * 16);
  L.v_fin = take((size_t)T * r_ws_of(p->max_rank) * 4);
  L.delta = take(delta_bytes(p, T));
  L.total = o;
  return L;
}

PoolView view_of(const mlora_pool_s* p) {
  PoolView v;
  v.base = p->base;
  v.zeros = p->zeros;
  v.rank = p->dev_rank;
  v.slot_elems = p->slot_elems;
  v.b_offset = p->b_offset;
  v.capacity = p->capacity;
  v.max_rank = p->max_rank;
  v.n_slices = (p->kind == 2 && p->slice_uniform) ? p->n_slices : 0;
  for (int m = 0; m < 8; ++m) v.slice_end[m] = m < p->n_slices ? p->slice_end[m] : 0;
  return v;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MLORA_OK : MLORA_ERR_HIP; }

// MLORA_FORCE_PATH=decode|gemm overrides the bf16 path choice (for tests and
// measurements); unset or anything else chooses by token count.
int forced_path() {
  const char* e = getenv("MLORA_FORCE_PATH");
  if (!e) return 0;
  return !strcmp(e, "decode") ? 1 : !strcmp(e, "gemm") ? 2 : !strcmp(e, "gemv") ? 3 : 0;
}

int check_launch() { return hip_status(hipGetLastError()); }

// MLORA_LOG=1: one line on stderr per layer call: the path taken and its sizes.
bool log_calls() {
  const char* e = getenv("MLORA_LOG");
  return e && e[0] == '1' && e[1] == 0;
}

void log_call(const char* path, int T, const mlora_pool_s* p, const SegView& sv, int lora_on, int ks,
              const char* shrink = "none") {
  fprintf(stderr,
          "mlora: path=%s T=%d d_in=%d d_out=%d dtype=%s lora_on=%d segments=%d%s ks=%d shrink=%s max_rank=%d\n",
          path, T, p->d_in, p->d_out, p->dtype == MLORA_BF16 ? "bf16" : "f32", lora_on, lora_on ? sv.n_seg : 0,
          sv.n_seg_dev ? "(bound)" : "", ks, shrink, p->max_rank);
}

// MLORA_DEBUG_VALIDATE=1: the layer entry points check sorted metadata on the
// device first (as mlora_validate, which synchronizes the stream) and return
// its error instead of running the layer.
bool debug_validate() {
  const char* e = getenv("MLORA_DEBUG_VALIDATE");
  return e && e[0] == '1' && e[1] == 0;
}

// The adapter term as a dense fp32 tile (k_expand_delta, added by the GEMM
// before its rounding) instead of the GEMM epilogue's MFMA expand: plain bf16
// pools of rank <= kDxMaxRank with a dense-term region in the workspace, on
// the tiled GEMM path, for pools whose largest rank is at least 32. The
// choice depends on the pool and T only, never on the segments, so a batch
// and its unsorted form (whose segments only the device knows) take the same
// path and give the same bits. Measured on the heterogeneous batch (256
// tokens, 5120 -> 5120, 112 adapters of ranks 8-64, mostly one token each):
// 82.0 us per LoRA-on call against 88.7 with the MFMA expand, whose busiest
// wave walks 69 (run, 16 rank column) units while others walk 2; on the
// verify batch (rank 16, two tokens per segment) the MFMA expand stays
// ahead, 69.7 against 82.9 us. MLORA_EXPAND=dense|mfma forces either where
// eligible.
bool use_dense_expand(const mlora_pool_s* p, const SegView& sv, int T, int lora_on) {
  if (!lora_on || sv.n_seg <= 0 || p->kind == 2 || p->max_rank > kDxMaxRank || p->d_out % 8 != 0 ||
      delta_bytes(p, T) == 0)
    return false;
  const char* e = getenv("MLORA_EXPAND");
  if (e && !strcmp(e, "dense")) return true;
  if (e && !strcmp(e, "mfma")) return false;
  return p->max_rank >= 32;
}

// Launch the layer on sorted metadata already resident on the device.
// w_scale != null: W holds FP8 e4m3 codes with a float32 scale per row (bf16
// pool, split-K decode path only; the caller has checked the shape).
int run_linear(const void* x, const void* W, mlora_pool_s* pool, const SegView& sv, int T,
               int lora_on, void* y, char* ws, hipStream_t stream, const float* w_scale = nullptr) {
  const WsLayout L = ws_layout(pool, T);
  LinearArgs a;
  a.x = x;
  a.W = W;
  a.y = y;
  a.T = T;
  a.d_in = pool->d_in;
  a.d_out = pool->d_out;
  a.lora_on = lora_on;
  a.sv = sv;
  a.pv = view_of(pool);
  a.v_part = (float*)(ws + L.v_part);
  a.pos_info = (int4*)(ws + L.pos_info);
  a.v_fin = (float*)(ws + L.v_fin);
  a.r_ws = r_ws_of(pool->max_rank);
  a.seg_grid = lora_on ? sv.n_seg : 0;
  a.delta = nullptr;
  a.gorder = 0;
  a.wnt = 0;
  if (pool->dtype == MLORA_BF16) {
    const int fp = forced_path();
    // The split-K decode path up to 64 tokens, except on wide layers from 48
    // tokens up; the tiled GEMM otherwise. Measured per path, token count and
    // pass with HBM counters in profiles/path_sweep.txt: on 4096 -> 4096 the
    // decode pair is the fastest LoRA-on path at every count from 1 to 64
    // (the GEMM takes 2-3x as long there); on 4096 -> 14336 the GEMM is
    // faster in both passes from 48 tokens and the decode pair below. Both
    // passes of a shape and token count take the same path, so a zero B
    // reproduces the LoRA-off bits.
    const bool wide = T >= 48 && pool->d_out >= 8192;
    const bool dec_ok = decode_supported(T, lora_on ? sv.n_seg : 0, pool->d_out, pool->max_rank);
    if (w_scale || (dec_ok && (fp == 1 || (fp == 0 && !wide)))) {
      DecodeArgs d;
      d.x = x;
      d.W = W;
      d.y = y;
      d.T = T;
      d.d_in = pool->d_in;
      d.d_out = pool->d_out;
      d.lora_on = lora_on;
      d.sv = sv;
      d.pv = a.pv;
      d.ypart = (float*)(ws + L.ypart);
      d.v_part = a.v_part;
      d.pos = a.pos_info;
      d.r_ws = a.r_ws;
      decode_plan(pool->d_in, pool->d_out, &d.n_tiles, &d.kc, &d.n_chunks);
      d.unit_rows = decode_unit_rows(lora_on ? sv.n_seg : 0, pool->max_rank, d.n_tiles);
      d.w_scale = w_scale;
      if (log_calls())
        log_call(w_scale ? "decode-fp8w" : "decode", T, pool, sv, lora_on, d.n_chunks, lora_on ? "fused" : "none");
      launch_decode_bf16(d, stream);
      return check_launch();
    }
    // short low-rank segments (a verify batch): one d_in chunk, so the shrink
    // writes the final scaled v and no finalize launch follows (measured
    // faster there; longer or higher-rank segments gain from the split); so
    // does every batch the short-segment shrink takes (it runs one chunk)
    LinearArgs one = a;
    one.ks = 1;
    const bool one_chunk = lora_on && ((T <= 16 * a.seg_grid && pool->max_rank <= 16) || shrink_short(one));
    a.ks = one_chunk ? 1 : choose_shrink_split_bf16(pool->d_in, shrink_items_bound(T, a.seg_grid, pool->max_rank));
    if (fp == 3 && T <= 64) {
      if (log_calls())
        log_call("gemv", T, pool, sv, lora_on, a.ks, !lora_on || a.seg_grid <= 0 ? "none" : shrink_short(a) ? "short" : "mfma");
      launch_shrink_bf16(a, stream);
      launch_gemv_bf16(a, stream);
      return check_launch();
    }
    if (use_dense_expand(pool, sv, T, lora_on)) a.delta = (float*)(ws + L.delta);
    if (log_calls())
      log_call(a.delta ? "gemm-dense-expand" : "gemm", T, pool, sv, lora_on, a.ks,
               !lora_on || a.seg_grid <= 0 ? "none" : shrink_short(a) ? "short" : "mfma");
    launch_linear_bf16(a, stream);
  } else {
    a.ks = 1;
    if (log_calls()) log_call("f32", T, pool, sv, lora_on, a.ks, lora_on ? "f32" : "none");
    launch_linear_f32(a, stream);
  }
  return check_launch();
}

// ---- scratch of the entry point that allocates nothing ----------------------
// mlora_linear_noalloc runs the layer with its workspace in this file-scope
// device array instead of a caller's buffer. Every GPU the library runs on
// holds its own copy, at its own address, until the process ends. In host
// code the array's name is only a stand-in: kernels and copies get the
// device address from hipGetSymbolAddress, taken once per device (with that
// device current) and kept in scratch_dev.
static __device__ __align__(256) unsigned char scratch[MLORA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices] = {};

// Device address of the current device's scratch (taken on the first call on
// that device).
int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MLORA_ERR_HIP;
  if (dev >= kMaxDevices) return MLORA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLORA_ERR_HIP;
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return MLORA_OK;
}

}  // namespace

extern "C" {

const char* mlora_status_string(int status) {
  switch (status) {
    case MLORA_OK: return "ok";
    case MLORA_ERR_INVALID_ARG: return "invalid argument";
    case MLORA_ERR_SHAPE: return "unsupported shape";
    case MLORA_ERR_DTYPE: return "unsupported dtype";
    case MLORA_ERR_RANK: return "bad adapter rank";
    case MLORA_ERR_ADAPTER: return "adapter id out of range or not registered";
    case MLORA_ERR_EXISTS: return "adapter id already registered";
    case MLORA_ERR_WORKSPACE: return "workspace or pool arena too small";
    case MLORA_ERR_METADATA: return "inconsistent segment metadata";
    case MLORA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

size_t mlora_pool_bytes(int d_in, int d_out, int dtype, int max_rank, int capacity) {
  if (!shape_ok(d_in, d_out, dtype, max_rank, capacity)) return 0;
  long long se, bo;
  slot_geometry(d_in, d_out, max_rank, dtype, &se, &bo);
  const size_t slots = align_up((size_t)capacity * (size_t)se * elem_size(dtype), kAlign);
  return slots + align_up((size_t)capacity * 4, kAlign) + kZeroBytes;
}

int mlora_pool_create(void* dev_mem, size_t bytes, int d_in, int d_out, int dtype, int max_rank,
                      int capacity, hipStream_t stream, mlora_pool_t* out) {
  if (!out || !dev_mem || !aligned16(dev_mem)) return MLORA_ERR_INVALID_ARG;
  *out = nullptr;
  if (elem_size(dtype) == 0) return MLORA_ERR_DTYPE;
  if (!shape_ok(d_in, d_out, dtype, max_rank, capacity)) return MLORA_ERR_SHAPE;
  const size_t need = mlora_pool_bytes(d_in, d_out, dtype, max_rank, capacity);
  if (bytes < need) return MLORA_ERR_WORKSPACE;
  mlora_pool_s* p = new (std::nothrow) mlora_pool_s();
  if (!p) return MLORA_ERR_INVALID_ARG;
  p->base = dev_mem;
  p->bytes = bytes;
  p->d_in = d_in;
  p->d_out = d_out;
  p->dtype = dtype;
  p->max_rank = max_rank;
  p->capacity = capacity;
  p->elem = elem_size(dtype);
  slot_geometry(d_in, d_out, max_rank, dtype, &p->slot_elems, &p->b_offset);
  const size_t slots = align_up((size_t)capacity * (size_t)p->slot_elems * p->elem, kAlign);
  p->dev_rank = (int32_t*)((char*)dev_mem + slots);
  p->zeros = (char*)dev_mem + slots + align_up((size_t)capacity * 4, kAlign);
  p->host_rank.assign(capacity, 0);
  launch_fill_u32(p->dev_rank, (size_t)capacity, 0u, stream);
  launch_fill_u32(p->zeros, kZeroBytes / 4, 0u, stream);
  const int st = check_launch();
  if (st != MLORA_OK) {
    delete p;
    return st;
  }
  *out = p;
  return MLORA_OK;
}

int mlora_pool_destroy(mlora_pool_t pool) {
  delete pool;
  return MLORA_OK;
}

// B columns of a slot's region, zero-filled first: bf16 pools hold
// ceil(rank / 16) blocks of [d_out][16] (bblk_off), fp32 pools d_out rows of
// round_up8(rank) columns.
size_t b_region_elems(const mlora_pool_s* p, int rank) {
  return (size_t)p->d_out * (p->dtype == MLORA_BF16 ? (rank + 15) & ~15 : (rank + 7) & ~7);
}

// Copy a row-major [rows, r] block of B (source row pitch r) to rows
// [n_off, n_off + rows) and rank columns [r_off, r_off + r) of the slot's B
// region (bdst): one 2D copy per block of 16 columns it meets in a bf16
// pool, one 2D copy of padded rows (pitch bld = round_up8 of the adapter's
// rank) in an fp32 pool.
int copy_b(const mlora_pool_s* p, char* bdst, int bld, const void* B, int rows, int n_off, int r_off, int r,
           hipStream_t stream) {
  const size_t el = p->elem;
  if (p->dtype != MLORA_BF16) {
    const hipError_t e = hipMemcpy2DAsync(bdst + ((size_t)n_off * bld + r_off) * el, (size_t)bld * el, B,
                                          (size_t)r * el, (size_t)r * el, (size_t)rows, hipMemcpyDefault, stream);
    return e == hipSuccess ? MLORA_OK : MLORA_ERR_HIP;
  }
  for (int c0 = r_off; c0 < r_off + r;) {
    const int blk = c0 / 16;
    const int c1 = std::min(r_off + r, 16 * blk + 16);
    char* dst = bdst + (((size_t)blk * p->d_out + n_off) * 16 + (c0 - 16 * blk)) * el;
    const char* src = (const char*)B + (size_t)(c0 - r_off) * el;
    const hipError_t e = hipMemcpy2DAsync(dst, 16 * el, src, (size_t)r * el, (size_t)(c1 - c0) * el, (size_t)rows,
                                          hipMemcpyDefault, stream);
    if (e != hipSuccess) return MLORA_ERR_HIP;
    c0 = c1;
  }
  return MLORA_OK;
}

int mlora_register_adapter(mlora_pool_t p, int adapter_id, int rank, const void* A, const void* B,
                           hipStream_t stream) {
  if (!p || !A || !B) return MLORA_ERR_INVALID_ARG;
  if (adapter_id < 0 || adapter_id >= p->capacity) return MLORA_ERR_ADAPTER;
  if (rank < 1 || rank > p->max_rank) return MLORA_ERR_RANK;
  if (p->host_rank[adapter_id] != 0) return MLORA_ERR_EXISTS;
  if (p->kind == 2) return MLORA_ERR_SHAPE;   // a pool of fused adapters takes fused ones only
  char* slot = (char*)p->base + (size_t)adapter_id * (size_t)p->slot_elems * p->elem;
  // A: [rank, d_in] contiguous
  hipError_t e = hipMemcpyAsync(slot, A, (size_t)rank * p->d_in * p->elem, hipMemcpyDefault, stream);
  if (e != hipSuccess) return MLORA_ERR_HIP;
  // B: [d_out, rank] -> the slot's layout, zero past the rank
  char* bdst = slot + (size_t)p->b_offset * p->elem;
  const int bld = (rank + 7) & ~7;
  if (b_region_elems(p, rank) != (size_t)p->d_out * rank) {
    launch_fill_u32(bdst, b_region_elems(p, rank) * p->elem / 4, 0u, stream);
    if (check_launch() != MLORA_OK) return MLORA_ERR_HIP;
  }
  if (copy_b(p, bdst, bld, B, p->d_out, 0, 0, rank, stream) != MLORA_OK) return MLORA_ERR_HIP;
  launch_set_slot_rank(p->dev_rank, adapter_id, rank, stream);
  if (check_launch() != MLORA_OK) return MLORA_ERR_HIP;
  p->host_rank[adapter_id] = rank;
  p->kind = 1;
  return MLORA_OK;
}

int mlora_register_adapter_fused(mlora_pool_t p, int adapter_id, int n_slices, const int* slice_rows,
                                 const int* slice_ranks, const void* const* A, const void* const* B,
                                 hipStream_t stream) {
  if (!p || !slice_rows || !slice_ranks || !A || !B) return MLORA_ERR_INVALID_ARG;
  if (n_slices < 1 || n_slices > MLORA_MAX_SLICES) return MLORA_ERR_SHAPE;
  if (adapter_id < 0 || adapter_id >= p->capacity) return MLORA_ERR_ADAPTER;
  if (p->host_rank[adapter_id] != 0) return MLORA_ERR_EXISTS;
  long long rows = 0;
  int rank = 0;
  for (int m = 0; m < n_slices; ++m) {
    if (!A[m] || !B[m]) return MLORA_ERR_INVALID_ARG;
    if (slice_rows[m] < 1) return MLORA_ERR_SHAPE;
    if (slice_ranks[m] < 1 || slice_ranks[m] > p->max_rank) return MLORA_ERR_RANK;
    rows += slice_rows[m];
    rank += slice_ranks[m];
    if (rank > p->max_rank) return MLORA_ERR_RANK;
  }
  if (rows != p->d_out) return MLORA_ERR_SHAPE;
  if (p->kind == 1) return MLORA_ERR_SHAPE;   // a pool of plain adapters takes plain ones only
  if (p->kind == 2) {                          // the pool's W stacks the same projections
    if (n_slices != p->n_slices) return MLORA_ERR_SHAPE;
    for (int m = 0, end = 0; m < n_slices; ++m) {
      end += slice_rows[m];
      if (end != p->slice_end[m]) return MLORA_ERR_SHAPE;
    }
  }
  char* slot = (char*)p->base + (size_t)adapter_id * (size_t)p->slot_elems * p->elem;
  char* bdst = slot + (size_t)p->b_offset * p->elem;
  const int bld = (rank + 7) & ~7;
  // B is block-diagonal: zero everywhere, then each slice's block
  launch_fill_u32(bdst, b_region_elems(p, rank) * p->elem / 4, 0u, stream);
  if (check_launch() != MLORA_OK) return MLORA_ERR_HIP;
  int r_off = 0, n_off = 0;
  for (int m = 0; m < n_slices; ++m) {
    const int r = slice_ranks[m];
    hipError_t e = hipMemcpyAsync(slot + (size_t)r_off * p->d_in * p->elem, A[m],
                                  (size_t)r * p->d_in * p->elem, hipMemcpyDefault, stream);
    if (e != hipSuccess) return MLORA_ERR_HIP;
    if (copy_b(p, bdst, bld, B[m], slice_rows[m], n_off, r_off, r, stream) != MLORA_OK) return MLORA_ERR_HIP;
    r_off += r;
    n_off += slice_rows[m];
  }
  launch_set_slot_rank(p->dev_rank, adapter_id, rank, stream);
  if (check_launch() != MLORA_OK) return MLORA_ERR_HIP;
  p->host_rank[adapter_id] = rank;
  if (p->kind != 2) {
    p->kind = 2;
    p->n_slices = n_slices;
    for (int m = 0, end = 0; m < n_slices; ++m) p->slice_end[m] = (end += slice_rows[m]);
  }
  for (int m = 1; m < n_slices; ++m)
    if (slice_ranks[m] != slice_ranks[0]) p->slice_uniform = false;
  return MLORA_OK;
}

int mlora_unregister_adapter(mlora_pool_t p, int adapter_id, hipStream_t stream) {
  if (!p) return MLORA_ERR_INVALID_ARG;
  if (adapter_id < 0 || adapter_id >= p->capacity) return MLORA_ERR_ADAPTER;
  if (p->host_rank[adapter_id] == 0) return MLORA_ERR_ADAPTER;
  launch_set_slot_rank(p->dev_rank, adapter_id, 0, stream);
  if (check_launch() != MLORA_OK) return MLORA_ERR_HIP;
  p->host_rank[adapter_id] = 0;
  return MLORA_OK;
}

int mlora_adapter_rank(mlora_pool_t p, int adapter_id) {
  if (!p || adapter_id < 0 || adapter_id >= p->capacity) return -1;
  return p->host_rank[adapter_id];
}

size_t mlora_workspace_bytes(mlora_pool_t p, int max_tokens) {
  if (!p || max_tokens < 0 || max_tokens > MLORA_MAX_TOKENS) return 0;
  // the layout grows with T, except where a region stops: the decode partial
  // tiles past 64 tokens and the dense adapter term past delta_tokens_max; a
  // smaller batch may then need more than a larger one, so the size is the
  // largest of the three candidates
  const size_t big = ws_layout(p, max_tokens).total;
  const size_t small = ws_layout(p, max_tokens < 64 ? max_tokens : 64).total;
  const size_t mid = ws_layout(p, delta_tokens_max(p, max_tokens)).total;
  const size_t m = big > small ? big : small;
  return m > mid ? m : mid;
}

int mlora_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!workspace || !aligned16(workspace)) return MLORA_ERR_INVALID_ARG;
  launch_fill_u32(workspace, workspace_bytes / 4, 0u, stream);
  return check_launch();
}

int mlora_linear(const void* x, const void* W, mlora_pool_t pool, const int32_t* seg_start,
                 const int32_t* seg_adapter, const int32_t* seg_rank, const float* seg_scale,
                 const int32_t* token_index, int n_tokens, int n_seg, int lora_on, void* y,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!pool) return MLORA_ERR_INVALID_ARG;
  if (lora_on != 0 && lora_on != 1) return MLORA_ERR_INVALID_ARG;
  if (n_tokens < 0 || n_tokens > MLORA_MAX_TOKENS) return MLORA_ERR_SHAPE;
  if (n_tokens == 0) return MLORA_OK;
  if (!x || !W || !y || !workspace) return MLORA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(W) || !aligned16(y) || !aligned16(workspace))
    return MLORA_ERR_INVALID_ARG;
  if (workspace_bytes < ws_layout(pool, n_tokens).total) return MLORA_ERR_WORKSPACE;
  SegView sv{};
  if (lora_on) {
    if (!seg_start || !seg_adapter || !seg_rank || !seg_scale) return MLORA_ERR_INVALID_ARG;
    if (n_seg < 1) return MLORA_ERR_METADATA;
    if (n_seg > MLORA_MAX_SEGMENTS) return MLORA_ERR_SHAPE;
    sv.seg_start = seg_start;
    sv.seg_adapter = seg_adapter;
    sv.seg_rank = seg_rank;
    sv.seg_scale = seg_scale;
    sv.token_index = token_index;
    sv.n_seg_dev = nullptr;
    sv.n_seg = n_seg;
    if (debug_validate()) {
      const int st = mlora_validate(pool, seg_start, seg_adapter, seg_rank, token_index, n_tokens, n_seg,
                                    workspace, workspace_bytes, stream);
      if (st != MLORA_OK) return st;
    }
  }
  return run_linear(x, W, pool, sv, n_tokens, lora_on, y, (char*)workspace, stream);
}

int mlora_linear_noalloc(const void* x, const void* W, mlora_pool_t pool, const int32_t* seg_start,
                         const int32_t* seg_adapter, const int32_t* seg_rank, const float* seg_scale,
                         const int32_t* token_index, int n_tokens, int n_seg, int lora_on, void* y,
                         hipStream_t stream) {
  if (!pool) return MLORA_ERR_INVALID_ARG;
  if (n_tokens < 0 || n_tokens > MLORA_MAX_TOKENS) return MLORA_ERR_SHAPE;
  if (n_tokens == 0) return MLORA_OK;
  // the whole workspace of the call must fit the scratch: larger calls are
  // refused before anything runs
  if (ws_layout(pool, n_tokens).total > (size_t)MLORA_NOALLOC_SCRATCH_BYTES) return MLORA_ERR_WORKSPACE;
  void* ws = nullptr;
  const int st = scratch_ptr(&ws);
  if (st != MLORA_OK) return st;
  return mlora_linear(x, W, pool, seg_start, seg_adapter, seg_rank, seg_scale, token_index, n_tokens,
                      n_seg, lora_on, y, ws, (size_t)MLORA_NOALLOC_SCRATCH_BYTES, stream);
}

int mlora_linear_fp8w(const void* x, const uint8_t* W_fp8, const float* w_scale, mlora_pool_t pool,
                      const int32_t* seg_start, const int32_t* seg_adapter, const int32_t* seg_rank,
                      const float* seg_scale, const int32_t* token_index, int n_tokens, int n_seg,
                      int lora_on, void* y, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  if (!pool) return MLORA_ERR_INVALID_ARG;
  if (pool->dtype != MLORA_BF16) return MLORA_ERR_DTYPE;
  if (lora_on != 0 && lora_on != 1) return MLORA_ERR_INVALID_ARG;
  if (n_tokens < 0 || n_tokens > MLORA_MAX_FP8W_TOKENS) return MLORA_ERR_SHAPE;
  if (pool->d_in % 16 != 0) return MLORA_ERR_SHAPE;
  if (n_tokens == 0) return MLORA_OK;
  if (!x || !W_fp8 || !w_scale || !y || !workspace) return MLORA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(W_fp8) || !aligned16(y) || !aligned16(workspace))
    return MLORA_ERR_INVALID_ARG;
  if (workspace_bytes < ws_layout(pool, n_tokens).total) return MLORA_ERR_WORKSPACE;
  SegView sv{};
  if (lora_on) {
    if (!seg_start || !seg_adapter || !seg_rank || !seg_scale) return MLORA_ERR_INVALID_ARG;
    if (n_seg < 1) return MLORA_ERR_METADATA;
    if (n_seg > MLORA_MAX_SEGMENTS) return MLORA_ERR_SHAPE;
    sv.seg_start = seg_start;
    sv.seg_adapter = seg_adapter;
    sv.seg_rank = seg_rank;
    sv.seg_scale = seg_scale;
    sv.token_index = token_index;
    sv.n_seg_dev = nullptr;
    sv.n_seg = n_seg;
  }
  if (!decode_supported(n_tokens, lora_on ? n_seg : 0, pool->d_out, pool->max_rank))
    return MLORA_ERR_SHAPE;
  if (lora_on && debug_validate()) {
    const int st = mlora_validate(pool, seg_start, seg_adapter, seg_rank, token_index, n_tokens, n_seg,
                                  workspace, workspace_bytes, stream);
    if (st != MLORA_OK) return st;
  }
  return run_linear(x, W_fp8, pool, sv, n_tokens, lora_on, y, (char*)workspace, stream, w_scale);
}

int mlora_build_segments(const int32_t* token_adapter, const float* adapter_scale, int n_tokens,
                         mlora_pool_t pool, int32_t* token_index, int32_t* seg_start,
                         int32_t* seg_adapter, int32_t* seg_rank, float* seg_scale,
                         int32_t* n_seg_out, hipStream_t stream) {
  if (!pool || !seg_start || !n_seg_out) return MLORA_ERR_INVALID_ARG;
  if (n_tokens < 0 || n_tokens > MLORA_MAX_UNSORTED_TOKENS) return MLORA_ERR_SHAPE;
  if (n_tokens > 0 && (!token_adapter || !adapter_scale || !token_index || !seg_adapter ||
                       !seg_rank || !seg_scale))
    return MLORA_ERR_INVALID_ARG;
  launch_build_segments(token_adapter, adapter_scale, n_tokens, view_of(pool), token_index,
                        seg_start, seg_adapter, seg_rank, seg_scale, n_seg_out, stream);
  return check_launch();
}

int mlora_linear_tokens(const void* x, const void* W, mlora_pool_t pool,
                        const int32_t* token_adapter, const float* adapter_scale, int n_tokens,
                        int lora_on, void* y, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  if (!pool) return MLORA_ERR_INVALID_ARG;
  if (lora_on != 0 && lora_on != 1) return MLORA_ERR_INVALID_ARG;
  if (n_tokens < 0 || n_tokens > MLORA_MAX_UNSORTED_TOKENS) return MLORA_ERR_SHAPE;
  if (n_tokens == 0) return MLORA_OK;
  if (!x || !W || !y || !workspace) return MLORA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(W) || !aligned16(y) || !aligned16(workspace))
    return MLORA_ERR_INVALID_ARG;
  const WsLayout L = ws_layout(pool, n_tokens);
  if (workspace_bytes < L.total) return MLORA_ERR_WORKSPACE;
  SegView sv{};
  if (lora_on) {
    if (!token_adapter || !adapter_scale) return MLORA_ERR_INVALID_ARG;
    char* ws = (char*)workspace;
    int32_t* ti = (int32_t*)(ws + L.token_index);
    int32_t* ss = (int32_t*)(ws + L.seg_start);
    int32_t* sa = (int32_t*)(ws + L.seg_adapter);
    int32_t* sr = (int32_t*)(ws + L.seg_rank);
    float* sc = (float*)(ws + L.seg_scale);
    int32_t* ns = (int32_t*)(ws + L.n_seg);
    launch_build_segments(token_adapter, adapter_scale, n_tokens, view_of(pool), ti, ss, sa, sr,
                          sc, ns, stream);
    const int st = check_launch();
    if (st != MLORA_OK) return st;
    sv.seg_start = ss;
    sv.seg_adapter = sa;
    sv.seg_rank = sr;
    sv.seg_scale = sc;
    sv.token_index = ti;
    sv.n_seg_dev = ns;
    sv.n_seg = n_tokens;  // upper bound on the device count
  }
  return run_linear(x, W, pool, sv, n_tokens, lora_on, y, (char*)workspace, stream);
}

int mlora_token_map(const int32_t* seg_start, const int32_t* seg_adapter, int n_tokens, int n_seg,
                    int32_t* token_seg, int32_t* token_adapter_out, hipStream_t stream) {
  if (n_tokens < 0 || n_seg < 0) return MLORA_ERR_SHAPE;
  if (n_tokens == 0) return MLORA_OK;
  if (!seg_start || (n_seg > 0 && !seg_adapter) || !token_seg || !token_adapter_out)
    return MLORA_ERR_INVALID_ARG;
  launch_token_map(seg_start, seg_adapter, n_tokens, n_seg, token_seg, token_adapter_out, stream);
  return check_launch();
}

int mlora_merge_adapter(const void* W_in, void* W_out, mlora_pool_t pool, int adapter_id,
                        float scale, hipStream_t stream) {
  if (!pool || !W_in || !W_out) return MLORA_ERR_INVALID_ARG;
  if (!aligned16(W_in) || !aligned16(W_out)) return MLORA_ERR_INVALID_ARG;
  const size_t wbytes = (size_t)pool->d_out * pool->d_in * pool->elem;
  const uintptr_t wi = (uintptr_t)W_in, wo = (uintptr_t)W_out;
  if (wi != wo && wi < wo + wbytes && wo < wi + wbytes) return MLORA_ERR_INVALID_ARG;  // partial overlap
  if (adapter_id < 0 || adapter_id >= pool->capacity) return MLORA_ERR_ADAPTER;
  const int rank = pool->host_rank[adapter_id];
  if (rank <= 0) return MLORA_ERR_ADAPTER;
  const char* slot = (const char*)pool->base + (size_t)adapter_id * (size_t)pool->slot_elems * pool->elem;
  MergeArgs a;
  a.W_in = W_in;
  a.W_out = W_out;
  a.A = slot;
  a.B = slot + (size_t)pool->b_offset * pool->elem;
  a.d_in = pool->d_in;
  a.d_out = pool->d_out;
  a.rank = rank;
  a.pitch = (rank + 7) & ~7;
  a.scale = scale;
  launch_merge(a, pool->dtype == MLORA_BF16, stream);
  return check_launch();
}

int mlora_validate(mlora_pool_t pool, const int32_t* seg_start, const int32_t* seg_adapter,
                   const int32_t* seg_rank, const int32_t* token_index, int n_tokens, int n_seg,
                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!pool || !seg_start || !workspace) return MLORA_ERR_INVALID_ARG;
  if (n_tokens < 0 || n_seg < 0 || n_tokens > MLORA_MAX_TOKENS) return MLORA_ERR_SHAPE;
  if (n_seg > 0 && !seg_adapter) return MLORA_ERR_INVALID_ARG;
  const WsLayout L = ws_layout(pool, n_tokens);
  if (workspace_bytes < L.total) return MLORA_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  int32_t* result = (int32_t*)(ws + L.err);
  launch_validate(seg_start, seg_adapter, seg_rank, token_index, n_tokens, n_seg, view_of(pool),
                  (int32_t*)(ws + L.counts), result, stream);
  int st = check_launch();
  if (st != MLORA_OK) return st;
  int32_t host = -1;
  if (hipMemcpyAsync(&host, result, sizeof(host), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return MLORA_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return MLORA_ERR_HIP;
  return host;
}

}  // extern "C"
