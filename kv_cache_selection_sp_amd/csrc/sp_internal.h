// Internal declarations shared by the HIP translation units of libspdecode.
// Not part of the public ABI (include/spdecode.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "spdecode.h"

namespace spk {

// Device-side view of the descriptor.
struct KVDev {
  int B, Hq, Hkv, G, D, P, max_pages, num_blocks;
  void* k_pool;
  void* v_pool;
  const int32_t* block_table;
  int32_t* seq_lens;
};

inline KVDev to_dev(const sp_paged_kv* kv) {
  KVDev d;
  d.B = kv->batch; d.Hq = kv->num_q_heads; d.Hkv = kv->num_kv_heads;
  d.G = kv->num_q_heads / kv->num_kv_heads; d.D = kv->head_dim; d.P = kv->page_size;
  d.max_pages = kv->max_pages_per_seq; d.num_blocks = kv->num_blocks;
  d.k_pool = kv->k_pool; d.v_pool = kv->v_pool;
  d.block_table = kv->block_table; d.seq_lens = kv->seq_lens;
  return d;
}

// ---------------------------------------------------------------- element types
// bf16 is carried as raw uint16_t bits; arithmetic is always fp32.
typedef uint16_t bf16_t;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float(((uint32_t)x) << 16); }

// Round-to-nearest-even fp32 -> bf16 (inputs here are finite).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}
template <typename T> __device__ __forceinline__ T from_f32(float f);
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float f) { return f32_to_bf16(f); }

// ---------------------------------------------------------------- layouts
// A (block, head) page holds P tokens x D dims of K and of V, contiguous.
//   K: chunk-tiled [D/E][P][E] with E = 16 / sizeof(T) elements per 16 bytes.
//   V: dim-major  [D][P].
template <typename T> struct Chunk { static constexpr int E = 16 / (int)sizeof(T); };

__device__ __forceinline__ size_t page_base(int blk, int h, int Hkv, int P, int D) {
  return ((size_t)blk * Hkv + h) * (size_t)P * D;
}
template <typename T>
__device__ __forceinline__ int k_off(int t, int d, int P) {
  constexpr int E = Chunk<T>::E;
  return ((d / E) * P + t) * E + (d % E);
}
__device__ __forceinline__ int v_off(int t, int d, int P) { return d * P + t; }

// Clamp a device length into [0, cap].
__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

// Order-preserving map fp32 -> uint32 (larger float -> larger key); -0 is
// folded onto +0 and NaN onto the smallest key.
__device__ __forceinline__ uint32_t float_key(float f) {
  if (f != f) return 0u;
  if (f == 0.0f) f = 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- block scan
// Exclusive prefix sum of one int per thread over a block of NT threads
// (NT a multiple of 64, <= 1024).  `wsum` is __shared__ int[NT/64 + 1].
// Returns the exclusive prefix; *total receives the block total.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wid] = x;
  __syncthreads();
  // every thread sums the (at most 16) wave totals itself: no serial step
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int t = wsum[w];
    before += w < wid ? t : 0;
    tot += t;
  }
  *total = tot;
  __syncthreads();   // wsum is rewritten by the next scan
  return before + x - v;
}

// The same scan without the closing barrier: the caller guarantees a barrier
// between this scan's reads of `wsum` and the next write to it (or uses
// another buffer for the next scan).
template <int NT>
__device__ __forceinline__ int block_exclusive_scan_open(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wid] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int t = wsum[w];
    before += w < wid ? t : 0;
    tot += t;
  }
  *total = tot;
  return before + x - v;
}

// ---------------------------------------------------------------- cross-lane
// Partners within a 16-lane row come from DPP moves (quad permutations,
// half-row and row mirrors, row shifts and broadcasts), which issue on the
// vector ALU instead of going through LDS.
template <int CTRL>
__device__ __forceinline__ float dpp_partner(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppSwap1 = 0xB1;        // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppSwap2 = 0x4E;        // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i within each 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i within each 16 lanes
constexpr int kSwizzleXor16 = 0x401f;  // bitmask swizzle: lane ^ 16 within 32


// Minimum and maximum of a uint32 over the wavefront (in every lane).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_partner_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ void wave_min_max(uint32_t& lo, uint32_t& hi) {
#define SPK_MM_STEP(PARTNER)                 \
  { const uint32_t a = PARTNER(lo), b = PARTNER(hi); lo = min(lo, a); hi = max(hi, b); }
  SPK_MM_STEP(dpp_partner_u<kDppSwap1>)
  SPK_MM_STEP(dpp_partner_u<kDppSwap2>)
  SPK_MM_STEP(dpp_partner_u<kDppHalfMirror>)
  SPK_MM_STEP(dpp_partner_u<kDppMirror>)
#undef SPK_MM_STEP
  // the four rows' values, read into scalar registers
  const uint32_t l0 = __builtin_amdgcn_readlane((int)lo, 0), l1 = __builtin_amdgcn_readlane((int)lo, 16);
  const uint32_t l2 = __builtin_amdgcn_readlane((int)lo, 32), l3 = __builtin_amdgcn_readlane((int)lo, 48);
  const uint32_t h0 = __builtin_amdgcn_readlane((int)hi, 0), h1 = __builtin_amdgcn_readlane((int)hi, 16);
  const uint32_t h2 = __builtin_amdgcn_readlane((int)hi, 32), h3 = __builtin_amdgcn_readlane((int)hi, 48);
  lo = min(min(l0, l1), min(l2, l3));
  hi = max(max(h0, h1), max(h2, h3));
}

// Inclusive prefix sum over the wavefront with DPP moves: row shifts by 1,
// 2, 4, 8 within each 16-lane row, then the row totals carried across rows
// with row broadcasts.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_src(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xf, false);
}
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += dpp_src<0x111, 0xf>(v);   // row_shr:1
  v += dpp_src<0x112, 0xf>(v);   // row_shr:2
  v += dpp_src<0x114, 0xf>(v);   // row_shr:4
  v += dpp_src<0x118, 0xf>(v);   // row_shr:8
  v += dpp_src<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
  v += dpp_src<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}

// Exclusive prefix sum of one int per thread over the workgroup: DPP wave
// scans, wave totals through LDS (one barrier).  The caller keeps a barrier
// between this scan's reads of `wsum` and the next write to it.
template <int NT>
__device__ __forceinline__ int block_scan_dpp(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int incl = wave_inclusive_scan(v);
  if (lane == 63) wsum[wid] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int t = wsum[w];
    before += w < wid ? t : 0;
    tot += t;
  }
  *total = tot;
  return before + incl - v;
}


// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  Arguments are validated by the
// API layer before these are called.
hipError_t launch_append(const KVDev& kv, int dtype, const void* k_new, const void* v_new,
                         int n_new, void* page_meta, const int32_t* pos_new, int32_t* slot_pos,
                         int slot_cap, hipStream_t s);
hipError_t launch_rebuild_meta(const KVDev& kv, int dtype, void* page_meta, hipStream_t s);

size_t select_workspace_bytes(const KVDev& kv);
size_t select_scores_bytes(const KVDev& kv);
// Workspace of the list top-k (page counts, then per-unit lists) used above
// the register top-k's page count; 0 at or below it.
size_t select_list_bytes(const KVDev& kv);
size_t list_counts_bytes(const KVDev& kv);
size_t page_topk_list_bytes(const KVDev& kv);
// Top-k over the page score rows [B][Hkv][max_pages] by the list path's
// threshold search: n_pages[b] pages per sequence, the first n_sink and the
// last n_recent always kept, rows of sel [B][Hkv][top_k] in ascending order
// padded with -1.  ws: page_topk_list_bytes(kv) bytes.
hipError_t launch_page_topk_list(const KVDev& kv, const float* scores, int32_t* n_pages, int top_k, int n_sink,
                                 int n_recent, int32_t* sel, void* ws, hipStream_t s);
// Selection options: pages always chosen, and the group aggregation of the
// page bound (false: sum over the group's query heads; true: the largest).
// One decode token per sequence appended inside the selection launch (the
// append of launch_append with n_new = 1, fused); k_new == nullptr: none.
struct AppendIn {
  const void* k_new = nullptr;     // [B][H_kv][D]
  const void* v_new = nullptr;     // [B][H_kv][D]
  const int32_t* pos_new = nullptr;
  int32_t* slot_pos = nullptr;
  int slot_cap = 0;
};
struct SelectOpts {
  int n_sink = 0;
  int n_recent = 0;
  bool group_max = false;
  AppendIn ap;
};
hipError_t launch_select(const KVDev& kv, int dtype, const void* q, const void* page_meta,
                         int top_k, const SelectOpts& o, int32_t* sel, float* page_scores, void* ws,
                         hipStream_t s);
// The same with the counters (per unit, then per sequence; zero between
// calls), the page scores and the list top-k's workspace (select_list_bytes;
// may be null when that is 0) at separate addresses.
hipError_t launch_select_split(const KVDev& kv, int dtype, const void* q, const void* page_meta, int top_k,
                               const SelectOpts& o, int32_t* sel, float* scores, int* counters, void* list_ws,
                               hipStream_t s);

struct AttnPlan {
  bool mfma;             // bf16 MFMA engine (else VALU engine)
  int n_wg;              // workgroups: the flattened tile range is cut into n_wg chunks
  int threads;           // workgroup size (256 or 512)
  long tiles_max;        // upper bound of the tiles one call streams
  size_t counter_bytes;  // per-unit arrival counters at the head of the workspace
  size_t ws_bytes;       // counters + split records (+ the dense tile prefix, global_prefix)
  bool global_prefix;    // dense with more sequences than LDS holds: prefix in the workspace
  size_t lds_bytes;      // dynamic LDS per workgroup
};
AttnPlan plan_attention(const KVDev& kv, int dtype, bool sparse, int top_k);
hipError_t launch_attention(const KVDev& kv, int dtype, const AttnPlan& plan, const void* q,
                            const int32_t* sel, const uint32_t* sel_mask, int top_k, float scale,
                            float* out, float* lse, float* logits, int logit_cap, void* ws,
                            hipStream_t s,
                            float* acc_scores = nullptr, int slot_cap = 0, int n_new = 0);
// The same with the arrival counters (zero between calls) and the split
// records at separate addresses.
hipError_t launch_attention_split(const KVDev& kv, int dtype, const AttnPlan& plan, const void* q,
                                  const int32_t* sel, const uint32_t* sel_mask, int top_k, float scale,
                                  float* out, float* lse, float* logits, int logit_cap, int* counters,
                                  float* records, hipStream_t s, float* acc_scores = nullptr,
                                  int slot_cap = 0, int n_new = 0);

// One Quest decode step in one launch (append + select + attend) when every
// workgroup of it can be resident at once (*fused = true), else the select
// and attention launches on the same workspace (*fused = false).
size_t quest_step_workspace_bytes(const KVDev& kv, int dtype, int top_k);
size_t quest_step_error_offset(const KVDev& kv);
hipError_t launch_quest_step(const KVDev& kv, int dtype, const void* q, const void* page_meta, int top_k,
                             const SelectOpts& o, int32_t* sel, float* page_scores, float scale, float* out,
                             float* lse, void* ws, hipStream_t s, bool* fused);
// Whether launch_quest_step would take the single launch (launches nothing).
hipError_t quest_step_single_launch(const KVDev& kv, int dtype, bool group_max, bool* single);

// SnapKV window scoring: two sweeps over the prompt keys, a merge of the
// per-chunk softmax states and a pooling pass (all sizes from the descriptor
// and the window length).
struct SnapPlan {
  int n_slab;              // row slabs of 256 rows per pass (R = G * n_obs rows in all)
  int n_pass;              // passes over the rows (1 for SnapKV windows)
  int nrg;                 // row groups (64 rows each) per workgroup: 1, 2 or 4
  int chunk1, n_chunk1;    // keys per workgroup and chunks per unit, normaliser sweep
  int chunk2, n_chunk2;    // the same for the score sweep
  size_t ml_off, lse_off, up_off, ws_bytes;
};
SnapPlan plan_snapkv(const KVDev& kv, int n_obs);
hipError_t launch_snapkv(const KVDev& kv, const SnapPlan& p, const void* q_obs, int n_obs,
                         float scale, int pool_kernel, int n_sink, float* scores, int slot_cap,
                         void* ws, hipStream_t s);
int snapkv_max_pool_kernel();
// Top-`budget` slots of one score row per sequence (ties: lower slot), as page
// entries with token masks replicated for every KV head; the workspace is the
// large eviction path's list layout with one unit per sequence.
hipError_t launch_token_topk_pages(const KVDev& kv, const float* scores, int slot_cap, int budget, void* ws,
                                   int32_t* sel_pages, uint32_t* sel_mask, int k_pages, hipStream_t s);
size_t token_topk_workspace_bytes(const KVDev& kv, int budget);
// OmniKV observation-layer selection: token scores (max logit over the query
// heads), then launch_token_topk_pages.
hipError_t launch_omnikv_select(const KVDev& kv, const void* q, int top_b, int32_t* sel_pages,
                                uint32_t* sel_mask, int k_pages, float* token_scores, int slot_cap, void* ws,
                                hipStream_t s);
int omnikv_max_q_heads();
int omnikv_max_group();

// H2O prefill chunk: probability column sums of the last n_q slots' queries
// (causal) added into the scores of every slot, the chunk's slots reset first.
hipError_t launch_h2o_prefill_scores(const KVDev& kv, const SnapPlan& p, const void* q_chunk, int n_q,
                                     float scale, float* scores, int slot_cap, void* ws, hipStream_t s);

hipError_t launch_h2o_accumulate(const KVDev& kv, const float* logits, const float* lse,
                                 int logit_cap, int n_new, float* scores, int slot_cap,
                                 hipStream_t s);
hipError_t launch_h2o_evict(const KVDev& kv, int dtype, float* scores, int32_t* slot_pos,
                            int slot_cap, int budget, int window, void* ws, hipStream_t s);
// Workspace of sp_h2o_evict_compact: 0 up to the fast path's capacity, else a
// per-unit header and list of `budget` kept slots (budget < 1: the capacity).
// true above the fast path's capacity (the workspace is then required)
bool h2o_evict_list_path(const KVDev& kv);
size_t h2o_evict_workspace_bytes(const KVDev& kv, int budget, int esize);

}  // namespace spk
