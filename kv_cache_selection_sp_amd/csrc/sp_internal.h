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

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  Arguments are validated by the
// API layer before these are called.
hipError_t launch_append(const KVDev& kv, int dtype, const void* k_new, const void* v_new,
                         int n_new, void* page_meta, const int32_t* pos_new, int32_t* slot_pos,
                         int slot_cap, hipStream_t s);
hipError_t launch_rebuild_meta(const KVDev& kv, int dtype, void* page_meta, hipStream_t s);

size_t select_workspace_bytes(const KVDev& kv);
hipError_t launch_select(const KVDev& kv, int dtype, const void* q, const void* page_meta,
                         int top_k, int32_t* sel, float* page_scores, void* ws, hipStream_t s);

struct AttnPlan {
  bool mfma;             // bf16 MFMA engine (else VALU engine)
  int n_wg;              // workgroups: the flattened tile range is cut into n_wg chunks
  int threads;           // workgroup size (256 or 512)
  long tiles_max;        // upper bound of the tiles one call streams
  size_t counter_bytes;  // per-unit arrival counters at the head of the workspace
  size_t ws_bytes;       // counters + split records
  size_t lds_bytes;      // dynamic LDS per workgroup
};
AttnPlan plan_attention(const KVDev& kv, int dtype, bool sparse, int top_k);
hipError_t launch_attention(const KVDev& kv, int dtype, const AttnPlan& plan, const void* q,
                            const int32_t* sel, int top_k, float scale, float* out, float* lse,
                            float* logits, int logit_cap, void* ws, hipStream_t s);

hipError_t launch_h2o_accumulate(const KVDev& kv, const float* logits, const float* lse,
                                 int logit_cap, int n_new, float* scores, int slot_cap,
                                 hipStream_t s);
hipError_t launch_h2o_evict(const KVDev& kv, int dtype, float* scores, int32_t* slot_pos,
                            int slot_cap, int budget, int window, hipStream_t s);

}  // namespace spk
