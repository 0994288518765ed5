// OmniKV token selection at an observation layer.
//
// "SparseEngine: Sparse-First Inference Engine", Appendix A.3, "OmniKV": an
// observation layer ranks every context position by its largest query-key
// logit across the query heads and keeps the selected-token budget; the
// sparse layers assigned to it reuse those positions over their own caches.
//
// omni_score_kernel: one workgroup per 256 consecutive slots of a sequence,
// one lane per slot.  The sequence's queries (all H_q heads, bf16) sit in
// LDS; a lane reads its slot's key for each KV head in turn (16-byte chunks,
// the next head's chunks in flight while the current head is scored) and
// takes r(j) = max over the query heads of q_a . k_{a/G, j}, with bf16 pair
// dot products accumulated in fp32 (v_dot2c_f32_bf16; the products are
// exact).  The K read is the whole cache once: the kernel is bound by HBM.
// The top-b of r and its conversion to page entries with token masks use the
// kept-slot list kernels of the large eviction path (one unit per sequence).
#include "sp_internal.h"

namespace spk {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kOmniThreads = 256;
constexpr int kOmniMaxHq = 128;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b),
                                         c, false);
}

template <int D>
__global__ void __launch_bounds__(kOmniThreads)
omni_score_kernel(KVDev kv, const bf16_t* __restrict__ q, float* __restrict__ scores, int slot_cap) {
  constexpr int NC = D / 8;                    // 16-byte chunks of a key
  extern __shared__ __align__(16) uint32_t qs[];   // [H_q][D / 2] bf16 pairs
  const int b = blockIdx.y, tid = threadIdx.x;
  const int P = kv.P, Hkv = kv.Hkv, G = kv.G, Hq = kv.Hq;
  const int cap = kv.max_pages * P;
  const int L = clamp_len(kv.seq_lens[b], cap);
  const int j0 = blockIdx.x * kOmniThreads;
  if (j0 >= L) return;
  const uint4* qsrc = reinterpret_cast<const uint4*>(q + (size_t)b * Hq * D);
  for (int i = tid; i < Hq * D / 8; i += kOmniThreads) reinterpret_cast<uint4*>(qs)[i] = qsrc[i];
  const int j = min(j0 + tid, L - 1);          // lanes past L score the last slot again (not stored)
  const int blk = kv.block_table[(size_t)b * kv.max_pages + j / P];
  const int bl = (blk >= 0 && blk < kv.num_blocks) ? blk : 0;   // invalid ids read block 0
  const bf16_t* kp = reinterpret_cast<const bf16_t*>(kv.k_pool);
  auto load = [&](uint4 (&k)[NC], int h) {
    const bf16_t* src = kp + page_base(bl, h, Hkv, P, D) + (size_t)(j % P) * 8;
#pragma unroll
    for (int c = 0; c < NC; ++c) k[c] = *reinterpret_cast<const uint4*>(src + (size_t)c * P * 8);
  };
  uint4 ka[NC], kb[NC];
  load(ka, 0);
  __syncthreads();
  float best = -INFINITY;
  for (int h = 0; h < Hkv; h += 2) {
    if (h + 1 < Hkv) load(kb, h + 1);
    for (int a = h * G; a < (h + 1) * G; ++a) {
      const uint4* qa = reinterpret_cast<const uint4*>(qs + a * (D / 2));
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint4 qv = qa[c];
        acc = dot2(ka[c].x, qv.x, acc);
        acc = dot2(ka[c].y, qv.y, acc);
        acc = dot2(ka[c].z, qv.z, acc);
        acc = dot2(ka[c].w, qv.w, acc);
      }
      best = fmaxf(best, acc);
    }
    if (h + 1 >= Hkv) break;
    if (h + 2 < Hkv) load(ka, h + 2);
    for (int a = (h + 1) * G; a < (h + 2) * G; ++a) {
      const uint4* qa = reinterpret_cast<const uint4*>(qs + a * (D / 2));
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint4 qv = qa[c];
        acc = dot2(kb[c].x, qv.x, acc);
        acc = dot2(kb[c].y, qv.y, acc);
        acc = dot2(kb[c].z, qv.z, acc);
        acc = dot2(kb[c].w, qv.w, acc);
      }
      best = fmaxf(best, acc);
    }
  }
  if (j0 + tid < L) scores[(size_t)b * slot_cap + j0 + tid] = best;
}

}  // namespace

int omnikv_max_q_heads() { return kOmniMaxHq; }

hipError_t launch_omnikv_select(const KVDev& kv, const void* q, int top_b, int32_t* sel_pages,
                                uint32_t* sel_mask, int k_pages, float* token_scores, int slot_cap, void* ws,
                                hipStream_t s) {
  const int cap = kv.max_pages * kv.P;
  const dim3 grid((cap + kOmniThreads - 1) / kOmniThreads, kv.B);
  const size_t lds = (size_t)kv.Hq * kv.D * sizeof(bf16_t);
  const bf16_t* qb = static_cast<const bf16_t*>(q);
  if (kv.D == 64) omni_score_kernel<64><<<grid, kOmniThreads, lds, s>>>(kv, qb, token_scores, slot_cap);
  else omni_score_kernel<128><<<grid, kOmniThreads, lds, s>>>(kv, qb, token_scores, slot_cap);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_token_topk_pages(kv, token_scores, slot_cap, top_b, ws, sel_pages, sel_mask, k_pages, s);
}

}  // namespace spk
