// OmniKV token selection at an observation layer.
//
// "SparseEngine: Sparse-First Inference Engine", Appendix A.3, "OmniKV": an
// observation layer ranks every context position by its largest query-key
// logit across the query heads and keeps the selected-token budget; the
// sparse layers assigned to it reuse those positions over their own caches.
//
// omni_score_kernel: each workgroup takes a run of 16-slot tiles (one page
// each) of one sequence, its waves taking every fourth tile.  For a tile it issues the
// loads of every KV head's 16 keys at once (up to eight heads at a time, one 1 KB
// wave load per 32 dims and head, the MFMA operand layout of the K pool),
// then per KV head forms S = Q_group . K^T with v_mfma_f32_16x16x32_bf16 (the
// group's query heads as rows, padded to 16, read from LDS), so a lane holds
// one slot and four head rows; the maximum over the valid rows, the KV heads
// and the four lane rows (gfx950 row swaps) is r(j).  The K read is the whole
// cache once: the kernel is bound by HBM.  The top-b of r and its conversion
// to page entries with token masks use the kept-slot list kernels of the
// large eviction path (one unit per sequence).
#include <algorithm>
#include <type_traits>

#include "sp_internal.h"

namespace spk {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kOmniThreads = 256;
constexpr int kOmniMaxHq = 128;
constexpr int kOmniMaxTiles = 1024;     // 16-slot tiles per workgroup at most
constexpr int kRsrcFlags = 0x00020000;  // buffer resource word 3: raw 32-bit dwords
constexpr int kNonTemporal = 2;         // buffer load cache policy: non-temporal

__device__ __forceinline__ float max_rows4(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int D, int NH>
__global__ void __launch_bounds__(kOmniThreads)
omni_score_kernel(KVDev kv, const bf16_t* __restrict__ q, float* __restrict__ scores, int slot_cap,
                  int tiles_per_wg) {
  constexpr int KS = D / 32;
  extern __shared__ __align__(16) uint4 qsh[];    // [H_q][D / 8] 16-byte chunks, then block ids
  const int b = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = lane & 15, g = lane >> 4;
  const int P = kv.P, Hkv = kv.Hkv, G = kv.G, Hq = kv.Hq;
  const int cap = kv.max_pages * P;
  const int L = clamp_len(kv.seq_lens[b], cap);
  const int n_tiles = (L + 15) / 16;
  const int t0 = blockIdx.x * tiles_per_wg, t1 = min(n_tiles, t0 + tiles_per_wg);
  if (t0 >= t1) return;
  // q and the block ids of the pages the tiles cover (a 16-slot tile lies in
  // one page) go to LDS, four loads per thread in flight (unconditional, at
  // clamped indices, so none waits behind a branch)
  const uint4* qsrc = reinterpret_cast<const uint4*>(q + (size_t)b * Hq * D);
  int* bsh = reinterpret_cast<int*>(qsh + Hq * D / 8);
  const int32_t* bt = kv.block_table + (size_t)b * kv.max_pages;
  const int pg0 = t0 * 16 / P, pg1 = (t1 * 16 - 1) / P + 1;
  const int blk0 = bt[min(pg0 + tid, pg1 - 1)];
  for (int i0 = 0; i0 < Hq * D / 8; i0 += 4 * kOmniThreads) {
    uint4 v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      v[r] = qsrc[min(i0 + r * kOmniThreads + tid, Hq * D / 8 - 1)];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      qsh[min(i0 + r * kOmniThreads + tid, Hq * D / 8 - 1)] = v[r];   // clamped lanes rewrite the last chunk
    }
  }
  for (int i = tid; i < pg1 - pg0; i += kOmniThreads) {
    const int blk = i == tid ? blk0 : bt[pg0 + i];
    bsh[i] = (blk >= 0 && blk < kv.num_blocks) ? blk : 0;   // invalid ids read block 0
  }
  __syncthreads();
  const bf16_t* kp = reinterpret_cast<const bf16_t*>(kv.k_pool);
  const int qrow = t < G ? t : 0;                 // rows past the group read row 0 (masked below)
  for (int tile = t0 + wid; tile < t1; tile += kOmniThreads / 64) {
    const int tok0 = tile * 16;
    const int page = tok0 / P;
    const int blk = __builtin_amdgcn_readfirstlane(bsh[page - pg0]);
    // the block's K pages of every head, read once: non-temporal buffer loads
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t*>(kp + page_base(blk, 0, Hkv, P, D)), (short)0, Hkv * P * D * 2, kRsrcFlags);
    const int off = tok0 - page * P;
    float best = -INFINITY;
    for (int h0 = 0; h0 < Hkv; h0 += NH) {
      uint4 kr[NH][KS];
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        const int h = min(h0 + hh, Hkv - 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          kr[hh][ks] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                           rk, (h * D / 8 + 4 * ks + g) * P * 16 + t * 16, off * 16, kNonTemporal));
      }
      // all of the group's loads are issued before the first product
      __builtin_amdgcn_sched_barrier(0);
      // every head of the group is scored (a clamped head repeats the last
      // one, which leaves the maximum unchanged), so no load is conditional
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        const uint4* qa = qsh + (min(h0 + hh, Hkv - 1) * G + qrow) * (D / 8);
        float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa[4 * ks + g]),
                                                        __builtin_bit_cast(bf16x8_t, kr[hh][ks]), acc, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * g + e < G) best = fmaxf(best, acc[e]);
      }
    }
    best = max_rows4(best);
    if (g == 0 && tok0 + t < L) scores[(size_t)b * slot_cap + tok0 + t] = best;
  }
}

}  // namespace

int omnikv_max_q_heads() { return kOmniMaxHq; }
int omnikv_max_group() { return 16; }

hipError_t launch_omnikv_select(const KVDev& kv, const void* q, int top_b, int32_t* sel_pages,
                                uint32_t* sel_mask, int k_pages, float* token_scores, int slot_cap, void* ws,
                                hipStream_t s) {
  const int cap = kv.max_pages * kv.P;
  const size_t lds = (size_t)kv.Hq * kv.D * sizeof(bf16_t) + kOmniMaxTiles * sizeof(int);
  const bf16_t* qb = static_cast<const bf16_t*>(q);
  // KV heads in flight per tile: up to eight, no more than the cache has.
  // The grid is one round of resident workgroups: the 16-slot tiles of every
  // sequence are split evenly over them (whole waves' worth each).
  hipError_t err = hipSuccess;
  auto run = [&](auto d, auto nh) {
    auto* kern = omni_score_kernel<decltype(d)::value, decltype(nh)::value>;
    int dev = 0, cus = 0, per_cu = 0;
    if ((err = hipGetDevice(&dev)) != hipSuccess) return;
    if ((err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return;
    if ((err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kOmniThreads, lds)) != hipSuccess)
      return;
    const long long tiles = (long long)kv.B * ((cap + 15) / 16);
    const long long resident = (long long)std::max(cus, 1) * std::max(per_cu, 1);
    const int waves = kOmniThreads / 64;
    long long per = (tiles + resident - 1) / resident;
    per = std::max<long long>(waves, (per + waves - 1) / waves * waves);
    const int tiles_per_wg = (int)std::min<long long>(std::min<long long>(per, kOmniMaxTiles), (cap + 15) / 16);
    const dim3 grid(((cap + 15) / 16 + tiles_per_wg - 1) / tiles_per_wg, kv.B);
    kern<<<grid, kOmniThreads, lds, s>>>(kv, qb, token_scores, slot_cap, tiles_per_wg);
  };
  using D64 = std::integral_constant<int, 64>;
  using D128 = std::integral_constant<int, 128>;
  auto by_heads = [&](auto d) {
    if (kv.Hkv >= 8) run(d, std::integral_constant<int, 8>{});
    else if (kv.Hkv >= 4) run(d, std::integral_constant<int, 4>{});
    else if (kv.Hkv >= 2) run(d, std::integral_constant<int, 2>{});
    else run(d, std::integral_constant<int, 1>{});
  };
  if (kv.D == 64) by_heads(D64{});
  else by_heads(D128{});
  if (err != hipSuccess) return err;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_token_topk_pages(kv, token_scores, slot_cap, top_b, ws, sel_pages, sel_mask, k_pages, s);
}

}  // namespace spk
