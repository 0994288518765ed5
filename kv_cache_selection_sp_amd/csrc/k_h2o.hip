// H2O score accumulation and eviction with order-preserving physical compaction.
//
// "SparseEngine: Sparse-First Inference Engine", Appendix A.3, "H2O:
// Accumulated Scores and Online Eviction": attention over the available set
// adds its weights to persistent scores (the newest token starts at zero); the
// retained set is a protected recent window plus the highest-scoring older
// tokens; KV outside it is evicted and retained scores persist.  Section 3.1,
// "Architectural Foundations": physical eviction rewrites the retained-slot
// mapping and the context length.
//
// Eviction runs one workgroup per (sequence, KV head).  The candidates are the
// slots before the window; radix select over their order-preserving score keys
// finds the (budget - window)-th largest, ties going to lower slots.  Kept slots
// are then compacted in ascending tiles of kTile slots: every kept slot's
// destination is its rank among kept slots, which is never above its source,
// so reading a whole tile into registers before writing it is race-free in
// place (a tile's writes land below every slot a later tile reads).
#include "sp_internal.h"

namespace spk {
namespace {

constexpr int kAccThreads = 256;
constexpr int kEvictThreads = 1024;
constexpr int kTile = 256;

__global__ void __launch_bounds__(kAccThreads)
h2o_accumulate_kernel(KVDev kv, const float* __restrict__ logits, const float* __restrict__ lse,
                      int logit_cap, int n_new, float* __restrict__ scores, int slot_cap) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int j = blockIdx.x * kAccThreads + threadIdx.x;
  const int L = clamp_len(kv.seq_lens[b], kv.max_pages * kv.P);
  if (j >= L) return;
  float* sp = scores + ((size_t)b * kv.Hkv + h) * slot_cap + j;
  float s = (j >= L - n_new) ? 0.f : *sp;
  for (int a = h * kv.G; a < (h + 1) * kv.G; ++a) {
    const size_t ra = (size_t)b * kv.Hq + a;
    s += expf(logits[ra * logit_cap + j] - lse[ra]);
  }
  *sp = s;
}

template <typename T>
__global__ void __launch_bounds__(kEvictThreads)
h2o_evict_kernel(KVDev kv, float* __restrict__ scores, int32_t* __restrict__ slot_pos, int slot_cap,
                 int budget, int window) {
  constexpr int E = Chunk<T>::E;
  __shared__ int hist[256];
  __shared__ int wsum[kEvictThreads / 64 + 1];
  __shared__ int s_digit, s_excl;
  __shared__ int mv_src[kTile], mv_dst[kTile];

  const int h = blockIdx.x, b = blockIdx.y;
  const int P = kv.P, D = kv.D;
  const int L = clamp_len(kv.seq_lens[b], kv.max_pages * P);
  if (L <= budget) return;
  const int nc = L - window;             // candidate slots [0, nc)
  const int keep_c = budget - window;    // candidates to keep
  float* srow = scores + ((size_t)b * kv.Hkv + h) * slot_cap;
  int32_t* prow = slot_pos ? slot_pos + ((size_t)b * kv.Hkv + h) * slot_cap : nullptr;
  const int tid = threadIdx.x;

  // ---- threshold: keep_c-th largest candidate key (keys re-read from L2 per pass)
  uint32_t prefix = 0, mask = 0;
  int krem = keep_c;
  if (keep_c > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < nc; i += kEvictThreads) {
        const uint32_t k = float_key(srow[i]);
        if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255], 1);
      }
      __syncthreads();
      const int v = tid < 256 ? hist[255 - tid] : 0;
      int total;
      const int excl = block_exclusive_scan<kEvictThreads>(v, wsum, &total);
      if (tid < 256 && excl < krem && krem <= excl + v) {
        s_digit = 255 - tid;
        s_excl = excl;
      }
      __syncthreads();
      prefix |= (uint32_t)s_digit << shift;
      mask |= 0xFFu << shift;
      krem -= s_excl;
      __syncthreads();
    }
  }

  // ---- compaction, ascending tiles
  const int Hkv = kv.Hkv;
  T* kpool = reinterpret_cast<T*>(kv.k_pool);
  T* vpool = reinterpret_cast<T*>(kv.v_pool);
  const int32_t* bt = kv.block_table + (size_t)b * kv.max_pages;
  const int nblk = kv.num_blocks;
  auto blk_ok = [nblk](int blk) { return blk >= 0 && blk < nblk; };   // others are skipped
  int eq_carry = 0, keep_carry = 0;
  for (int t0 = 0; t0 < L; t0 += kTile) {
    // flags: threads [0, kTile) own slots t0 + tid; the others contribute zeros
    const int s = t0 + tid;
    const bool mine = tid < kTile && s < L;
    int eq = 0, gt = 0;
    if (mine && s < nc && keep_c > 0) {
      const uint32_t k = float_key(srow[s]);
      gt = k > prefix;
      eq = k == prefix;
    }
    int eq_tot, keep_tot;
    const int eq_rank = eq_carry + block_exclusive_scan<kEvictThreads>(eq, wsum, &eq_tot);
    const int keep = mine && (s >= nc || gt || (eq && eq_rank < krem)) ? 1 : 0;
    const int dst = keep_carry + block_exclusive_scan<kEvictThreads>(keep, wsum, &keep_tot);
    eq_carry += eq_tot;
    // ordered list of this tile's moves (kept slots whose destination changes)
    const int is_mv = (keep && dst != s) ? 1 : 0;
    int n_mv;
    const int mv_rank = block_exclusive_scan<kEvictThreads>(is_mv, wsum, &n_mv);
    if (is_mv) {
      mv_src[mv_rank] = s;
      mv_dst[mv_rank] = dst;
    }
    keep_carry += keep_tot;
    __syncthreads();
    if (n_mv > 0) {
      // phase A: read every moving slot's payload into registers
      constexpr int kMaxKTasks = (kTile * 16 + kEvictThreads - 1) / kEvictThreads;  // <= D/E chunks
      const int nch = D / E;
      uint4 kreg[kMaxKTasks * 2];
#pragma unroll
      for (int k = 0; k < kMaxKTasks * 2; ++k) kreg[k] = make_uint4(0u, 0u, 0u, 0u);
      const int nk = n_mv * nch;
      // V elements: move index fastest so consecutive threads touch adjacent
      // tokens of one dim row
      constexpr int kMaxVTasks = kTile * 128 / kEvictThreads;
      T vreg[kMaxVTasks];
#pragma unroll
      for (int k = 0; k < kMaxVTasks; ++k) vreg[k] = T(0);
      const int nv = n_mv * D;
      float sreg = 0.f;
      int32_t preg = 0;
#pragma unroll
      for (int k = 0; k < kMaxKTasks * 2; ++k) {
        const int i = tid + k * kEvictThreads;
        if (i < nk) {
          const int m = i % n_mv, c = i / n_mv;
          const int src = mv_src[m];
          const int blk = bt[src / P];
          if (blk_ok(blk))
            kreg[k] = *reinterpret_cast<const uint4*>(kpool + page_base(blk, h, Hkv, P, D) +
                                                      (size_t)(c * P + src % P) * E);
        }
      }
#pragma unroll
      for (int k = 0; k < kMaxVTasks; ++k) {
        const int i = tid + k * kEvictThreads;
        if (i < nv) {
          const int m = i % n_mv, d = i / n_mv;
          const int src = mv_src[m];
          const int blk = bt[src / P];
          if (blk_ok(blk)) vreg[k] = vpool[page_base(blk, h, Hkv, P, D) + v_off(src % P, d, P)];
        }
      }
      if (tid < n_mv) {
        sreg = srow[mv_src[tid]];
        if (prow) preg = prow[mv_src[tid]];
      }
      __syncthreads();
      // phase B: write to the destinations
#pragma unroll
      for (int k = 0; k < kMaxKTasks * 2; ++k) {
        const int i = tid + k * kEvictThreads;
        if (i < nk) {
          const int m = i % n_mv, c = i / n_mv;
          const int dst_s = mv_dst[m];
          const int blk = bt[dst_s / P];
          if (blk_ok(blk))
            *reinterpret_cast<uint4*>(kpool + page_base(blk, h, Hkv, P, D) +
                                      (size_t)(c * P + dst_s % P) * E) = kreg[k];
        }
      }
#pragma unroll
      for (int k = 0; k < kMaxVTasks; ++k) {
        const int i = tid + k * kEvictThreads;
        if (i < nv) {
          const int m = i % n_mv, d = i / n_mv;
          const int dst_s = mv_dst[m];
          const int blk = bt[dst_s / P];
          if (blk_ok(blk)) vpool[page_base(blk, h, Hkv, P, D) + v_off(dst_s % P, d, P)] = vreg[k];
        }
      }
      if (tid < n_mv) {
        srow[mv_dst[tid]] = sreg;
        if (prow) prow[mv_dst[tid]] = preg;
      }
    }
    __syncthreads();
  }
}

__global__ void clamp_lens_kernel(int32_t* seq_lens, int B, int budget, int cap) {
  for (int b = blockIdx.x * blockDim.x + threadIdx.x; b < B; b += gridDim.x * blockDim.x) {
    const int L = clamp_len(seq_lens[b], cap);
    if (L > budget) seq_lens[b] = budget;
  }
}

template <typename T>
hipError_t evict_t(const KVDev& kv, float* scores, int32_t* slot_pos, int slot_cap, int budget,
                   int window, hipStream_t s) {
  dim3 grid(kv.Hkv, kv.B);
  h2o_evict_kernel<T><<<grid, kEvictThreads, 0, s>>>(kv, scores, slot_pos, slot_cap, budget, window);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  clamp_lens_kernel<<<1, 256, 0, s>>>(kv.seq_lens, kv.B, budget, kv.max_pages * kv.P);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_h2o_accumulate(const KVDev& kv, const float* logits, const float* lse,
                                 int logit_cap, int n_new, float* scores, int slot_cap,
                                 hipStream_t s) {
  const int cap = kv.max_pages * kv.P;
  dim3 grid((cap + kAccThreads - 1) / kAccThreads, kv.Hkv, kv.B);
  h2o_accumulate_kernel<<<grid, kAccThreads, 0, s>>>(kv, logits, lse, logit_cap, n_new, scores, slot_cap);
  return hipGetLastError();
}

hipError_t launch_h2o_evict(const KVDev& kv, int dtype, float* scores, int32_t* slot_pos,
                            int slot_cap, int budget, int window, hipStream_t s) {
  if (dtype == SP_BF16) return evict_t<bf16_t>(kv, scores, slot_pos, slot_cap, budget, window, s);
  return evict_t<float>(kv, scores, slot_pos, slot_cap, budget, window, s);
}

}  // namespace spk
