// Quest page scoring and per-KV-head top-k.
//
// "SparseEngine: Sparse-First Inference Engine", Appendix A.3, "Quest:
// Query-Dependent Page Selection": a page's estimate upper-bounds the
// query-key logit of every token in it (it need not equal any token's logit),
// and pages are ranked by that estimate.  For query head a and page p,
//   U_a(p) = sum_c max(q_ac * min_pc, q_ac * max_pc).
// Since max(q*m, q*M) = max(q,0)*M + min(q,0)*m exactly (min <= max), the
// KV-head score S_h(p) = sum_{a in group} U_a(p) equals
//   sum_c Qpos_c * max_pc + Qneg_c * min_pc,
//   Qpos_c = sum_a max(q_ac, 0),  Qneg_c = sum_a min(q_ac, 0),
// i.e. one FMA per summary element for the whole group.  Only the fp32
// summation order differs from the definition.
//
// Scoring streams the page summaries: a page's 2*D summary values are read by
// LPP lanes with one 16-byte load each.  A workgroup owns a long chunk of one
// (sequence, KV head)'s pages, stages their block ids in LDS once, and then
// keeps two groups of loads in flight per wave, so the scan runs at streaming
// bandwidth instead of waiting on a block-table lookup per page.
//
// Top-k runs in the same launch: the last workgroup of a (sequence, KV head)
// to finish scoring (per-unit arrival counter; scores published with
// device-scope stores) selects that unit's pages.  Radix select over
// order-preserving 32-bit keys in LDS finds the k-th largest key.  The select
// starts at the highest bit where the unit's keys differ (all keys share the
// bits above it) and uses 11-bit digits, so it takes at most three passes, and
// it stops early when the boundary bin is taken whole.  Pages above the k-th
// key are taken, and among pages equal to it the lowest indices, so ties go to
// the lower page.  The chosen pages are written in ascending order, their
// positions found with wave ballots and two block scans.
#include "sp_internal.h"

namespace spk {
namespace {

constexpr int kScoreThreads = 256;
constexpr int kScoreWaves = kScoreThreads / 64;
constexpr int kGroup = 8;             // page rows per load group: loads in flight per lane
constexpr int kMaxChunk = 1024;       // pages per workgroup (their block ids sit in LDS)
constexpr int kScoreWgTarget = 512;   // workgroups per call: one resident round on 256 CUs
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T, int D>
struct ScoreShape {
  static constexpr int E = Chunk<T>::E;
  static constexpr int LPP = 2 * D / E;                   // lanes per page summary
  static constexpr int PPR = 64 / LPP;                    // pages per wave row
  static_assert(LPP <= 64 && (64 % LPP) == 0, "summary chunks must tile a wavefront");
};

// Top-k of one (sequence, KV head) by the workgroup that finished its
// scoring last; the scores are read with device-scope loads into LDS keys.
// Thread t owns the contiguous key run [t*R, (t+1)*R) (R a multiple of 4,
// read with 16-byte LDS loads).  Radix select over 11-bit digits from the
// highest bit where the keys differ; once the boundary bin holds at most 64
// keys, one wave finds the exact k-th largest key among them by counting, and
// a boundary bin taken whole ends the search at once.  The chosen pages are
// written in ascending order: per-run counts and two block scans.
constexpr int kCand = 64;

struct TopkLds {
  uint32_t* keys;   // [R * kScoreThreads]
  int* hist;        // [kBins]
  int* wsum;        // [kScoreWaves + 1]
  uint32_t* cand;   // [kCand]
  int* sh;          // [8]
};

__device__ void topk_unit(const float* __restrict__ row, int N, int top_k, int32_t* __restrict__ out,
                          const TopkLds& S) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (top_k >= N) {                          // every page is selected
    for (int i = tid; i < top_k; i += kScoreThreads) out[i] = i < N ? i : -1;
    return;
  }
  uint32_t* keys = S.keys;
  int* hist = S.hist;
  int* sh = S.sh;
  const int R = ((N + kScoreThreads - 1) / kScoreThreads + 3) & ~3;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  // the scores, 8 independent loads in flight per thread
  for (int i = tid; i < R * kScoreThreads; i += 8 * kScoreThreads) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int ie = i + e * kScoreThreads;
      v[e] = ie < N ? __hip_atomic_load(row + ie, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int ie = i + e * kScoreThreads;
      if (ie < R * kScoreThreads) {
        const uint32_t k = ie < N ? float_key(v[e]) : 0u;
        if (ie < N) { kmin = min(kmin, k); kmax = max(kmax, k); }
        keys[ie] = k;
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
  }
  if (lane == 0) { hist[2 * wid] = (int)kmin; hist[2 * wid + 1] = (int)kmax; }
  if (tid == 0) sh[3] = 0;
  __syncthreads();
  kmin = 0xffffffffu;
  kmax = 0u;
#pragma unroll
  for (int w = 0; w < kScoreWaves; ++w) {
    kmin = min(kmin, (uint32_t)hist[2 * w]);
    kmax = max(kmax, (uint32_t)hist[2 * w + 1]);
  }
  const int i0 = tid * R;
  // the run of this thread, 4 keys at a time: f(index, key)
  auto for_run = [&](auto&& f) {
    for (int x = 0; x < R; x += 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(keys + i0 + x);
      f(i0 + x, v.x); f(i0 + x + 1, v.y); f(i0 + x + 2, v.z); f(i0 + x + 3, v.w);
    }
  };
  // keys with (key & mask) > prefix are taken; of those with (key & mask) ==
  // prefix, the krem with the lowest indices are taken
  const uint32_t diff = kmin ^ kmax;
  const uint32_t common = diff == 0u ? 0xffffffffu : ~(0xffffffffu >> __clz(diff));
  uint32_t prefix = kmax & common, mask = common;
  int hb = diff == 0u ? -1 : 31 - __clz(diff);    // highest bit still undecided
  int krem = top_k;
  __syncthreads();                                 // hist is reused below
  while (hb >= 0) {
    const int shift = hb >= kDigitBits - 1 ? hb - (kDigitBits - 1) : 0;
    const int nb = 1 << (hb - shift + 1);
    for (int i = tid; i < nb; i += kScoreThreads) hist[i] = 0;
    __syncthreads();
    for_run([&](int i, uint32_t k) {
      if (i < N && (k & mask) == prefix) atomicAdd(&hist[(k >> shift) & (uint32_t)(nb - 1)], 1);
    });
    __syncthreads();
    // thread t owns bins (hi - bpt, hi], counted from the top
    const int bpt = nb >= kScoreThreads ? nb / kScoreThreads : 1;
    const int hi = nb - 1 - tid * bpt;
    int c = 0;
    for (int x = 0; x < bpt; ++x)
      if (hi - x >= 0) c += hist[hi - x];
    int total;
    int above = block_exclusive_scan<kScoreThreads>(c, S.wsum, &total);
    if (above < krem && krem <= above + c) {
      for (int x = 0; x < bpt; ++x) {
        const int cb = hist[hi - x];
        if (krem <= above + cb) { sh[0] = hi - x; sh[1] = above; sh[2] = cb; break; }
        above += cb;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sh[0] << shift;
    mask |= (uint32_t)(nb - 1) << shift;
    krem -= sh[1];
    hb = shift - 1;
    const int cb = sh[2];
    if (krem == cb || hb < 0) break;               // bin taken whole, or key fully resolved
    if (cb <= kCand) {
      // the boundary bin's keys, unordered, into LDS; one wave finds the
      // krem-th largest of them by counting
      for_run([&](int i, uint32_t k) {
        if (i < N && (k & mask) == prefix) S.cand[atomicAdd(&sh[3], 1)] = k;
      });
      __syncthreads();
      if (wid == 0 && lane < cb) {
        const uint32_t v = S.cand[lane];
        int g = 0, e = 0;
        for (int x = 0; x < cb; ++x) {
          const uint32_t y = S.cand[x];
          g += y > v;
          e += y >= v;
        }
        if (g < krem && krem <= e) { sh[4] = (int)v; sh[5] = g; }
      }
      __syncthreads();
      prefix = (uint32_t)sh[4];
      mask = 0xffffffffu;
      krem -= sh[5];
      break;
    }
    __syncthreads();
  }
  // index-ordered output over the runs
  int n_eq = 0;
  for_run([&](int i, uint32_t k) { n_eq += i < N && (k & mask) == prefix; });
  int tot;
  const int eq_rank0 = block_exclusive_scan<kScoreThreads>(n_eq, S.wsum, &tot);
  int n_take = 0, r = eq_rank0;
  for_run([&](int i, uint32_t k) {
    const uint32_t km = k & mask;
    const bool eq = i < N && km == prefix;
    n_take += i < N && (km > prefix || (eq && r < krem));
    r += eq;
  });
  int pos = block_exclusive_scan<kScoreThreads>(n_take, S.wsum, &tot);
  r = eq_rank0;
  for_run([&](int i, uint32_t k) {
    const uint32_t km = k & mask;
    const bool eq = i < N && km == prefix;
    if (i < N && (km > prefix || (eq && r < krem))) out[pos++] = i;
    r += eq;
  });
}

// One workgroup per (sequence, KV head, chunk of `chunk` logical pages).  The
// chunk's block ids are staged in LDS, then each wave streams its rows (PPR
// pages each) in groups of kGroup rows through a two-group register ring: a
// group's loads are issued before the previous group is reduced.  Scores are
// published with device-scope stores; the last workgroup of the unit to
// finish (per-unit arrival counter) runs the top-k.
template <typename T, int D>
__global__ void __launch_bounds__(kScoreThreads)
select_kernel(KVDev kv, const T* __restrict__ q, const T* __restrict__ meta, float* __restrict__ scores,
              int chunk, int n_chunks, int top_k, int32_t* __restrict__ sel, int* __restrict__ counters) {
  using S = ScoreShape<T, D>;
  constexpr int E = S::E, LPP = S::LPP, PPR = S::PPR;
  // scoring: qsum, sblk, sc; top-k (after scoring): keys, hist, cand, sh
  extern __shared__ __align__(16) uint32_t lds[];
  float (*qsum)[D] = reinterpret_cast<float (*)[D]>(lds);          // [2][D]: Qneg, Qpos
  int* sblk = reinterpret_cast<int*>(lds + 2 * D);                 // [kMaxChunk]
  float* sc = reinterpret_cast<float*>(lds + 2 * D + kMaxChunk);    // [kMaxChunk] the chunk's scores
  __shared__ int wsum[kScoreWaves + 1];
  __shared__ int s_last;

  const int u = blockIdx.x / n_chunks, c = blockIdx.x % n_chunks;
  const int b = u / kv.Hkv, h = u % kv.Hkv;
  const int P = kv.P, G = kv.G;
  const int L = clamp_len(kv.seq_lens[b], kv.max_pages * P);
  const int n_pages = (L + P - 1) / P;
  const int p_lo = c * chunk, p_hi = min(p_lo + chunk, kv.max_pages);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  float* srow = scores + (size_t)u * kv.max_pages;
  const int32_t* bt_row = kv.block_table + (size_t)b * kv.max_pages;

  for (int d = tid; d < D; d += kScoreThreads) {
    float qp = 0.f, qn = 0.f;
    for (int a = 0; a < G; ++a) {
      const float x = to_f32(q[((size_t)b * kv.Hq + h * G + a) * D + d]);
      qp += x > 0.f ? x : 0.f;
      qn += x < 0.f ? x : 0.f;
    }
    qsum[0][d] = qn;
    qsum[1][d] = qp;
  }
  for (int i = tid; i < p_hi - p_lo; i += kScoreThreads) {
    const int p = p_lo + i;
    int blk = p < n_pages ? bt_row[p] : -1;
    if (blk >= kv.num_blocks) blk = -1;
    sblk[i] = blk;
  }
  __syncthreads();

  const int j = lane % LPP;                 // 16-byte chunk of the summary read by this lane
  const int row = j / (LPP / 2);            // 0: minimum row, 1: maximum row
  const int dim0 = (j % (LPP / 2)) * E;
  const int sub = lane / LPP;
  float w[E];
#pragma unroll
  for (int e = 0; e < E; ++e) w[e] = qsum[row][dim0 + e];

  const int n_rows = (p_hi - p_lo + PPR - 1) / PPR;
  const int my_rows = wave < n_rows ? (n_rows - wave + kScoreWaves - 1) / kScoreWaves : 0;
  const int n_groups = __builtin_amdgcn_readfirstlane((my_rows + kGroup - 1) / kGroup);
  // page of row slot r of group gi (rows of this wave: wave, wave + 4, ...)
  auto page_of = [&](int gi, int r) { return p_lo + (wave + kScoreWaves * (gi * kGroup + r)) * PPR + sub; };
  // loads are unconditional (an invalid page reads block 0's summary and is
  // discarded), so every group issues the same number of loads
  auto issue = [&](u32x4 (&m)[kGroup], int gi) {
#pragma unroll
    for (int r = 0; r < kGroup; ++r) {
      const int p = page_of(gi, r);
      const int blk = p < p_hi ? sblk[p - p_lo] : -1;
      const T* src = meta + ((size_t)(blk < 0 ? 0 : blk) * kv.Hkv + (blk < 0 ? 0 : h)) * 2 * D + j * E;
      m[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
    }
  };
  auto reduce = [&](const u32x4 (&m)[kGroup], int gi) {
#pragma unroll
    for (int r = 0; r < kGroup; ++r) {
      union { u32x4 u; T e[E]; } mm;
      mm.u = m[r];
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) part = fmaf(w[e], to_f32(mm.e[e]), part);
#pragma unroll
      for (int o = LPP / 2; o >= 1; o >>= 1) part += __shfl_xor(part, o, 64);
      const int p = page_of(gi, r);
      if (j == 0 && p < p_hi) sc[p - p_lo] = sblk[p - p_lo] >= 0 ? part : -INFINITY;
    }
  };
  if (n_groups > 0) {
    u32x4 ga[kGroup], gb[kGroup];
    issue(ga, 0);
    __builtin_amdgcn_sched_barrier(0);
    issue(gb, n_groups > 1 ? 1 : 0);
    __builtin_amdgcn_sched_barrier(0);
    for (int gi = 0; gi < n_groups; gi += 2) {
      reduce(ga, gi);
      __builtin_amdgcn_sched_barrier(0);
      issue(ga, gi + 2 < n_groups ? gi + 2 : n_groups - 1);
      __builtin_amdgcn_sched_barrier(0);
      if (gi + 1 < n_groups) reduce(gb, gi + 1);
      __builtin_amdgcn_sched_barrier(0);
      issue(gb, gi + 3 < n_groups ? gi + 3 : n_groups - 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // publish the chunk's scores as one coalesced run of device-scope stores,
  // complete at the point of coherence before the workgroup counts itself in
  __syncthreads();
  for (int i = tid; i < p_hi - p_lo; i += kScoreThreads)
    __hip_atomic_store(srow + p_lo + i, sc[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&counters[u], 1) == n_chunks - 1;
  __syncthreads();
  if (!s_last) return;
  if (tid == 0) __hip_atomic_store(&counters[u], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();                          // the scoring LDS is reused
  TopkLds tl;
  const int R = ((n_pages + kScoreThreads - 1) / kScoreThreads + 3) & ~3;
  tl.keys = lds;
  tl.hist = reinterpret_cast<int*>(lds + R * kScoreThreads);
  tl.cand = lds + R * kScoreThreads + kBins;
  tl.sh = reinterpret_cast<int*>(lds + R * kScoreThreads + kBins + kCand);
  tl.wsum = wsum;
  topk_unit(srow, n_pages, top_k, sel + (size_t)u * top_k, tl);
}

// Dynamic LDS of the select kernel: the larger of the scoring layout and the
// top-k layout for max_pages keys.
inline size_t select_lds_bytes(int max_pages, int D) {
  const size_t score = (size_t)(2 * D + 2 * kMaxChunk) * 4;
  const int R = ((max_pages + kScoreThreads - 1) / kScoreThreads + 3) & ~3;
  const size_t topk = (size_t)(R * kScoreThreads + kBins + kCand + 8) * 4;
  return score > topk ? score : topk;
}

template <typename T, int D>
hipError_t select_t(const KVDev& kv, const void* q, const void* meta, int top_k, int32_t* sel,
                    float* scores, int* counters, hipStream_t s) {
  using S = ScoreShape<T, D>;
  // chunks per unit: about kScoreWgTarget workgroups in all, chunks a
  // multiple of one row per wave and at most kMaxChunk pages
  const int units = kv.B * kv.Hkv;
  const int quantum = S::PPR * kScoreWaves;
  int n_chunks = (kScoreWgTarget + units - 1) / units;
  int chunk = (kv.max_pages + n_chunks - 1) / n_chunks;
  chunk = (chunk + quantum - 1) / quantum * quantum;
  if (chunk > kMaxChunk) chunk = kMaxChunk;
  n_chunks = (kv.max_pages + chunk - 1) / chunk;
  select_kernel<T, D><<<units * n_chunks, kScoreThreads, select_lds_bytes(kv.max_pages, D), s>>>(
      kv, static_cast<const T*>(q), static_cast<const T*>(meta), scores, chunk, n_chunks, top_k, sel,
      counters);
  return hipGetLastError();
}

}  // namespace

size_t select_counter_bytes(const KVDev& kv) {
  return ((size_t)kv.B * kv.Hkv * sizeof(int) + 255) & ~(size_t)255;
}

size_t select_workspace_bytes(const KVDev& kv) {
  return select_counter_bytes(kv) + (size_t)kv.B * kv.Hkv * kv.max_pages * sizeof(float);
}

hipError_t launch_select(const KVDev& kv, int dtype, const void* q, const void* page_meta,
                         int top_k, int32_t* sel, float* page_scores, void* ws, hipStream_t s) {
  int* counters = static_cast<int*>(ws);
  float* scores = page_scores ? page_scores
                              : reinterpret_cast<float*>(static_cast<char*>(ws) + select_counter_bytes(kv));
  if (dtype == SP_BF16) {
    if (kv.D == 128) return select_t<bf16_t, 128>(kv, q, page_meta, top_k, sel, scores, counters, s);
    return select_t<bf16_t, 64>(kv, q, page_meta, top_k, sel, scores, counters, s);
  }
  if (kv.D == 128) return select_t<float, 128>(kv, q, page_meta, top_k, sel, scores, counters, s);
  return select_t<float, 64>(kv, q, page_meta, top_k, sel, scores, counters, s);
}

}  // namespace spk
