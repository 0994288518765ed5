// Device code of the Quest page scoring and top-k (select_kernel) as inline
// functions, shared by the selection launch and the fused decode step.  See
// k_select.hip for the method and the design.
#pragma once
#include "sp_internal.h"

namespace spk {
namespace seldev {

constexpr int kScoreThreads = 256;
constexpr int kScoreWaves = kScoreThreads / 64;
constexpr int kGroup = 4;             // page rows per load group: loads in flight per lane
// a scoring chunk is at most 4 pages per thread (their block ids sit in LDS)
constexpr int kScoreWgTarget = 512;   // workgroups per call: one resident round on 256 CUs
constexpr int kQPer = 8;              // query elements loaded per thread per pass
constexpr int kGroupMaxHeads = 16;    // max-over-group aggregation: query heads per KV head
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Sum of v over aligned groups of LPP lanes (LPP in {16, 32, 64}), returned
// in every lane of the group: DPP steps within each 16-lane row, a swizzle
// for 16 -> 32 and a lane permute for 32 -> 64.
template <int LPP>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp_partner<kDppSwap1>(v);
  v += dpp_partner<kDppSwap2>(v);
  v += dpp_partner<kDppHalfMirror>(v);
  v += dpp_partner<kDppMirror>(v);
  if constexpr (LPP >= 32) v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), kSwizzleXor16));
  if constexpr (LPP >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// Maximum over GP heads (a power of two, 2..16) of a page's bound, for 32
// lanes per page, by a reduce-scatter over the heads instead of one 32-lane
// sum per head.  pa[s] is this lane's partial dot product for slot s; lane l
// holds in slot s the head s ^ hmask(l), hmask taking GP/4, GP/8, GP/16 from
// lane bits 1, 0 and 3 (see max_slot_mask).  Each exchange level halves the
// slots: across lane bit 4 (the min and max summary rows) a row swap, then
// across bits 1, 0 and 3 DPP moves, a lane keeping the first half of its
// slots and adding its partner's second half, which holds the same heads.
// The lane bits left over are summed (DPP rotations by 4 and 8 within the
// row sum bits 2 and 3 together; a swizzle sums bit 2 alone), and the maximum
// is taken across the exchange bits.  Every lane ends with the maximum.
constexpr int kDppRor4 = 0x124;        // row_ror:4: lane (i + 4) mod 16 within each 16 lanes
constexpr int kDppRor8 = 0x128;        // row_ror:8: lane i ^ 8 within each 16 lanes
constexpr int kSwizzleXor4 = 0x101f;   // bitmask swizzle: lane ^ 4 within 32

__device__ __forceinline__ int max_slot_mask(int lane, int GP) {
  int m = 0;
  if (GP >= 4 && (lane & 2)) m ^= GP / 4;
  if (GP >= 8 && (lane & 1)) m ^= GP / 8;
  if (GP >= 16 && (lane & 8)) m ^= GP / 16;
  return m;
}

template <int GP>
__device__ __forceinline__ float scatter_max32(float (&pa)[GP]) {
#pragma unroll
  for (int s = 0; s < GP / 2; ++s) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(pa[s]), __float_as_uint(pa[s + GP / 2]),
                                                    false, false);
    pa[s] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
  if constexpr (GP >= 4) {
#pragma unroll
    for (int s = 0; s < GP / 4; ++s) pa[s] += dpp_partner<kDppSwap2>(pa[s + GP / 4]);
  }
  if constexpr (GP >= 8) {
#pragma unroll
    for (int s = 0; s < GP / 8; ++s) pa[s] += dpp_partner<kDppSwap1>(pa[s + GP / 8]);
  }
  if constexpr (GP >= 16) pa[0] += dpp_partner<kDppRor8>(pa[1]);
  float v = pa[0];
  if constexpr (GP == 2) {
    v += dpp_partner<kDppSwap1>(v);
    v += dpp_partner<kDppSwap2>(v);
    v += dpp_partner<kDppHalfMirror>(v);
    v += dpp_partner<kDppMirror>(v);
  } else if constexpr (GP == 4) {
    v += dpp_partner<kDppSwap1>(v);
    v += dpp_partner<kDppRor4>(v);
    v += dpp_partner<kDppRor8>(v);
  } else if constexpr (GP == 8) {
    v += dpp_partner<kDppRor4>(v);
    v += dpp_partner<kDppRor8>(v);
  } else {
    v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), kSwizzleXor4));
  }
  {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  }
  if constexpr (GP >= 4) v = fmaxf(v, dpp_partner<kDppSwap2>(v));
  if constexpr (GP >= 8) v = fmaxf(v, dpp_partner<kDppSwap1>(v));
  if constexpr (GP >= 16) v = fmaxf(v, dpp_partner<kDppRor8>(v));
  return v;
}

// The group maximum of one page row: this lane's GP packed dot products
// (v_dot2_f32_bf16 over its 8 summary values), then scatter_max32.
template <int GP>
__device__ __forceinline__ float row_max32(const uint32_t (&w2)[kGroupMaxHeads][4], const u32x4& x) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  float pa[GP];
#pragma unroll
  for (int sl = 0; sl < GP; ++sl) {
    float pr = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      pr = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w2[sl][i]),
                                           __builtin_bit_cast(bf16x2_t, (uint32_t)x[i]), pr, false);
    pa[sl] = pr;
  }
  return scatter_max32<GP>(pa);
}

template <typename T, int D>
struct ScoreShape {
  static constexpr int E = Chunk<T>::E;
  static constexpr int LPP = 2 * D / E;                   // lanes per page summary
  static constexpr int PPR = 64 / LPP;                    // pages per wave row
  static_assert(LPP <= 64 && (64 % LPP) == 0, "summary chunks must tile a wavefront");
};

// Top-k of one (sequence, KV head) by the workgroup that finished its
// scoring last.  Thread t owns the contiguous key run [t*R, t*R + R),
// R = ceil(N / NT) <= RM, held in registers; the scores are read with
// device-scope loads, all of a run at once.  Radix select over the range of
// the undecided keys, up to 2048 bins of (key - lo) >> shift per pass; once
// the boundary bin holds at most kCand keys, one wave finds the exact k-th
// largest key among them by counting, and a boundary bin taken whole ends
// the search at once.  The
// chosen pages are written in ascending order: one block scan of the packed
// (greater, equal) counts of the runs gives every run its output position.
constexpr int kCand = 64;

// Fused decode step only: besides the page indices, the top-k writes a
// resolved descriptor per selected page, (block id << 6) | tokens of the page
// (all ones for padding), tagged with the call's epoch of the unit in the high
// word, through to the point of coherence, for the attention workgroups of
// the same launch: a descriptor whose tag is the current epoch is this call's.
// Block ids come from the scoring workgroups' published copy of the
// block-table row.
struct Resolve {
  const int32_t* blk_row = nullptr;   // the sequence's block-table row
  int num_blocks = 0;                 // block ids outside [0, num_blocks) are skipped
  uint64_t* desc = nullptr;           // [top_k] (epoch << 32) | descriptor
  int L = 0, P = 0;                   // the sequence's tokens and the page size
  uint32_t epoch = 0;                 // this call's epoch of the unit
};
// The block id of a page (the block table does not change during the call,
// so a plain load), or -1 if out of range.
__device__ __forceinline__ int resolve_blk(const Resolve& rs, int page) {
  const int bv = rs.blk_row[page];
  return (bv >= 0 && bv < rs.num_blocks) ? bv : -1;
}
__device__ __forceinline__ uint64_t page_desc(int blk, int page, const Resolve& rs) {
  const int nv = min(rs.P, rs.L - page * rs.P);
  const uint32_t d = (blk < 0 || nv <= 0) ? 0xffffffffu : (((uint32_t)blk << 6) | (uint32_t)nv);
  return ((uint64_t)rs.epoch << 32) | d;
}
__device__ __forceinline__ uint64_t pad_desc(const Resolve& rs) { return ((uint64_t)rs.epoch << 32) | 0xffffffffu; }
__device__ __forceinline__ void store_coherent(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t load_coherent(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct TopkLds {
  int* hist;        // [kBins]
  int* wsum;        // [waves + 1]
  int* wsum2;       // [waves + 1]
  uint32_t* cand;   // [kCand]
  int* sh;          // [8 + 2 * waves]
};

template <int RM, bool RES, int NT = kScoreThreads>
__device__ __forceinline__ void topk_unit(const float* __restrict__ row, int N, int top_k, int n_sink, int n_recent,
                          int32_t* __restrict__ out, const TopkLds& S, const Resolve& rs) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (top_k >= N) {                          // every page is selected
    for (int i = tid; i < top_k; i += NT) {
      out[i] = i < N ? i : -1;
      if constexpr (RES) store_coherent(rs.desc + i, i < N ? page_desc(resolve_blk(rs, i), i, rs) : pad_desc(rs));
    }
    return;
  }
  int* hist = S.hist;
  int* sh = S.sh;
  const int R = (N + NT - 1) / NT;
  const int i0 = tid * R;
  const int nv = max(0, min(R, N - i0));     // keys in this thread's run
  uint32_t key[RM];
  {
    float v[RM];
#pragma unroll
    for (int x = 0; x < RM; ++x)
      v[x] = x < nv ? __hip_atomic_load(row + i0 + x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.f;
    // while the loads are in flight: a zero histogram, a zero candidate count
    for (int i = tid; i < kBins; i += NT) hist[i] = 0;
    if (tid == 0) sh[3] = 0;
    // forced pages (the first n_sink, the last n_recent) take the largest
    // key, above every score's key, so the select keeps them
#pragma unroll
    for (int x = 0; x < RM; ++x)
      key[x] = (i0 + x < n_sink || i0 + x >= N - n_recent) ? 0xffffffffu : float_key(v[x]);
  }
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int x = 0; x < RM; ++x)
    if (x < nv) { kmin = min(kmin, key[x]); kmax = max(kmax, key[x]); }
  wave_min_max(kmin, kmax);
  if (lane == 0) { sh[8 + 2 * wid] = (int)kmin; sh[8 + 2 * wid + 1] = (int)kmax; }
  __syncthreads();
  kmin = 0xffffffffu;
  kmax = 0u;
#pragma unroll
  for (int w = 0; w < (NT / 64); ++w) {
    kmin = min(kmin, (uint32_t)sh[8 + 2 * w]);
    kmax = max(kmax, (uint32_t)sh[8 + 2 * w + 1]);
  }
  // Undecided keys lie in [lo, lo + span]: those above are taken, those
  // below are not, and krem of the undecided are still to take.  A pass
  // histograms the undecided keys by (key - lo) >> shift, the shift leaving
  // at most 2048 bins over the span, so the keys spread over the bins
  // whatever bits they share (a digit of the keys' own bits below their
  // highest differing one crowds keys that straddle a power of two into a
  // few bins); the bin holding the krem-th key becomes the new range, at
  // most 2^shift wide, so three passes resolve any span.  The result is a
  // threshold T: keys above T are taken, and of the keys equal to T the krem
  // with the lowest indices.
  uint32_t lo = kmin, span = kmax - kmin;
  uint32_t thr = kmin;
  int krem = top_k;
  // at most three passes narrow any span to one value (each cuts 11 bits)
  for (int pass = 0; pass < 4; ++pass) {
    if (span == 0u) { thr = lo; break; }        // one key value left: ties by index
    const int shift = max(0, 32 - (int)__clz(span) - kDigitBits);
    const int top_bin = (int)(span >> shift);   // < kBins
    const int nb = 1 << (32 - (int)__clz((uint32_t)top_bin));   // power of two > top_bin, <= kBins
#pragma unroll
    for (int x = 0; x < RM; ++x)
      if (x < nv && key[x] - lo <= span) atomicAdd(&hist[(key[x] - lo) >> shift], 1);
    __syncthreads();
    // thread t owns bins (hi - bpt, hi], counted from the top (bpt <= 8;
    // the owned bins are bpt-aligned, so 8 of them are two 16-byte reads)
    const int bpt = nb >= NT ? nb / NT : 1;
    const int hi = nb - 1 - tid * bpt;
    int hv[8];                                   // hv[x] = count of bin hi - x
    if (bpt == 8) {
      const int4 a = *reinterpret_cast<const int4*>(hist + hi - 7);
      const int4 z = *reinterpret_cast<const int4*>(hist + hi - 3);
      hv[0] = z.w; hv[1] = z.z; hv[2] = z.y; hv[3] = z.x;
      hv[4] = a.w; hv[5] = a.z; hv[6] = a.y; hv[7] = a.x;
    } else {
#pragma unroll
      for (int x = 0; x < 8; ++x) hv[x] = (x < bpt && hi - x >= 0) ? hist[hi - x] : 0;
    }
    int c = 0;
#pragma unroll
    for (int x = 0; x < 8; ++x) c += hv[x];
    int total;
    int above = block_scan_dpp<NT>(c, S.wsum, &total);
    if (above < krem && krem <= above + c) {
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        if (x < bpt && krem > above && krem <= above + hv[x]) { sh[0] = hi - x; sh[1] = above; sh[2] = hv[x]; }
        above += hv[x];
      }
    }
    __syncthreads();
    const uint32_t b_lo = (uint32_t)sh[0] << shift;            // the bin's offset from lo
    krem -= sh[1];
    const int cb = sh[2];
    if (krem == cb) {
      // the boundary bin taken whole: every key from lo + b_lo up is taken
      if (lo + b_lo == 0u) { thr = 0u; krem = N; }            // every key (none is below 0)
      else { thr = lo + b_lo - 1u; krem = 0; }
      break;
    }
    const uint32_t nspan = min(span - b_lo, (shift == 0 ? 0u : (1u << shift) - 1u));
    lo += b_lo;
    span = nspan;
    if (cb <= kCand) {
      // the boundary bin's keys, unordered, into LDS; one wave finds the
      // krem-th largest of them by counting, reading the others' keys lane
      // by lane
#pragma unroll
      for (int x = 0; x < RM; ++x)
        if (x < nv && key[x] - lo <= span) S.cand[atomicAdd(&sh[3], 1)] = key[x];
      __syncthreads();
      if (wid == 0) {
        const int cbu = __builtin_amdgcn_readfirstlane(cb);
        const uint32_t v = lane < cbu ? S.cand[lane] : 0u;
        int g = 0, e = 0;
        for (int x = 0; x < cbu; ++x) {
          const uint32_t y = (uint32_t)__builtin_amdgcn_readlane((int)v, x);
          g += y > v;
          e += y >= v;
        }
        if (lane < cbu && g < krem && krem <= e) { sh[4] = (int)v; sh[5] = g; }
      }
      __syncthreads();
      thr = (uint32_t)sh[4];
      krem -= sh[5];
      break;
    }
    // the next pass: clear the bins used (every thread has read them)
    for (int i = tid; i < nb; i += NT) hist[i] = 0;
    __syncthreads();
  }
  const uint32_t prefix = thr, mask = 0xffffffffu;
  // index-ordered output: taken keys before this run = greater keys before
  // it + min(equal keys before it, krem)
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int x = 0; x < RM; ++x) {
    if (x < nv) {
      const uint32_t km = key[x] & mask;
      n_gt += km > prefix;
      n_eq += km == prefix;
    }
  }
  int tot;
  const int ex = block_scan_dpp<NT>(n_gt | (n_eq << 16), S.wsum2, &tot);
  const int eq_before = ex >> 16;
  int pos = (ex & 0xffff) + min(eq_before, krem), r = eq_before;
  // When it fits in the histogram's space (no longer read), the selection is
  // placed in LDS first and written out in coalesced runs: a few full-width
  // stores per wave instead of one partial store per key slot, which matters
  // when the memory queues are busy.  Block ids are looked up for the
  // selected pages only.
  const bool staged = top_k <= kBins;
  int* lsel = hist;
#pragma unroll
  for (int x = 0; x < RM; ++x) {
    if (x < nv) {
      const uint32_t km = key[x] & mask;
      const bool eq = km == prefix;
      if (km > prefix || (eq && r < krem)) {
        if (staged) {
          lsel[pos] = i0 + x;
        } else {
          out[pos] = i0 + x;
          if constexpr (RES) store_coherent(rs.desc + pos, page_desc(resolve_blk(rs, i0 + x), i0 + x, rs));
        }
        ++pos;
      }
      r += eq;
    }
  }
  if (staged) {
    __syncthreads();
    for (int i = tid; i < top_k; i += NT) {
      const int p = lsel[i];
      out[i] = p;
      if constexpr (RES) store_coherent(rs.desc + i, page_desc(resolve_blk(rs, p), p, rs));
    }
  }
}

// One workgroup per (sequence, KV head, chunk of `chunk` logical pages).  The
// chunk's block ids are staged in LDS, then each wave streams its rows (PPR
// pages each) in groups of kGroup rows through a two-group register ring: a
// group's loads are issued before the previous group is reduced.  Scores are
// published with device-scope stores; the last workgroup of the unit to
// finish (per-unit arrival counter) runs the top-k.
//
// With ap.k_new set, the launch also appends one decode token per sequence
// (the new token is a candidate, as after a separate append).  In the
// workgroup whose chunk holds the token's page, the lanes that stream that
// page's summary fold the token's key into the summary they loaded and score
// the page from the result, so the page costs no extra load or barrier; the
// new summary, the token's K and V and its position are written after the
// stream (no store sits between the stream's loads).  The sequence length is raised by
// the last unit of the sequence to finish (per-sequence arrival counter),
// after every workgroup of the sequence has read the old length.
// Fused decode step only (FUSED): the appended token's K and V are written
// through to the point of coherence, and the top-k workgroup looks up the
// block ids of the selected pages, writes the epoch-tagged resolved
// descriptors and then raises the unit's epoch.
struct SelFused {
  uint64_t* desc = nullptr;   // [units][top_k] epoch-tagged resolved descriptors
  uint32_t* epoch = nullptr;  // [units] the unit's epoch: one more per call, raised by its top-k
};

// GM: 0 sums the group's bounds; 1 takes their maximum for fp32 data; 2 takes
// it for bf16 data, with the weights packed in pairs for v_dot2_f32_bf16
// (fp32 weights of 16 heads would take 16 * 8 registers per lane).
template <typename T, int D, int RM, int GM, bool FUSED, int NT = kScoreThreads>
__device__ __forceinline__ void select_block(
    const KVDev& kv, const T* __restrict__ q, const T* __restrict__ meta, float* __restrict__ scores, int chunk,
    int n_chunks, int top_k, int n_sink, int n_recent, int32_t* __restrict__ sel, int* __restrict__ counters,
    const AppendIn& ap, const SelFused& fz, int vblk, uint32_t* epoch_out = nullptr) {
  using S = ScoreShape<T, D>;
  constexpr int E = S::E, LPP = S::LPP, PPR = S::PPR;
  constexpr int NW = NT / 64;                // waves
  constexpr int MC = 4 * NT;                 // most pages of one chunk
  constexpr int QP = (16 * 128 + NT - 1) / NT;   // query elements staged per thread
  // scoring: sblk, sc, qst; top-k (after scoring, same memory): hist, cand, sh
  extern __shared__ __align__(16) uint32_t lds[];
  int* sblk = reinterpret_cast<int*>(lds);                          // [MC] block ids
  float* sc = reinterpret_cast<float*>(lds + MC);             // [MC] the chunk's scores
  float* qst = reinterpret_cast<float*>(lds + 2 * MC);        // [G][D] the group's queries
  __shared__ int wsum[2][NW + 1];
  __shared__ int s_last;
  constexpr int NC = D / E;                 // 16-byte chunks per summary row
  // fused append: new K and V chunks, the page's old summary, its new summary
  __shared__ u32x4 s_kv[2][NC];              // fused append: the new token's K and V chunks

  // every pointer the prologue's loads need, in scalar registers from the
  // first batch of argument loads (otherwise later argument loads, sunk
  // towards their uses, each cost a round trip before the prologue's loads)
  asm volatile("" ::"s"(q), "s"(meta), "s"(kv.seq_lens), "s"(kv.block_table), "s"(ap.k_new), "s"(ap.v_new),
               "s"(scores), "s"(sel), "s"(counters), "s"(top_k), "s"(n_sink), "s"(n_recent));
  const int u = vblk / n_chunks, c = vblk % n_chunks;
  const int b = u / kv.Hkv, h = u % kv.Hkv;
  const int P = kv.P, G = kv.G;
  const int p_lo = c * chunk, p_hi = min(p_lo + chunk, kv.max_pages);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  float* srow = scores + (size_t)u * kv.max_pages;
  const int32_t* bt_row = kv.block_table + (size_t)b * kv.max_pages;

  // The length, the chunk's block ids (the block-table row is max_pages
  // long, so it is read before the length is known and checked after) and
  // the group's queries: every load is issued before any is used.
  // One round trip for the prologue: the length, the chunk's block ids, the
  // new token and the group's queries are all issued, then waited for once.
  // Indices are clamped rather than guarded (a load in its own branch would
  // be waited for there), and the length is first used after the wait (a
  // readfirstlane next to its load would wait for it alone).
  int len_raw = kv.seq_lens[b];
  // fused step: the unit's epoch before this call (read before this
  // workgroup counts in, so before the unit's top-k can raise it)
  uint32_t ep_old = 0;
  if constexpr (FUSED) ep_old = __hip_atomic_load(fz.epoch + u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  int bt[MC / NT];
#pragma unroll
  for (int r = 0; r < MC / NT; ++r)
    bt[r] = bt_row[min(p_lo + tid + r * NT, p_hi - 1)];
  // the new token's K (lanes j < NC of each 2 * NC) and V chunks of this
  // head; loaded by every lane from a valid address (the queries' row
  // without an append), kept by lanes tid < 2 * NC
  const bool app = ap.k_new != nullptr;
  static_assert(QP * NT >= 16 * 128, "one pass stages the queries of up to 16 heads of 128 dims");
  const T* qrow = q + ((size_t)b * kv.Hq + h * G) * D;
  const int jn = tid % (2 * NC);
  const T* kv_src = app ? static_cast<const T*>(jn < NC ? ap.k_new : ap.v_new) + ((size_t)b * kv.Hkv + h) * D +
                              (jn % NC) * E
                        : qrow;
  const u32x4 kv_new = *reinterpret_cast<const u32x4*>(kv_src);
  T qv[QP];
#pragma unroll
  for (int e = 0; e < QP; ++e) qv[e] = qrow[min(e * NT + tid, G * D - 1)];
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("" : "+v"(len_raw));
  if constexpr (FUSED) {
    asm volatile("" : "+v"(ep_old));
    if (epoch_out != nullptr && tid == 0) *epoch_out = ep_old + 1u;
  }
#pragma unroll
  for (int e = 0; e < QP; ++e) {
    const int i = e * NT + tid;
    if (i < G * D) qst[i] = to_f32(qv[e]);
  }
  const int L0 = clamp_len(len_raw, kv.max_pages * P);
  const int nt = (app && L0 < kv.max_pages * P) ? 1 : 0;   // appended tokens (0 when full)
  const int L = L0 + nt;
  const int n_pages = (L + P - 1) / P;
  const int pg_new = L0 / P;
  const bool own = nt > 0 && pg_new >= p_lo && pg_new < p_hi;
  // where this workgroup's stream meets the new token's page
  const int own_row = (pg_new - p_lo) / PPR;
  const int own_wave = own_row % NW, own_k = own_row / NW, own_sub = (pg_new - p_lo) % PPR;
#pragma unroll
  for (int r = 0; r < MC / NT; ++r) {
    const int i = tid + r * NT, p = p_lo + i;
    if (p < p_hi) sblk[i] = (p < n_pages && bt[r] >= 0 && bt[r] < kv.num_blocks) ? bt[r] : -1;
  }
  if (app && tid < 2 * NC) s_kv[tid / NC][tid % NC] = kv_new;
  __syncthreads();
  const int j = lane % LPP;                 // 16-byte chunk of the summary read by this lane
  const int row = j / (LPP / 2);            // 0: minimum row, 1: maximum row
  const int dim0 = (j % (LPP / 2)) * E;
  const int sub = lane / LPP;
  // this lane's weights for channels dim0 .. dim0 + E - 1: max(q, 0) on the
  // maximum row, min(q, 0) on the minimum row; summed over the group (sum
  // aggregation, one dot product per page) or kept per head (max
  // aggregation: G dot products per page, then the largest).  A weight of
  // bf16 data is a bf16 value (the positive or negative part of a bf16 query
  // element), so the packed form (GM == 2) is exact.
  constexpr bool GMAX = GM != 0;
  constexpr bool PK = GM == 2;
  static_assert(GM == 0 || (GM == 2) == (sizeof(T) == 2), "the maximum: packed weights for bf16 data");
  constexpr int WH = GM == 0 ? 1 : kGroupMaxHeads;
  // bf16, 32 lanes per page: the reduce-scatter form (scatter_max32) over
  // GP >= G slots, lane l computing head s ^ hmask in slot s; slots whose
  // head is G or more repeat head 0, which leaves the maximum unchanged
  constexpr bool BFLY = PK && LPP == 32;
  const int GP = G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : G <= 8 ? 8 : 16;
  const int hmask = BFLY ? max_slot_mask(lane, GP) : 0;
  float w[PK ? 1 : WH][E];
  uint32_t w2[PK ? WH : 1][E / 2];
#pragma unroll
  for (int a = 0; a < (PK ? 1 : WH); ++a)
#pragma unroll
    for (int e = 0; e < E; ++e) w[a][e] = 0.f;
#pragma unroll
  for (int a = 0; a < (PK ? WH : 1); ++a)
#pragma unroll
    for (int e = 0; e < E / 2; ++e) w2[a][e] = 0u;
  if constexpr (BFLY) {
#pragma unroll
    for (int sl = 0; sl < WH; ++sl) {
      int hd = sl ^ hmask;
      hd = hd < G ? hd : 0;
#pragma unroll
      for (int e = 0; e < E; e += 4) {
        const float4 x = *reinterpret_cast<const float4*>(qst + hd * D + dim0 + e);
        const float v4[4] = {x.x, x.y, x.z, x.w};
        float t[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) t[f] = row ? fmaxf(v4[f], 0.f) : fminf(v4[f], 0.f);
        w2[sl][e / 2] = (__float_as_uint(t[0]) >> 16) | (__float_as_uint(t[1]) & 0xffff0000u);
        w2[sl][e / 2 + 1] = (__float_as_uint(t[2]) >> 16) | (__float_as_uint(t[3]) & 0xffff0000u);
      }
    }
  }
  for (int a = 0; a < (BFLY ? 0 : G); ++a) {
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      const float4 x = *reinterpret_cast<const float4*>(qst + a * D + dim0 + e);
      const float v4[4] = {x.x, x.y, x.z, x.w};
      float t[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) t[f] = row ? fmaxf(v4[f], 0.f) : fminf(v4[f], 0.f);
      if constexpr (PK) {
        const uint32_t lo = (__float_as_uint(t[0]) >> 16) | (__float_as_uint(t[1]) & 0xffff0000u);
        const uint32_t hi = (__float_as_uint(t[2]) >> 16) | (__float_as_uint(t[3]) & 0xffff0000u);
#pragma unroll
        for (int hh = 0; hh < WH; ++hh)
          if (hh == a) { w2[hh][e / 2] = lo; w2[hh][e / 2 + 1] = hi; }
      } else {
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          if constexpr (GMAX) {
#pragma unroll
            for (int hh = 0; hh < WH; ++hh)
              if (hh == a) w[hh][e + f] = t[f];
          } else {
            w[0][e + f] += t[f];
          }
        }
      }
    }
  }

  const int n_rows = (p_hi - p_lo + PPR - 1) / PPR;
  const int my_rows = wave < n_rows ? (n_rows - wave + NW - 1) / NW : 0;
  const int n_groups = __builtin_amdgcn_readfirstlane((my_rows + kGroup - 1) / kGroup);
  // page of row slot r of group gi (rows of this wave: wave, wave + 4, ...)
  auto page_of = [&](int gi, int r) { return p_lo + (wave + NW * (gi * kGroup + r)) * PPR + sub; };
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
  // all rows' lane partials first, then the group sums side by side, so the
  // rows' reduction chains overlap
  u32x4 fold_keep = {0u, 0u, 0u, 0u};
  auto reduce = [&](const u32x4 (&m)[kGroup], int gi) {
    float part[kGroup];
    float xs[PK ? 1 : kGroup][E];
    u32x4 xw[PK ? kGroup : 1];
#pragma unroll
    for (int r = 0; r < kGroup; ++r) {
      union U { u32x4 u; T e[E]; };
      U mm;
      mm.u = m[r];
      if (own && wave == own_wave && gi * kGroup + r == own_k && sub == own_sub) {
        // the appended token's page: this lane's chunk of the loaded (old)
        // summary takes the token's key (minimum row: lanes j < NC), or is
        // the key alone when the token opens the page; kept for the write
        // after the stream, and scored below like any other page
        U kk;
        kk.u = s_kv[0][j % NC];
        const bool fold = (L0 % P) != 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float x = to_f32(kk.e[e]), o = to_f32(mm.e[e]);
          const float n = !fold ? x : (j < NC ? (x < o ? x : o) : (x > o ? x : o));
          mm.e[e] = from_f32<T>(n);
        }
        fold_keep = mm.u;
      }
      if constexpr (PK) {
        xw[r] = mm.u;
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) xs[r][e] = to_f32(mm.e[e]);
      }
    }
    if constexpr (BFLY) {
      static_assert(E == 8, "32 lanes per page: 8 bf16 values a lane");
      typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int r = 0; r < kGroup; ++r) {
        if (GP == 1) {
          float pr = 0.f;
#pragma unroll
          for (int i = 0; i < E / 2; ++i)
            pr = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w2[0][i]),
                                                 __builtin_bit_cast(bf16x2_t, (uint32_t)xw[r][i]), pr, false);
          part[r] = group_sum<LPP>(pr);
        } else if (GP == 2) {
          part[r] = row_max32<2>(w2, xw[r]);
        } else if (GP == 4) {
          part[r] = row_max32<4>(w2, xw[r]);
        } else if (GP == 8) {
          part[r] = row_max32<8>(w2, xw[r]);
        } else {
          part[r] = row_max32<16>(w2, xw[r]);
        }
      }
    } else if constexpr (PK) {
      typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int r = 0; r < kGroup; ++r) part[r] = -INFINITY;
#pragma unroll
      for (int a = 0; a < WH; ++a) {
        if (a >= G) break;
        float pa[kGroup];
#pragma unroll
        for (int r = 0; r < kGroup; ++r) {
          float pr = 0.f;
#pragma unroll
          for (int i = 0; i < E / 2; ++i)
            pr = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w2[a][i]),
                                                 __builtin_bit_cast(bf16x2_t, (uint32_t)xw[r][i]), pr, false);
          pa[r] = pr;
        }
#pragma unroll
        for (int r = 0; r < kGroup; ++r) part[r] = fmaxf(part[r], group_sum<LPP>(pa[r]));
      }
    } else if constexpr (GMAX) {
#pragma unroll
      for (int r = 0; r < kGroup; ++r) part[r] = -INFINITY;
#pragma unroll
      for (int a = 0; a < WH; ++a) {
        if (a >= G) break;
        float pa[kGroup];
#pragma unroll
        for (int r = 0; r < kGroup; ++r) {
          float pr = 0.f;
#pragma unroll
          for (int e = 0; e < E; ++e) pr = fmaf(w[a][e], xs[r][e], pr);
          pa[r] = pr;
        }
#pragma unroll
        for (int r = 0; r < kGroup; ++r) part[r] = fmaxf(part[r], group_sum<LPP>(pa[r]));
      }
    } else {
#pragma unroll
      for (int r = 0; r < kGroup; ++r) {
        float pr = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) pr = fmaf(w[0][e], xs[r][e], pr);
        part[r] = pr;
      }
#pragma unroll
      for (int r = 0; r < kGroup; ++r) part[r] = group_sum<LPP>(part[r]);
    }
#pragma unroll
    for (int r = 0; r < kGroup; ++r) {
      const int p = page_of(gi, r);
      if (j == 0 && p < p_hi) sc[p - p_lo] = sblk[p - p_lo] >= 0 ? part[r] : -INFINITY;
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
  if (own) {
    // the appended token's K and V, its page's new summary and its position
    const int blk = sblk[pg_new - p_lo];
    if (wave == own_wave && sub == own_sub && blk >= 0)
      *reinterpret_cast<u32x4*>(const_cast<T*>(meta) + ((size_t)blk * kv.Hkv + h) * 2 * D + j * E) = fold_keep;
    const int off = L0 % P;
    if (tid < NC && blk >= 0) {
      union { u32x4 u; T e[E]; } vv;
      vv.u = s_kv[1][tid];
      const size_t base = page_base(blk, h, kv.Hkv, P, D);
      T* kpool = reinterpret_cast<T*>(kv.k_pool);
      T* vpool = reinterpret_cast<T*>(kv.v_pool);
      if constexpr (FUSED) {
        // read by attention workgroups of this launch on any XCD: written
        // through to the point of coherence (K as dwords; V by read-modify-
        // write of the dword holding this token and its page neighbour, whose
        // value this sequence's appends alone write)
        uint32_t* kd = reinterpret_cast<uint32_t*>(kpool + base + (size_t)(tid * P + off) * E);
        const u32x4 kk = s_kv[0][tid];
        __hip_atomic_store(kd + 0, kk.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(kd + 1, kk.y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(kd + 2, kk.z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(kd + 3, kk.w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if constexpr (sizeof(T) == 4) {
#pragma unroll
          for (int e = 0; e < E; ++e)
            __hip_atomic_store(reinterpret_cast<uint32_t*>(vpool + base + v_off(off, tid * E + e, P)),
                               __float_as_uint(to_f32(vv.e[e])), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          uint32_t old[E];
#pragma unroll
          for (int e = 0; e < E; ++e)
            old[e] = __hip_atomic_load(reinterpret_cast<const uint32_t*>(vpool + base + v_off(off & ~1, tid * E + e, P)),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const uint32_t mine = (uint32_t)__builtin_bit_cast(uint16_t, vv.e[e]);
            const uint32_t nw = (off & 1) ? ((old[e] & 0xffffu) | (mine << 16)) : ((old[e] & 0xffff0000u) | mine);
            __hip_atomic_store(reinterpret_cast<uint32_t*>(vpool + base + v_off(off & ~1, tid * E + e, P)), nw,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      } else {
        *reinterpret_cast<u32x4*>(kpool + base + (size_t)(tid * P + off) * E) = s_kv[0][tid];
#pragma unroll
        for (int e = 0; e < E; ++e) vpool[base + v_off(off, tid * E + e, P)] = vv.e[e];
      }
    }
    if (tid == 0 && ap.slot_pos != nullptr)
      ap.slot_pos[((size_t)b * kv.Hkv + h) * ap.slot_cap + L0] = ap.pos_new ? ap.pos_new[b] : L0;
  }
  // publish the chunk's scores as one coalesced run of device-scope stores,
  // complete at the point of coherence before the workgroup counts itself in
  __syncthreads();
  for (int i = tid; i < p_hi - p_lo; i += NT)
    __hip_atomic_store(srow + p_lo + i, sc[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&counters[u], 1) == n_chunks - 1;
  __syncthreads();
  if (!s_last) return;
  __syncthreads();                          // the scoring LDS is reused
  TopkLds tl;
  tl.hist = reinterpret_cast<int*>(lds);
  tl.cand = lds + kBins;
  tl.sh = reinterpret_cast<int*>(lds + kBins + kCand);
  tl.wsum = wsum[0];
  tl.wsum2 = wsum[1];
  Resolve rs;
  if constexpr (FUSED) {
    rs.blk_row = bt_row;
    rs.num_blocks = kv.num_blocks;
    rs.desc = fz.desc + (size_t)u * top_k;
    rs.L = L;
    rs.P = P;
    rs.epoch = ep_old + 1u;
  }
  if constexpr (RM > 0) {
    topk_unit<RM, FUSED, NT>(srow, n_pages, top_k, n_sink, n_recent, sel + (size_t)u * top_k, tl, rs);
  } else {
    // scoring only (RM == 0): sel is the per-sequence page count for a top-k
    // that runs after this launch; every unit of the sequence writes the same
    // count, the length every workgroup read in its prologue
    if (tid == 0) sel[b] = n_pages;
  }
  // fused step: the unit's epoch for the next call (every workgroup of the
  // unit read the old one in its prologue, before it counted in)
  if constexpr (FUSED) {
    if (tid == 0) __hip_atomic_store(fz.epoch + u, ep_old + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (app && tid == 0) {
    // the last unit of the sequence to finish raises its length: every
    // workgroup of the sequence has read the old one by now (counted after
    // the top-k, so the top-k does not wait for this round trip)
    int* seq_counter = counters + kv.B * kv.Hkv + b;
    if (atomicAdd(seq_counter, 1) == kv.Hkv - 1) {
      kv.seq_lens[b] = L;
      __hip_atomic_store(seq_counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // the counter is left zero for the next call; issued last, so that no
  // barrier of the top-k waits for this store
  if (tid == 0) __hip_atomic_store(&counters[u], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Chunking of the scoring: about kScoreWgTarget workgroups in all, chunks a
// multiple of one row per wave and at most 4 pages per thread.
template <typename T, int D, int NT = kScoreThreads>
inline void select_chunks(const KVDev& kv, int* chunk_out, int* n_chunks_out, int target = kScoreWgTarget) {
  using S = ScoreShape<T, D>;
  constexpr int kMaxChunk = 4 * NT;
  const int units = kv.B * kv.Hkv;
  const int quantum = S::PPR * (NT / 64);
  int n_chunks = (target + units - 1) / units;
  int chunk = (kv.max_pages + n_chunks - 1) / n_chunks;
  chunk = (chunk + quantum - 1) / quantum * quantum;
  if (chunk > kMaxChunk) chunk = kMaxChunk;
  n_chunks = (kv.max_pages + chunk - 1) / chunk;
  *chunk_out = chunk;
  *n_chunks_out = n_chunks;
}

// Dynamic LDS of the select kernel: the larger of the scoring layout and the
// top-k layout, in 4-byte words.
inline size_t select_lds_bytes(int G, int D, int NT = kScoreThreads) {
  const size_t score = (size_t)(2 * 4 * NT + G * D) * 4;
  const size_t topk = (size_t)(kBins + kCand + 8 + 2 * (NT / 64)) * 4;
  return score > topk ? score : topk;
}
}  // namespace seldev
}  // namespace spk
