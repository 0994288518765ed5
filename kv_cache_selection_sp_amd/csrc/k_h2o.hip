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
// finds the (budget - window)-th largest, ties going to lower slots.  Every
// kept slot's destination is its rank among kept slots, which is never above
// its source, so the slots move down in place.
//
//   * Fast path (slot capacity <= kEvFastMax): 256 threads; the candidate
//     keys, the block-table row and the destination -> source map live in
//     LDS.  Radix select over 11-bit digits from the highest bit where the
//     keys differ, exact by counting once the boundary bin is small.  Two
//     block scans give every kept slot its destination and locate the first
//     hole; only destinations from the first hole on are written, in rounds
//     of kEvRound destination slots taken in ascending order.  A round reads
//     all its sources before it writes any destination; every later round's
//     sources lie above this round's destinations, so no source is
//     overwritten before it is read.
//   * Large path (larger capacities): a list kernel (radix select over the
//     scores in global memory, then the ascending list of kept slots in a
//     workspace) and two move kernels, one for the entries whose sources are
//     also destinations (in ascending rounds) and one, across many
//     workgroups, for the rest.
#include "lds_layout.h"
#include "sp_internal.h"

namespace spk {
namespace {

constexpr int kAccThreads = 256;
constexpr int kAccBlocks = 4;         // slot blocks per unit (each strides over the slots)
constexpr int kMaxGroup = 16;         // query heads per KV head (the API's limit)

// One workgroup per (slot block, KV head, sequence); the workgroups of a unit
// stride over its occupied slots.  A slot's G logits are loaded together
// (the group is at most kMaxGroup heads), then exponentiated and summed.
__global__ void __launch_bounds__(kAccThreads)
h2o_accumulate_kernel(KVDev kv, const float* __restrict__ logits, const float* __restrict__ lse,
                      int logit_cap, int n_new, float* __restrict__ scores, int slot_cap) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int G = kv.G;
  const int L = clamp_len(kv.seq_lens[b], kv.max_pages * kv.P);
  const size_t ra0 = (size_t)b * kv.Hq + (size_t)h * G;
  float lz[kMaxGroup];
#pragma unroll
  for (int a = 0; a < kMaxGroup; ++a) lz[a] = a < G ? lse[ra0 + a] : 0.f;
  float* srow = scores + ((size_t)b * kv.Hkv + h) * slot_cap;
  for (int j = blockIdx.x * kAccThreads + threadIdx.x; j < L; j += gridDim.x * kAccThreads) {
    float z[kMaxGroup];
#pragma unroll
    for (int a = 0; a < kMaxGroup; ++a) z[a] = a < G ? logits[(ra0 + a) * logit_cap + j] : 0.f;
    const float old = srow[j];
    float s = (j >= L - n_new) ? 0.f : old;
#pragma unroll
    for (int a = 0; a < kMaxGroup; ++a)
      if (a < G) s += expf(z[a] - lz[a]);
    srow[j] = s;
  }
}

// ------------------------------------------------------------ fast eviction
constexpr int kEvThreads = 256;
constexpr int kEvWaves = kEvThreads / 64;
constexpr int kEvFastMax = 8192;      // slot capacity of the fast path (LDS: keys, 16-bit map)
constexpr int kEvRound = 64;          // destination slots moved per round (a power of two)
constexpr int kEvDigit = 11;
using evlds::kEvBins;
using evlds::kEvCand;
static_assert(kEvBins == 1 << kEvDigit, "radix bins of the threshold search");
constexpr int kWinPre = 128;          // recent windows up to this size are read ahead
constexpr int kWinPages = 16;         // block ids held in registers for the read ahead (pages
                                      // from the one before the window's first on)
constexpr int kDevScopeNone = 0;

// LDS layout of the fast path (ev_layout) in lds_layout.h.
using evlds::EvLayout;
using evlds::ev_layout;

// V of bf16 destinations [a, b) from sources [a + k, b + k), k >= 1, moved
// as 16-byte chunks (8 tokens of one dim row of the dim-major page).  The
// 8 tokens of a destination chunk come from the two source chunks covering
// their shifted positions, joined by a byte-align of the shift k mod 8 (the
// same for every chunk).  Slots below a in the first destination chunk keep
// their values (that chunk is read, merged, written); slots at or above b
// may take any value (they are past the range; the caller writes or drops
// them).  One lane owns one dim row and walks its chunks in ascending order,
// in phases that read every source of the phase before writing: a phase's
// sources lie at or above its destinations and later phases read only above
// them, and no other lane touches the row, so no barrier (and no wait for
// stores to complete) is needed.
constexpr int kVPhase = 12;           // destination chunks per lane per phase

__device__ __forceinline__ uint4 shift_tokens(const uint4 lo, const uint4 hi, int r) {
  // r is the same in every lane: the dword offset is a uniform branch
  uint32_t o[5];
  switch (r >> 1) {
    case 0: o[0] = lo.x; o[1] = lo.y; o[2] = lo.z; o[3] = lo.w; o[4] = hi.x; break;
    case 1: o[0] = lo.y; o[1] = lo.z; o[2] = lo.w; o[3] = hi.x; o[4] = hi.y; break;
    case 2: o[0] = lo.z; o[1] = lo.w; o[2] = hi.x; o[3] = hi.y; o[4] = hi.z; break;
    default: o[0] = lo.w; o[1] = hi.x; o[2] = hi.y; o[3] = hi.z; o[4] = hi.w; break;
  }
  if (r & 1)
    return make_uint4(__builtin_amdgcn_alignbyte(o[1], o[0], 2), __builtin_amdgcn_alignbyte(o[2], o[1], 2),
                      __builtin_amdgcn_alignbyte(o[3], o[2], 2), __builtin_amdgcn_alignbyte(o[4], o[3], 2));
  return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ void shift_move_v(bf16_t* __restrict__ vpool, const int* lbt, int mp, int nblk, int h, int Hkv,
                             int P, int D, int lp, int a, int b, int k) {
  const int d = threadIdx.x;                  // this lane's dim row
  if (a >= b || d >= D) return;
  const int lc = lp - 3;                      // log2(chunks per page row)
  const int r = k & 7, gk = k >> 3;           // shift: whole chunks and tokens
  // chunk g = tokens [8g, 8g + 8) of the row, on page g >> lc
  auto at = [&](int g) -> uint4* {
    const int page = g >> lc;
    return reinterpret_cast<uint4*>(vpool + page_base(lbt[page], h, Hkv, P, D) + (size_t)(d << lp) +
                                    ((g & ((1 << lc) - 1)) << 3));
  };
  auto ok = [&](int g) {
    const int page = g >> lc;
    return page < mp && lbt[page] >= 0 && lbt[page] < nblk;
  };
  const int g_first = a >> 3, g_last = (b - 1) >> 3;
  for (int g0 = g_first; g0 <= g_last; g0 += kVPhase) {
    const int n = min(kVPhase, g_last + 1 - g0);
    uint4 src[kVPhase + 1];
#pragma unroll
    for (int i = 0; i <= kVPhase; ++i) {
      const int gs = g0 + gk + i;
      src[i] = (i <= n && (i < n || r != 0) && ok(gs)) ? *at(gs) : make_uint4(0u, 0u, 0u, 0u);
    }
    uint4 old = make_uint4(0u, 0u, 0u, 0u);
    const bool merge = g0 == g_first && (a & 7) != 0;
    if (merge && ok(g0)) old = *at(g0);
#pragma unroll
    for (int i = 0; i < kVPhase; ++i) {
      if (i >= n || !ok(g0 + i)) continue;
      uint4 v = shift_tokens(src[i], src[i + 1], r);
      if (i == 0 && merge) {
        // keep the slots below a: tokens [0, a & 7) from the old chunk
        const int keep = a & 7;
        uint32_t vv[4] = {v.x, v.y, v.z, v.w};
        const uint32_t ov[4] = {old.x, old.y, old.z, old.w};
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int t0 = 2 * x;
          if (t0 + 1 < keep) vv[x] = ov[x];
          else if (t0 < keep) vv[x] = (vv[x] & 0xffff0000u) | (ov[x] & 0x0000ffffu);
        }
        v = make_uint4(vv[0], vv[1], vv[2], vv[3]);
      }
      *at(g0 + i) = v;
    }
  }
}

template <typename T>
__global__ void __launch_bounds__(kEvThreads)
h2o_evict_fast_kernel(KVDev kv, float* __restrict__ scores, int32_t* __restrict__ slot_pos, int slot_cap,
                      int budget, int window, int* __restrict__ seq_counters) {
  constexpr int E = Chunk<T>::E;
  extern __shared__ __align__(16) uint32_t lds[];
  __shared__ int wsum[2][kEvWaves + 1];
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int P = kv.P, D = kv.D, Hkv = kv.Hkv, mp = kv.max_pages;
  const int cap = mp * P;
  const int L = clamp_len(kv.seq_lens[b], cap);
  if (L <= budget) return;
  const int nc = L - window;             // candidate slots [0, nc)
  const int keep_c = budget - window;    // candidates kept, 0 <= keep_c < nc
  float* srow = scores + ((size_t)b * Hkv + h) * slot_cap;
  int32_t* prow = slot_pos ? slot_pos + ((size_t)b * Hkv + h) * slot_cap : nullptr;
  const EvLayout lay = ev_layout(cap, mp);
  uint32_t* keys = lds + lay.keys;
  uint16_t* srcmap = reinterpret_cast<uint16_t*>(lds + lay.srcmap);   // destination -> source slot
  int* lbt = reinterpret_cast<int*>(lds + lay.lbt);
  int* hist = reinterpret_cast<int*>(lds + lay.hist);
  uint32_t* cand = lds + lay.cand;
  int* sh = reinterpret_cast<int*>(lds + lay.sh);

  // ---- candidate scores and the block-table row into LDS (direct loads)
  const int32_t* bt_row = kv.block_table + (size_t)b * mp;
  // block ids of the pages around the recent window (kWinPages from wp0),
  // one per lane of every wave, loaded with the staging below: the window's
  // reads ahead take them from registers instead of one LDS lookup each
  const int lp0 = __builtin_ctz((unsigned)P);
  const int wp0 = max(0, (nc >> lp0) - 1);
  const int blk_w = bt_row[min(wp0 + lane, mp - 1)];
  for (int i = wid * 64; i < nc; i += kEvThreads)
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(srow + min(i + lane, nc - 1)),
                                     (__attribute__((address_space(3))) void*)(keys + i), 4, 0,
                                     kDevScopeNone);
  for (int i = wid * 64; i < mp; i += kEvThreads)
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(bt_row + min(i + lane, mp - 1)),
                                     (__attribute__((address_space(3))) void*)(lbt + i), 4, 0,
                                     kDevScopeNone);
  for (int i = tid; i < kEvBins; i += kEvThreads) hist[i] = 0;
  if (tid == 0) { sh[3] = 0; sh[6] = 0x7fffffff; sh[7] = -1; }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Moves use tasks (destination m = tid % kEvRound, K chunk or V dimension
  // q0 + k * (kEvThreads / kEvRound), q0 = tid / kEvRound): neighbouring
  // lanes move neighbouring slots.  P is a power of two.
  T* kpool = reinterpret_cast<T*>(kv.k_pool);
  T* vpool = reinterpret_cast<T*>(kv.v_pool);
  const int nblk = kv.num_blocks;
  const int lp = __builtin_ctz((unsigned)P);
  const int nch = D / E;
  constexpr int kRoundShift = 6;                      // log2(kEvRound)
  constexpr int kStride = kEvThreads >> kRoundShift;  // chunks / dimensions between a lane's tasks
  constexpr int kMaxK = kEvRound * (128 / E) / kEvThreads;   // 16-byte K chunks per thread (D <= 128)
  constexpr int kMaxV = kEvRound * 128 / kEvThreads;         // V elements per thread (D <= 128)
  const int m_lane = tid & (kEvRound - 1);
  const int q0 = tid >> kRoundShift;
  auto kaddr = [&](int slot, int c, int blk) {
    return kpool + page_base(blk, h, Hkv, P, D) + (size_t)((c << lp) + (slot & (P - 1))) * E;
  };
  auto vaddr = [&](int slot, int d, int blk) {
    return vpool + page_base(blk, h, Hkv, P, D) + (size_t)(d << lp) + (slot & (P - 1));
  };
  const int n_ev_all = L - budget;        // slots evicted, >= 1
  // The recent window always moves, by n_ev slots, to [keep_c, budget).  With
  // 2-byte elements and a window of at most kWinPre slots its K, scores and
  // positions are read now, while the threshold is found, and written after
  // the candidates that move (those are read before any write lands on their
  // slots); its V then moves as a shift of 16-byte chunks.
  constexpr bool kPreOk = sizeof(T) == 2;
  const bool win_pre = kPreOk && window > 0 && window <= kWinPre;
  uint4 kw[kWinPre / kEvRound][kMaxK];
  float sw[kWinPre / kEvRound];
  int32_t pw[kWinPre / kEvRound];
  if (win_pre) {
#pragma unroll
    for (int r = 0; r < kWinPre / kEvRound; ++r) {
      const int m = r * kEvRound + m_lane;
      const int src = nc + (m < window ? m : 0);
      const int bs = __shfl(blk_w, min((src >> lp) - wp0, kWinPages - 1), 64);
      const bool ok = m < window && bs >= 0 && bs < nblk;
#pragma unroll
      for (int k = 0; k < kMaxK; ++k) {
        const int c = q0 + k * kStride;
        kw[r][k] = (ok && c < nch) ? *reinterpret_cast<const uint4*>(kaddr(src, c, bs)) : make_uint4(0u, 0u, 0u, 0u);
      }
      sw[r] = m < window && q0 == 0 ? srow[src] : 0.f;
      pw[r] = m < window && q0 == 0 && prow ? prow[src] : 0;
    }
  }
  // and its V source chunks: lane d < D holds, for its dim row, the chunks
  // g0 + n_ev / 8 + i (g0 = keep_c / 8) that the destination chunks
  // g0 .. (budget - 1) / 8 draw from (chunk = 8 tokens = 16 bytes)
  constexpr int kWinChunks = kWinPre / 8 + 3;
  uint4 vwin[kWinChunks];
  const int wg0 = keep_c >> 3, wgl = (budget - 1) >> 3;
  if (win_pre && tid < D) {
    const int lc = lp - 3;
    const int gs0 = wg0 + (n_ev_all >> 3);
#pragma unroll
    for (int i = 0; i < kWinChunks; ++i) {
      const int gs = gs0 + i;
      const int page = gs >> lc;
      const int bw = __builtin_amdgcn_readlane(blk_w, min(max(page - wp0, 0), kWinPages - 1));
      const bool ok = i <= wgl - wg0 + 1 && page < mp && bw >= 0 && bw < nblk;
      vwin[i] = ok ? *reinterpret_cast<const uint4*>(vpool + page_base(bw, h, Hkv, P, D) +
                                                    (size_t)(tid << lp) + ((gs & ((1 << lc) - 1)) << 3))
                   : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  // keys in place, 4 per thread per step, with their extremes
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  for (int i = tid * 4; i < nc; i += 4 * kEvThreads) {
    const uint4 v = *reinterpret_cast<const uint4*>(keys + i);
    const uint32_t kv4[4] = {float_key(__uint_as_float(v.x)), float_key(__uint_as_float(v.y)),
                             float_key(__uint_as_float(v.z)), float_key(__uint_as_float(v.w))};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (i + e < nc) { kmin = min(kmin, kv4[e]); kmax = max(kmax, kv4[e]); }
    *reinterpret_cast<uint4*>(keys + i) = uint4{kv4[0], kv4[1], kv4[2], kv4[3]};
  }
  wave_min_max(kmin, kmax);
  if (lane == 0) { sh[8 + 2 * wid] = (int)kmin; sh[8 + 2 * wid + 1] = (int)kmax; }
  __syncthreads();
  kmin = 0xffffffffu;
  kmax = 0u;
#pragma unroll
  for (int w = 0; w < kEvWaves; ++w) {
    kmin = min(kmin, (uint32_t)sh[8 + 2 * w]);
    kmax = max(kmax, (uint32_t)sh[8 + 2 * w + 1]);
  }

  const int n_ev = L - budget;            // slots evicted, >= 1
  int e0;                                  // first evicted slot; destinations [e0, budget) move
  if (n_ev == 1) {
    // one slot goes: the last candidate holding the smallest key (equal
    // keys keep the lower slots); every later slot moves down by one
    int last = -1;
    for (int i = tid * 4; i < nc; i += 4 * kEvThreads) {
      const uint4 v = *reinterpret_cast<const uint4*>(keys + i);
      const uint32_t k4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (i + e < nc && k4[e] == kmin) last = i + e;
    }
    if (last >= 0) atomicMax(&sh[7], last);
    __syncthreads();
    e0 = sh[7];
  } else {
  // ---- threshold: the keep_c-th largest candidate key.  Candidates with
  // (key & mask) > prefix are kept; of those with (key & mask) == prefix, the
  // krem with the lowest slots.  keep_c == 0 keeps none (no key reaches ~0).
  uint32_t prefix = 0xffffffffu, mask = 0xffffffffu;
  int krem = 0;
  if (keep_c > 0) {
    const int R = ((nc + kEvThreads - 1) / kEvThreads + 3) & ~3;
    const int i0 = tid * R;
    auto for_run = [&](auto&& f) {
      for (int x = 0; x < R; x += 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(keys + i0 + x);
        const uint32_t k4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (i0 + x + e < nc) f(k4[e]);
      }
    };
    const uint32_t diff = kmin ^ kmax;
    const uint32_t common = diff == 0u ? 0xffffffffu : ~(0xffffffffu >> __clz(diff));
    prefix = kmax & common;
    mask = common;
    int hb = diff == 0u ? -1 : 31 - __clz(diff);
    krem = keep_c;
    while (hb >= 0) {
      const int shift = hb >= kEvDigit - 1 ? hb - (kEvDigit - 1) : 0;
      const int nb = 1 << (hb - shift + 1);
      for_run([&](uint32_t k) {
        if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & (uint32_t)(nb - 1)], 1);
      });
      __syncthreads();
      // thread t owns bins (hi - bpt, hi], counted from the top (bpt <= 8)
      const int bpt = nb >= kEvThreads ? nb / kEvThreads : 1;
      const int hi = nb - 1 - tid * bpt;
      int hv[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) hv[x] = (x < bpt && hi - x >= 0) ? hist[hi - x] : 0;
      int c = 0;
#pragma unroll
      for (int x = 0; x < 8; ++x) c += hv[x];
      int total;
      int above = block_scan_dpp<kEvThreads>(c, wsum[0], &total);
      if (above < krem && krem <= above + c) {
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          if (x < bpt && krem > above && krem <= above + hv[x]) { sh[0] = hi - x; sh[1] = above; sh[2] = hv[x]; }
          above += hv[x];
        }
      }
      __syncthreads();
      prefix |= (uint32_t)sh[0] << shift;
      mask |= (uint32_t)(nb - 1) << shift;
      krem -= sh[1];
      hb = shift - 1;
      const int cb = sh[2];
      if (krem == cb || hb < 0) break;             // bin taken whole, or key resolved
      if (cb <= kEvCand) {
        for_run([&](uint32_t k) {
          if ((k & mask) == prefix) cand[atomicAdd(&sh[3], 1)] = k;
        });
        __syncthreads();
        if (wid == 0) {
          const int cbu = __builtin_amdgcn_readfirstlane(cb);
          const uint32_t v = lane < cbu ? cand[lane] : 0u;
          int g = 0, e = 0;
          for (int x = 0; x < cbu; ++x) {
            const uint32_t y = (uint32_t)__builtin_amdgcn_readlane((int)v, x);
            g += y > v;
            e += y >= v;
          }
          if (lane < cbu && g < krem && krem <= e) { sh[4] = (int)v; sh[5] = g; }
        }
        __syncthreads();
        prefix = (uint32_t)sh[4];
        mask = 0xffffffffu;
        krem -= sh[5];
        break;
      }
      for (int i = tid; i < nb; i += kEvThreads) hist[i] = 0;
      __syncthreads();
    }
  }

  // ---- kept flags over [0, L): thread t owns slots [t*R2, t*R2 + R2)
  const int R2 = (L + kEvThreads - 1) / kEvThreads;
  const int s0 = tid * R2, s1 = min(L, s0 + R2);
  int n_eq = 0;
  for (int s = s0; s < s1 && s < nc; ++s) n_eq += (keys[s] & mask) == prefix;
  int tot;
  const int eq_before = block_scan_dpp<kEvThreads>(n_eq, wsum[1], &tot);
  int n_keep = 0, r = eq_before, hole = 0x7fffffff;
  for (int s = s0; s < s1; ++s) {
    bool keep = true;
    if (s < nc) {
      const uint32_t km = keys[s] & mask;
      const bool eq = km == prefix;
      keep = km > prefix || (eq && r < krem);
      r += eq;
    }
    n_keep += keep;
    if (!keep && s < hole) hole = s;
  }
  const int kept_before = block_scan_dpp<kEvThreads>(n_keep, wsum[0], &tot);
  if (hole != 0x7fffffff) atomicMin(&sh[6], hole);
  // destination -> source for every kept slot that moves
  int dst = kept_before;
  r = eq_before;
  for (int s = s0; s < s1; ++s) {
    bool keep = true;
    if (s < nc) {
      const uint32_t km = keys[s] & mask;
      const bool eq = km == prefix;
      keep = km > prefix || (eq && r < krem);
      r += eq;
    }
    if (keep) {
      if (dst != s) srcmap[dst] = (uint16_t)s;
      ++dst;
    }
  }
  __syncthreads();
  e0 = sh[6];
  }

  // ---- moves: destinations [e0, j_end) in rounds of kEvRound, ascending.
  // With 2-byte elements and one evicted slot the range is a shift by one:
  // V goes as 16-byte chunks after the rounds (which then move K, scores and
  // positions only).
  const int j_end = win_pre ? keep_c : budget;
  const bool v_shift = kPreOk && n_ev == 1;
  for (int j0 = e0; j0 < j_end; j0 += kEvRound) {
    const int nm = min(kEvRound, j_end - j0);
    uint4 kreg[kMaxK];
    T vreg[kMaxV];
    float sreg = 0.f;
    int32_t preg = 0;
    const bool live = m_lane < nm;
    const int src = !live ? 0 : (n_ev == 1 ? j0 + m_lane + 1 : (int)srcmap[j0 + m_lane]);
    const int ds = j0 + m_lane;
    const int bs = live ? lbt[src >> lp] : -1;
    const int bd = live ? lbt[ds >> lp] : -1;
    const bool src_ok = bs >= 0 && bs < nblk, dst_ok = bd >= 0 && bd < nblk;
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
      const int c = q0 + k * kStride;
      kreg[k] = (src_ok && c < nch) ? *reinterpret_cast<const uint4*>(kaddr(src, c, bs))
                                    : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < kMaxV; ++k) {
      const int d = q0 + k * kStride;
      vreg[k] = (!v_shift && src_ok && d < D) ? *vaddr(src, d, bs) : T(0);
    }
    if (tid < nm) {
      sreg = srow[src];
      if (prow) preg = prow[src];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
      const int c = q0 + k * kStride;
      if (dst_ok && c < nch) *reinterpret_cast<uint4*>(kaddr(ds, c, bd)) = kreg[k];
    }
#pragma unroll
    for (int k = 0; k < kMaxV; ++k) {
      const int d = q0 + k * kStride;
      if (!v_shift && dst_ok && d < D) *vaddr(ds, d, bd) = vreg[k];
    }
    if (tid < nm) {
      srow[ds] = sreg;
      if (prow) prow[ds] = preg;
    }
    __syncthreads();
  }

  // ---- the preloaded window to [keep_c, budget)
  if (win_pre) {
#pragma unroll
    for (int r = 0; r < kWinPre / kEvRound; ++r) {
      const int m = r * kEvRound + m_lane;
      const int ds = keep_c + m;
      const int bd = m < window ? lbt[ds >> lp] : -1;
      if (bd < 0 || bd >= nblk) continue;
#pragma unroll
      for (int k = 0; k < kMaxK; ++k) {
        const int c = q0 + k * kStride;
        if (c < nch) *reinterpret_cast<uint4*>(kaddr(ds, c, bd)) = kw[r][k];
      }
      if (q0 == 0) {
        srow[ds] = sw[r];
        if (prow) prow[ds] = pw[r];
      }
    }
  }
  // ---- V by 16-byte chunks: with one evicted slot every kept slot from e0
  // on shifts by one (candidates and window alike: one pass); otherwise the
  // candidates moved element by element above and the window shifts by n_ev
  if constexpr (kPreOk) {
    bf16_t* vp = reinterpret_cast<bf16_t*>(kv.v_pool);
    if (!win_pre || (v_shift && e0 < keep_c)) {
      // candidates shift too (or no read-ahead): one pass over [e0, budget)
      if (v_shift) shift_move_v(vp, lbt, mp, nblk, h, Hkv, P, D, lp, e0, budget, 1);
    } else if (tid < D) {
      // the window from the chunks read ahead; the first chunk keeps its
      // slots below keep_c (final by now: the rounds above ended in a barrier)
      const int lc = lp - 3, r = n_ev & 7;
      const int keep = keep_c & 7;
      uint4 old = make_uint4(0u, 0u, 0u, 0u);
      const int p0 = wg0 >> lc;
      const bool ok0 = lbt[p0] >= 0 && lbt[p0] < nblk;
      uint4* c0p = reinterpret_cast<uint4*>(vp + page_base(ok0 ? lbt[p0] : 0, h, Hkv, P, D) + (size_t)(tid << lp) +
                                            ((wg0 & ((1 << lc) - 1)) << 3));
      if (keep != 0 && ok0) old = *c0p;
#pragma unroll
      for (int i = 0; i + 1 < kWinChunks; ++i) {
        const int g = wg0 + i;
        if (g > wgl) break;
        const int page = g >> lc;
        if (lbt[page] < 0 || lbt[page] >= nblk) continue;
        uint4 v = shift_tokens(vwin[i], vwin[i + 1], r);
        if (i == 0 && keep != 0) {
          uint32_t vv[4] = {v.x, v.y, v.z, v.w};
          const uint32_t ov[4] = {old.x, old.y, old.z, old.w};
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int t0 = 2 * x;
            if (t0 + 1 < keep) vv[x] = ov[x];
            else if (t0 < keep) vv[x] = (vv[x] & 0xffff0000u) | (ov[x] & 0x0000ffffu);
          }
          v = make_uint4(vv[0], vv[1], vv[2], vv[3]);
        }
        *reinterpret_cast<uint4*>(vp + page_base(lbt[page], h, Hkv, P, D) + (size_t)(tid << lp) +
                                  ((g & ((1 << lc) - 1)) << 3)) = v;
      }
    }
  }
  // With per-sequence counters, the last head of the sequence to finish sets
  // the length to the budget (every head's workgroup read the old length when
  // it started) and leaves its counter zero; without them a separate launch
  // clamps the lengths after this kernel.
  if (seq_counters != nullptr && tid == 0) {
    if (atomicAdd(&seq_counters[b], 1) == Hkv - 1) {
      kv.seq_lens[b] = budget;
      __hip_atomic_store(&seq_counters[b], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ------------------------------------------------------------ large eviction
// Capacities above kEvFastMax use a workspace that holds, per unit, a header
// (whether the unit evicts, the count n_low below, the radix-select state), a
// 2048-bin histogram, per-slice counts and the ascending list of the kept
// slots (entry i = the source of destination slot i).  Kernels, in order:
//   * init: header from the length, histogram cleared;
//   * three rounds of hist: slices of kSelSlice candidate scores, one
//     workgroup each, count the keys that match the current prefix into an
//     LDS histogram of the next digit (11, 11 and 10 bits), added into the
//     unit's histogram; the unit's last slice workgroup to count in then
//     picks the digit that holds the (budget - window)-th largest key, which
//     after the third round gives the exact threshold T and the number of
//     ties at T to keep (the lowest slots);
//   * count: per slice, kept slots above T (and window slots) and ties;
//   * write: a slice's first destination is the count of kept slots before
//     it (all the slots above T plus the first krem ties), its waves and
//     lanes scan on top of that, and every kept slot writes its list entry;
//     kept slots below budget are counted into n_low;
//   * gather: entries [0, n_low) read slots below budget, which are
//     destinations too, so every such source is read into a scratch area in
//     destination order (K rows, V groups, scores, positions) before any
//     slot is written: workgroups over entries, the launch boundary being
//     the barrier.  Entries with list[i] == i do not move;
//   * move: entries [0, n_low) are written from the scratch area, entries
//     [n_low, budget) straight from their sources, which lie at or above
//     budget where nothing writes; workgroups over entries.
// V moves as 16-byte groups of E destination tokens of one dim row.  A group
// that starts below n_low is gathered whole (its tokens from n_low on come
// from their high sources, tokens past budget keep their values) and written
// from the scratch area; a group from n_low on is moved from its sources.
// The same threshold search keeps, besides the window, a number of leading
// slots (head; zero for eviction): the Quest top-k over page scores uses it
// for page counts beyond its register top-k, with the sink pages as head and
// the recent pages as window.
constexpr int kSelThreads = 256;
constexpr int kSelPer = 16;                              // keys per thread and slice
constexpr int kSelSlice = kSelThreads * kSelPer;         // keys per slice workgroup
constexpr int kLgHeader = 16;                            // ints of the per-unit header
constexpr int kLgBins = 2048;
constexpr int kMoveEntries = 64;      // entries per workgroup pass of the gather and move kernels
constexpr int kMoveThreads = 256;
constexpr int kMoveWgs = 32;          // workgroups per unit of the gather and move kernels (at most)
// header fields
constexpr int kHActive = 0, kHLow = 1, kHPrefix = 2, kHMask = 3, kHKrem = 4, kHThresh = 5, kHArrive = 6;

struct LgView {
  int32_t* hdr;
  int32_t* hist;
  int32_t* counts;   // [slice][2]: kept above T (and window), ties at T
  int32_t* list;
};
__host__ __device__ inline int lg_slices(int cap) { return (cap + kSelSlice - 1) / kSelSlice; }
__host__ __device__ inline size_t lg_stride(int cap, int budget) {
  return (size_t)kLgHeader + kLgBins + 2 * (size_t)lg_slices(cap) + budget;
}
// Scratch of the low moves, after every unit's list area: per unit, for
// destination slots [0, nb) with nb = budget rounded up to kMoveEntries, K
// rows [nb][D], V groups [nb / E][D][E], scores [nb], positions [nb].
__host__ __device__ inline int low_rows(int budget) {
  return (budget + kMoveEntries - 1) / kMoveEntries * kMoveEntries;
}
__host__ __device__ inline size_t low_unit_bytes(int budget, int D, int esize) {
  const size_t nb = (size_t)low_rows(budget);
  return (nb * D * esize * 2 + nb * 8 + 255) & ~(size_t)255;
}
__host__ __device__ inline size_t low_scratch_offset(int units, int cap, int budget) {
  return ((size_t)units * lg_stride(cap, budget) * sizeof(int32_t) + 255) & ~(size_t)255;
}
template <typename T>
struct LowScratch {
  T* k;
  T* v;
  float* s;
  int32_t* p;
};
template <typename T>
__device__ __forceinline__ LowScratch<T> low_scratch(void* ws, int u, int units, int cap, int budget, int D) {
  char* base = static_cast<char*>(ws) + low_scratch_offset(units, cap, budget) +
               (size_t)u * low_unit_bytes(budget, D, (int)sizeof(T));
  const size_t nb = (size_t)low_rows(budget);
  LowScratch<T> r;
  r.k = reinterpret_cast<T*>(base);
  r.v = r.k + nb * D;
  r.s = reinterpret_cast<float*>(r.v + nb * D);
  r.p = reinterpret_cast<int32_t*>(r.s + nb);
  return r;
}

__device__ __forceinline__ LgView lg_view(int32_t* ws, int u, int cap, int budget) {
  LgView v;
  v.hdr = ws + (size_t)u * lg_stride(cap, budget);
  v.hist = v.hdr + kLgHeader;
  v.counts = v.hist + kLgBins;
  v.list = v.counts + 2 * lg_slices(cap);
  return v;
}

// hist[bin] += 1 for the valid lanes.  The lanes sharing the first two
// leaders' bins add with one atomic each (score keys crowd into few bins of
// the top digit, where same-address atomics would serialise); the rest add
// one by one.
__device__ __forceinline__ void hist_add(int* hist, uint32_t bin, bool valid) {
  uint64_t act = __ballot(valid);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    if (act == 0) break;
    const int leader = __ffsll((unsigned long long)act) - 1;
    const uint32_t lb = (uint32_t)__builtin_amdgcn_readlane((int)bin, leader);
    const uint64_t m = __ballot(valid && bin == lb);
    if ((int)(threadIdx.x & 63) == leader) atomicAdd(&hist[lb], (int)__popcll(m));
    valid = valid && bin != lb;
    act &= ~m;
  }
  if (valid) atomicAdd(&hist[bin], 1);
}

__device__ __forceinline__ void lg_digit(int pass, int& bits, int& shift) {
  bits = pass < 2 ? 11 : 10;
  shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
}

__global__ void __launch_bounds__(kSelThreads)
evict_init_kernel(KVDev kv, int budget, int head, int window, int32_t* __restrict__ ws) {
  const int h = blockIdx.x, b = blockIdx.y, u = b * kv.Hkv + h, tid = threadIdx.x;
  const int cap = kv.max_pages * kv.P;
  LgView v = lg_view(ws, u, cap, budget);
  const int L = clamp_len(kv.seq_lens[b], cap);
  if (tid == 0) {
    v.hdr[kHActive] = L > budget;
    v.hdr[kHLow] = 0;
    v.hdr[kHPrefix] = 0;
    v.hdr[kHMask] = 0;
    v.hdr[kHKrem] = budget - window - head;
    v.hdr[kHThresh] = (int)0xffffffffu;   // above every key: no candidate kept when nothing is left to pick
    v.hdr[kHArrive] = 0;
  }
  for (int i = tid; i < kLgBins; i += kSelThreads) v.hist[i] = 0;
}

// One pass of the threshold search: every slice workgroup counts its keys
// that match the prefix into an LDS histogram of the next digit and adds the
// non-zero bins into the unit's histogram; the last slice workgroup of the
// unit to count in (arrival counter in the header) then picks the digit that
// holds the krem-th largest key, clears the histogram and the counter for
// the next pass and extends the prefix.
__global__ void __launch_bounds__(kSelThreads)
evict_hist_kernel(KVDev kv, const float* __restrict__ scores, int slot_cap, int budget, int head, int window,
                  int pass, int32_t* __restrict__ ws) {
  __shared__ int hist[kLgBins];
  __shared__ int wsum[kSelThreads / 64 + 1];
  __shared__ int s_last, s_digit, s_excl;
  const int x = blockIdx.x, h = blockIdx.y, b = blockIdx.z, u = b * kv.Hkv + h, tid = threadIdx.x;
  const int cap = kv.max_pages * kv.P;
  LgView v = lg_view(ws, u, cap, budget);
  const int L = clamp_len(kv.seq_lens[b], cap);
  const int nc = L - window;
  if (L <= budget || budget - window - head <= 0 || x * kSelSlice >= nc) return;
  int bits, shift;
  lg_digit(pass, bits, shift);
  const int nb = 1 << bits;
  const uint32_t prefix = (uint32_t)v.hdr[kHPrefix], mask = (uint32_t)v.hdr[kHMask];
  const int krem = v.hdr[kHKrem];
  const float* srow = scores + (size_t)u * slot_cap;
  for (int i = tid; i < nb; i += kSelThreads) hist[i] = 0;
  float val[kSelPer];
  const int i0 = x * kSelSlice + tid;
#pragma unroll
  for (int k = 0; k < kSelPer; ++k) val[k] = srow[min(i0 + k * kSelThreads, nc - 1)];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kSelPer; ++k) {
    const uint32_t key = float_key(val[k]);
    const int sl = i0 + k * kSelThreads;
    hist_add(hist, (key >> shift) & (nb - 1), sl < nc && sl >= head && (key & mask) == prefix);
  }
  __syncthreads();
  for (int i = tid; i < nb; i += kSelThreads)
    if (hist[i]) atomicAdd(&v.hist[i], hist[i]);
  // the bins are added (at the point of coherence) before this workgroup counts in
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int n_slices = (nc + kSelSlice - 1) / kSelSlice;
  if (tid == 0) {
    s_last = atomicAdd(&v.hdr[kHArrive], 1) == n_slices - 1;
    s_digit = 0;
    s_excl = 0;
  }
  __syncthreads();
  if (!s_last) return;
  // the pick: thread t owns bins hi, hi - 1, ..., hi - 7 (descending)
  const int hi = nb - 1 - 8 * tid;
  int hv[8], c = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    hv[k] = hi - k >= 0 ? __hip_atomic_load(&v.hist[hi - k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
    c += hv[k];
  }
  int tot;
  const int excl = block_scan_dpp<kSelThreads>(c, wsum, &tot);
  if (c > 0 && excl < krem && krem <= excl + c) {
    int a = excl;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (krem > a && krem <= a + hv[k]) { s_digit = hi - k; s_excl = a; }
      a += hv[k];
    }
  }
  // the histogram is cleared for the next pass
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (hi - k >= 0) __hip_atomic_store(&v.hist[hi - k], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (tid == 0) {
    const uint32_t np = prefix | ((uint32_t)s_digit << shift);
    v.hdr[kHPrefix] = (int)np;
    v.hdr[kHMask] = (int)(mask | ((uint32_t)(nb - 1) << shift));
    v.hdr[kHKrem] = krem - s_excl;
    if (pass == 2) v.hdr[kHThresh] = (int)np;
    v.hdr[kHArrive] = 0;
  }
}

// Kept (above T, or among the first head or in the window) and tied slots
// of one slice of [0, L).
__device__ __forceinline__ void lg_flags(int sl, int end, int head, int nc, uint32_t T, float val, bool& def,
                                         bool& eq) {
  const uint32_t key = float_key(val);
  def = sl < end && (sl >= nc || sl < head || key > T);
  eq = sl < end && sl >= head && sl < nc && key == T;
}

__global__ void __launch_bounds__(kSelThreads)
evict_count_kernel(KVDev kv, const float* __restrict__ scores, int slot_cap, int budget, int head, int window,
                   int32_t* __restrict__ ws) {
  __shared__ int red[2][kSelThreads / 64];
  const int x = blockIdx.x, h = blockIdx.y, b = blockIdx.z, u = b * kv.Hkv + h, tid = threadIdx.x;
  const int cap = kv.max_pages * kv.P;
  LgView v = lg_view(ws, u, cap, budget);
  const int L = clamp_len(kv.seq_lens[b], cap);
  if (L <= budget) return;
  const int nc = L - window;
  const uint32_t T = (uint32_t)v.hdr[kHThresh];
  const float* srow = scores + (size_t)u * slot_cap;
  const int lane = tid & 63, wid = tid >> 6;
  // wave wid: slots [x * kSelSlice + wid * 64 * kSelPer, +64 * kSelPer), lane: kSelPer in a row
  const int j0 = x * kSelSlice + (wid * 64 + lane) * kSelPer;
  const int end = min(L, (x + 1) * kSelSlice);
  float val[kSelPer];
#pragma unroll
  for (int k = 0; k < kSelPer; ++k) val[k] = srow[min(j0 + k, nc - 1)];
  int cd = 0, ce = 0;
#pragma unroll
  for (int k = 0; k < kSelPer; ++k) {
    bool d, e;
    lg_flags(j0 + k, end, head, nc, T, val[k], d, e);
    cd += d;
    ce += e;
  }
  cd = __builtin_amdgcn_readlane(wave_inclusive_scan(cd), 63);
  ce = __builtin_amdgcn_readlane(wave_inclusive_scan(ce), 63);
  if (lane == 0) { red[0][wid] = cd; red[1][wid] = ce; }
  __syncthreads();
  if (tid == 0) {
    int td = 0, te = 0;
#pragma unroll
    for (int w = 0; w < kSelThreads / 64; ++w) { td += red[0][w]; te += red[1][w]; }
    v.counts[2 * x] = td;
    v.counts[2 * x + 1] = te;
  }
}

__global__ void __launch_bounds__(kSelThreads)
evict_write_kernel(KVDev kv, const float* __restrict__ scores, int slot_cap, int budget, int head, int window,
                   int32_t* __restrict__ ws) {
  __shared__ int red[2][kSelThreads / 64];
  __shared__ int s_base[2];
  const int x = blockIdx.x, h = blockIdx.y, b = blockIdx.z, u = b * kv.Hkv + h, tid = threadIdx.x;
  const int cap = kv.max_pages * kv.P;
  LgView v = lg_view(ws, u, cap, budget);
  const int L = clamp_len(kv.seq_lens[b], cap);
  if (L <= budget || x * kSelSlice >= L) return;
  const int nc = L - window;
  const uint32_t T = (uint32_t)v.hdr[kHThresh];
  const int krem = v.hdr[kHKrem];
  const float* srow = scores + (size_t)u * slot_cap;
  const int lane = tid & 63, wid = tid >> 6;
  const int j0 = x * kSelSlice + (wid * 64 + lane) * kSelPer;
  const int end = min(L, (x + 1) * kSelSlice);
  float val[kSelPer];
#pragma unroll
  for (int k = 0; k < kSelPer; ++k) val[k] = srow[min(j0 + k, nc - 1)];
  // kept slots and ties in the slices before this one
  int pd = 0, pe = 0;
  for (int j = tid; j < x; j += kSelThreads) { pd += v.counts[2 * j]; pe += v.counts[2 * j + 1]; }
  pd = __builtin_amdgcn_readlane(wave_inclusive_scan(pd), 63);
  pe = __builtin_amdgcn_readlane(wave_inclusive_scan(pe), 63);
  int cd = 0, ce = 0;
#pragma unroll
  for (int k = 0; k < kSelPer; ++k) {
    bool d, e;
    lg_flags(j0 + k, end, head, nc, T, val[k], d, e);
    cd += d;
    ce += e;
  }
  const int id = wave_inclusive_scan(cd), ie = wave_inclusive_scan(ce);
  if (lane == 0) { red[0][wid] = pd; red[1][wid] = pe; }
  __syncthreads();
  if (tid == 0) {
    int td = 0, te = 0;
#pragma unroll
    for (int w = 0; w < kSelThreads / 64; ++w) { td += red[0][w]; te += red[1][w]; }
    s_base[0] = td;
    s_base[1] = te;
  }
  __syncthreads();
  if (lane == 63) { red[0][wid] = id; red[1][wid] = ie; }
  __syncthreads();
  // ties and above-T slots before this lane's slots, over the whole unit
  int def_before = s_base[0] + id - cd, eq_before = s_base[1] + ie - ce;
  for (int w = 0; w < wid; ++w) { def_before += red[0][w]; eq_before += red[1][w]; }
  // destination = kept slots before: all above T, and the first krem ties
  int d = def_before + min(eq_before, krem);
  int eq_seen = eq_before, low = 0;
  int32_t* list = v.list;
#pragma unroll
  for (int k = 0; k < kSelPer; ++k) {
    const int sl = j0 + k;
    bool df, eq;
    lg_flags(sl, end, head, nc, T, val[k], df, eq);
    const bool keep = df || (eq && eq_seen < krem);
    eq_seen += eq;
    if (keep) {
      if (d < budget) list[d] = sl;     // exactly budget entries; the guard only bounds the store
      ++d;
      low += sl < budget;
    }
  }
  low = __builtin_amdgcn_readlane(wave_inclusive_scan(low), 63);
  if (lane == 0 && low) atomicAdd(&v.hdr[kHLow], low);
}

// The source of destination slot i: its list entry below budget; a slot past
// budget keeps its value.
__device__ __forceinline__ int move_src(const int32_t* list, int i, int budget) {
  return i < budget ? list[i] : i;
}

// Gather: for every entry below n_low that moves, its K row, score and
// position; for every V group that starts below n_low and holds a moving
// token, the whole 16-byte group per dim row.  Reads the pools, writes only
// the scratch area.  Workgroups stride over the unit's entries in passes of
// kMoveEntries.
template <typename T>
__global__ void __launch_bounds__(kMoveThreads)
evict_gather_kernel(KVDev kv, const float* __restrict__ scores, const int32_t* __restrict__ slot_pos,
                    int slot_cap, int budget, int32_t* __restrict__ ws) {
  constexpr int E = Chunk<T>::E;
  constexpr int kGroups = kMoveEntries / E;
  constexpr int kKT = kMoveEntries * (128 / E) / kMoveThreads;   // K chunk tasks per thread (D <= 128)
  constexpr int kVT = kGroups * 128 / kMoveThreads;              // V group tasks per thread
  __shared__ int s_src[kMoveEntries], s_sblk[kMoveEntries], s_dblk[kGroups];
  const int h = blockIdx.y, b = blockIdx.z, u = b * kv.Hkv + h, tid = threadIdx.x;
  const int cap = kv.max_pages * kv.P;
  const LgView lv = lg_view(ws, u, cap, budget);
  if (lv.hdr[kHActive] == 0) return;
  const int n_low = lv.hdr[kHLow];
  const int32_t* list = lv.list;
  const int P = kv.P, D = kv.D, Hkv = kv.Hkv, nch = D / E;
  const T* kpool = reinterpret_cast<const T*>(kv.k_pool);
  const T* vpool = reinterpret_cast<const T*>(kv.v_pool);
  const int32_t* bt = kv.block_table + (size_t)b * kv.max_pages;
  const int nblk = kv.num_blocks;
  auto blk_of = [&](int slot) { const int bl = bt[slot / P]; return (bl >= 0 && bl < nblk) ? bl : -1; };
  const float* srow = scores + (size_t)u * slot_cap;
  const int32_t* prow = slot_pos ? slot_pos + (size_t)u * slot_cap : nullptr;
  const LowScratch<T> sc = low_scratch<T>(ws, u, kv.B * Hkv, cap, budget, D);
  for (int i0 = blockIdx.x * kMoveEntries; i0 < n_low; i0 += gridDim.x * kMoveEntries) {
    if (tid < kMoveEntries) {
      const int i = i0 + tid;
      const int src = move_src(list, i, budget);
      s_src[tid] = src;
      s_sblk[tid] = src != i ? blk_of(src) : -1;
    }
    __syncthreads();
    if (tid < kGroups) {
      // a group below n_low with a moving token and a valid destination page
      const int g0 = i0 + tid * E;
      bool mv = false;
#pragma unroll
      for (int x = 0; x < E; ++x) mv |= s_src[tid * E + x] != g0 + x;
      s_dblk[tid] = (g0 < n_low && mv) ? blk_of(g0) : -1;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kKT; ++k) {
      const int t = tid + k * kMoveThreads, m = t % kMoveEntries, c = t / kMoveEntries;
      const int bs = s_sblk[m];
      if (c < nch && i0 + m < n_low && bs >= 0)
        *reinterpret_cast<uint4*>(sc.k + (size_t)(i0 + m) * D + c * E) =
            *reinterpret_cast<const uint4*>(kpool + page_base(bs, h, Hkv, P, D) +
                                            (size_t)(c * P + s_src[m] % P) * E);
    }
#pragma unroll
    for (int k = 0; k < kVT; ++k) {
      const int t = tid + k * kMoveThreads, dd = t % 128, j = t / 128;
      const int bd = s_dblk[j];
      if (dd < D && bd >= 0) {
        const int g0 = i0 + j * E;
        const T* drow = vpool + page_base(bd, h, Hkv, P, D) + v_off(g0 % P, dd, P);
        T val[E];
#pragma unroll
        for (int x = 0; x < E; ++x) {
          const int m = j * E + x, bs = s_sblk[m];
          val[x] = bs >= 0 ? vpool[page_base(bs, h, Hkv, P, D) + v_off(s_src[m] % P, dd, P)] : drow[x];
        }
        __builtin_memcpy(sc.v + ((size_t)(g0 / E) * D + dd) * E, val, 16);
      }
    }
    if (tid < kMoveEntries && i0 + tid < n_low && s_src[tid] != i0 + tid) {
      sc.s[i0 + tid] = srow[s_src[tid]];
      if (prow) sc.p[i0 + tid] = prow[s_src[tid]];
    }
    __syncthreads();   // the LDS tables are rewritten by the next pass
  }
}

// Move: entries [0, n_low) and the V groups that start below n_low from the
// scratch area (the gather launch has read every low source), entries
// [n_low, budget) and the later V groups from their sources at or above
// budget, which nothing writes.  Workgroups stride over the unit's entries.
// The choices of what moves repeat the gather's: an entry moves when its
// source differs from its slot; its K (and its tokens in V groups) only when
// its source page is valid; a V group when it holds a moving token and its
// page is valid.
template <typename T>
__global__ void __launch_bounds__(kMoveThreads)
evict_move_kernel(KVDev kv, float* __restrict__ scores, int32_t* __restrict__ slot_pos, int slot_cap,
                  int budget, int32_t* __restrict__ ws) {
  constexpr int E = Chunk<T>::E;
  constexpr int kGroups = kMoveEntries / E;
  constexpr int kKT = kMoveEntries * (128 / E) / kMoveThreads;
  constexpr int kVT = kGroups * 128 / kMoveThreads;
  __shared__ int s_src[kMoveEntries], s_sblk[kMoveEntries], s_dblk[kGroups];
  const int h = blockIdx.y, b = blockIdx.z, u = b * kv.Hkv + h, tid = threadIdx.x;
  const int cap = kv.max_pages * kv.P;
  const LgView lv = lg_view(ws, u, cap, budget);
  if (lv.hdr[kHActive] == 0) return;
  const int n_low = lv.hdr[kHLow];
  const int32_t* list = lv.list;
  const int P = kv.P, D = kv.D, Hkv = kv.Hkv, nch = D / E;
  T* kpool = reinterpret_cast<T*>(kv.k_pool);
  T* vpool = reinterpret_cast<T*>(kv.v_pool);
  const int32_t* bt = kv.block_table + (size_t)b * kv.max_pages;
  const int nblk = kv.num_blocks;
  auto blk_of = [&](int slot) { const int bl = bt[slot / P]; return (bl >= 0 && bl < nblk) ? bl : -1; };
  float* srow = scores + (size_t)u * slot_cap;
  int32_t* prow = slot_pos ? slot_pos + (size_t)u * slot_cap : nullptr;
  const LowScratch<T> sc = low_scratch<T>(ws, u, kv.B * Hkv, cap, budget, D);
  for (int i0 = blockIdx.x * kMoveEntries; i0 < budget; i0 += gridDim.x * kMoveEntries) {
    if (tid < kMoveEntries) {
      const int i = i0 + tid;
      const int src = move_src(list, i, budget);
      s_src[tid] = src;
      s_sblk[tid] = src != i ? blk_of(src) : -1;
    }
    __syncthreads();
    if (tid < kGroups) {
      const int g0 = i0 + tid * E;
      bool mv = false;
#pragma unroll
      for (int x = 0; x < E; ++x) mv |= s_src[tid * E + x] != g0 + x;
      s_dblk[tid] = (g0 < budget && mv) ? blk_of(g0) : -1;
    }
    __syncthreads();
    // every load of the pass first, then every store
    uint4 kr[kKT];
#pragma unroll
    for (int k = 0; k < kKT; ++k) {
      const int t = tid + k * kMoveThreads, m = t % kMoveEntries, c = t / kMoveEntries;
      const int bs = s_sblk[m];
      kr[k] = make_uint4(0u, 0u, 0u, 0u);
      if (c < nch && bs >= 0) {
        if (i0 + m < n_low)
          kr[k] = *reinterpret_cast<const uint4*>(sc.k + (size_t)(i0 + m) * D + c * E);
        else
          kr[k] = *reinterpret_cast<const uint4*>(kpool + page_base(bs, h, Hkv, P, D) +
                                                  (size_t)(c * P + s_src[m] % P) * E);
      }
    }
    uint4 vr[kVT];
#pragma unroll
    for (int k = 0; k < kVT; ++k) {
      const int t = tid + k * kMoveThreads, dd = t % 128, j = t / 128;
      const int bd = s_dblk[j];
      vr[k] = make_uint4(0u, 0u, 0u, 0u);
      if (dd < D && bd >= 0) {
        const int g0 = i0 + j * E;
        if (g0 < n_low) {
          vr[k] = *reinterpret_cast<const uint4*>(sc.v + ((size_t)(g0 / E) * D + dd) * E);
        } else {
          const T* drow = vpool + page_base(bd, h, Hkv, P, D) + v_off(g0 % P, dd, P);
          T val[E];
#pragma unroll
          for (int x = 0; x < E; ++x) {
            const int m = j * E + x, bs = s_sblk[m];
            val[x] = bs >= 0 ? vpool[page_base(bs, h, Hkv, P, D) + v_off(s_src[m] % P, dd, P)] : drow[x];
          }
          __builtin_memcpy(&vr[k], val, 16);
        }
      }
    }
    float sr = 0.f;
    int32_t pr = 0;
    const bool mv_me = tid < kMoveEntries && i0 + tid < budget && s_src[tid] != i0 + tid;
    if (mv_me) {
      if (i0 + tid < n_low) {
        sr = sc.s[i0 + tid];
        if (prow) pr = sc.p[i0 + tid];
      } else {
        sr = srow[s_src[tid]];
        if (prow) pr = prow[s_src[tid]];
      }
    }
#pragma unroll
    for (int k = 0; k < kKT; ++k) {
      const int t = tid + k * kMoveThreads, m = t % kMoveEntries, c = t / kMoveEntries;
      const int bd = s_dblk[m / E];
      if (c < nch && s_sblk[m] >= 0 && bd >= 0)
        *reinterpret_cast<uint4*>(kpool + page_base(bd, h, Hkv, P, D) + (size_t)(c * P + (i0 + m) % P) * E) = kr[k];
    }
#pragma unroll
    for (int k = 0; k < kVT; ++k) {
      const int t = tid + k * kMoveThreads, dd = t % 128, j = t / 128;
      const int bd = s_dblk[j];
      if (dd < D && bd >= 0) {
        const int g0 = i0 + j * E;
        *reinterpret_cast<uint4*>(vpool + page_base(bd, h, Hkv, P, D) + v_off(g0 % P, dd, P)) = vr[k];
      }
    }
    if (mv_me) {
      srow[i0 + tid] = sr;
      if (prow) prow[i0 + tid] = pr;
    }
    __syncthreads();   // the LDS tables are rewritten by the next pass
  }
}

// OmniKV: the ascending list of selected slots (or every slot when the
// sequence holds at most `budget`) as page entries with token masks, the same
// for every KV head; entries past the last page are -1 with mask 0.  One
// workgroup per (sequence, KV head) walks the list in tiles of 1024 entries
// staged in LDS (with the entry before the tile and the P - 1 after it): an
// entry that starts a page finds its place by a block scan and ORs the token
// bits of the entries that follow it in the same page (at most P of them).
constexpr int kPgThreads = 1024;
__global__ void __launch_bounds__(kPgThreads)
tokens_to_pages_kernel(KVDev kv, int Hkv_out, int budget, const int32_t* __restrict__ ws,
                       int32_t* __restrict__ sel_pages, uint32_t* __restrict__ sel_mask, int k_pages) {
  constexpr int kStage = kPgThreads + 1 + 32;
  __shared__ int s_slot[kStage];            // s_slot[k] = slot of list entry i0 - 1 + k
  __shared__ int wsum[kPgThreads / 64 + 1];
  const int b = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int P = kv.P, cap = kv.max_pages * P;
  const LgView v = lg_view(const_cast<int32_t*>(ws), b, cap, budget);
  const int L = clamp_len(kv.seq_lens[b], cap);
  const bool listed = L > budget && v.hdr[kHActive] != 0;
  const int n = listed ? budget : L;
  int32_t* pg_out = sel_pages + ((size_t)b * Hkv_out + h) * k_pages;
  uint32_t* mk_out = sel_mask + ((size_t)b * Hkv_out + h) * k_pages;
  int base = 0;                             // entries written by earlier tiles
  for (int i0 = 0; i0 < n; i0 += kPgThreads) {
    for (int k = tid; k < kStage; k += kPgThreads) {
      const int i = i0 - 1 + k;
      s_slot[k] = (i >= 0 && i < n) ? (listed ? v.list[i] : i) : 0;
    }
    __syncthreads();
    const int i = i0 + tid;
    const int cur = s_slot[tid + 1], page = cur / P;
    const bool start = i < n && (i == 0 || s_slot[tid] / P != page);
    int total;
    const int out = base + block_scan_dpp<kPgThreads>(start ? 1 : 0, wsum, &total);
    if (start && out < k_pages) {
      uint32_t mask = 0;
      for (int j = 0; j < P && i + j < n; ++j) {
        const int sj = s_slot[tid + 1 + j];
        if (sj / P != page) break;
        mask |= 1u << (sj - page * P);
      }
      pg_out[out] = page;
      mk_out[out] = mask;
    }
    base += total;
    __syncthreads();                        // the next tile restages s_slot and wsum
  }
  for (int e = base + tid; e < k_pages; e += kPgThreads) {
    pg_out[e] = -1;
    mk_out[e] = 0u;
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
                   int window, void* ws, hipStream_t s) {
  dim3 grid(kv.Hkv, kv.B);
  const int cap = kv.max_pages * kv.P;
  // a budget of the capacity or more evicts nothing; the workspace's lists
  // are sized for at most the capacity
  if (budget > cap) budget = cap;
  if (window > budget) window = budget;
  if (cap <= kEvFastMax) {
    // ws: per-sequence counters (the length update fused into the kernel),
    // or nullptr (a separate clamp launch)
    int* seq_counters = static_cast<int*>(ws);
    const size_t lds = (size_t)ev_layout(cap, kv.max_pages).total * 4;
    h2o_evict_fast_kernel<T><<<grid, kEvThreads, lds, s>>>(kv, scores, slot_pos, slot_cap, budget, window,
                                                           seq_counters);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || seq_counters != nullptr) return e;
  } else {
    int32_t* w = static_cast<int32_t*>(ws);
    const dim3 units(kv.Hkv, kv.B), slices(lg_slices(cap), kv.Hkv, kv.B);
    evict_init_kernel<<<units, kSelThreads, 0, s>>>(kv, budget, 0, window, w);
    for (int pass = 0; pass < 3; ++pass)
      evict_hist_kernel<<<slices, kSelThreads, 0, s>>>(kv, scores, slot_cap, budget, 0, window, pass, w);
    evict_count_kernel<<<slices, kSelThreads, 0, s>>>(kv, scores, slot_cap, budget, 0, window, w);
    evict_write_kernel<<<slices, kSelThreads, 0, s>>>(kv, scores, slot_cap, budget, 0, window, w);
    const int passes = (budget + kMoveEntries - 1) / kMoveEntries;
    const dim3 movers(passes < kMoveWgs ? passes : kMoveWgs, kv.Hkv, kv.B);
    evict_gather_kernel<T><<<movers, kMoveThreads, 0, s>>>(kv, scores, slot_pos, slot_cap, budget, w);
    evict_move_kernel<T><<<movers, kMoveThreads, 0, s>>>(kv, scores, slot_pos, slot_cap, budget, w);
  }
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
  const int nx = (cap + kAccThreads - 1) / kAccThreads;
  dim3 grid(nx < kAccBlocks ? nx : kAccBlocks, kv.Hkv, kv.B);
  h2o_accumulate_kernel<<<grid, kAccThreads, 0, s>>>(kv, logits, lse, logit_cap, n_new, scores, slot_cap);
  return hipGetLastError();
}

hipError_t launch_h2o_evict(const KVDev& kv, int dtype, float* scores, int32_t* slot_pos,
                            int slot_cap, int budget, int window, void* ws, hipStream_t s) {
  if (dtype == SP_BF16) return evict_t<bf16_t>(kv, scores, slot_pos, slot_cap, budget, window, ws, s);
  return evict_t<float>(kv, scores, slot_pos, slot_cap, budget, window, ws, s);
}

// Top-`budget` slots of one score row per sequence (ties: lower slot), as
// page entries with token masks for every KV head of `kv`.
hipError_t launch_token_topk_pages(const KVDev& kv, const float* scores, int slot_cap, int budget, void* ws,
                                   int32_t* sel_pages, uint32_t* sel_mask, int k_pages, hipStream_t s) {
  KVDev one = kv;          // one unit per sequence
  one.Hkv = 1;
  int32_t* w = static_cast<int32_t*>(ws);
  const int cap = kv.max_pages * kv.P;
  if (budget > cap) budget = cap;   // every slot is kept; the lists are sized for at most the capacity
  const dim3 units(1, kv.B), slices(lg_slices(cap), 1, kv.B);
  evict_init_kernel<<<units, kSelThreads, 0, s>>>(one, budget, 0, 0, w);
  for (int pass = 0; pass < 3; ++pass)
    evict_hist_kernel<<<slices, kSelThreads, 0, s>>>(one, scores, slot_cap, budget, 0, 0, pass, w);
  evict_count_kernel<<<slices, kSelThreads, 0, s>>>(one, scores, slot_cap, budget, 0, 0, w);
  evict_write_kernel<<<slices, kSelThreads, 0, s>>>(one, scores, slot_cap, budget, 0, 0, w);
  tokens_to_pages_kernel<<<dim3(kv.B, kv.Hkv), kPgThreads, 0, s>>>(one, kv.Hkv, budget, w, sel_pages, sel_mask,
                                                               k_pages);
  return hipGetLastError();
}

namespace {
// Quest selection rows from the kept-page lists: ascending page indices,
// padded with -1; a unit with at most budget pages takes all of them.
__global__ void __launch_bounds__(kSelThreads)
list_to_sel_kernel(KVDev pv, int top_k, int budget, int32_t* __restrict__ ws, int32_t* __restrict__ sel) {
  const int h = blockIdx.y, b = blockIdx.z, u = b * pv.Hkv + h;
  const int cap = pv.max_pages;
  const int L = clamp_len(pv.seq_lens[b], cap);
  const int32_t* list = lg_view(ws, u, cap, budget).list;
  int32_t* row = sel + (size_t)u * top_k;
  for (int i = blockIdx.x * kSelThreads + threadIdx.x; i < top_k; i += gridDim.x * kSelThreads)
    row[i] = L > budget ? (i < budget ? list[i] : -1) : (i < L ? i : -1);
}

}  // namespace

hipError_t launch_page_topk_list(const KVDev& kv, const float* scores, int32_t* n_pages, int top_k, int n_sink,
                                 int n_recent, int32_t* sel, void* ws, hipStream_t s) {
  KVDev pv = kv;           // one slot per page; the lengths are the page counts
  pv.P = 1;
  pv.seq_lens = n_pages;
  const int cap = kv.max_pages;
  // a top_k of every page keeps all of them; the lists are sized for at most
  // the page count
  const int budget = top_k < cap ? top_k : cap;
  int32_t* w = static_cast<int32_t*>(ws);
  const dim3 units(kv.Hkv, kv.B), slices(lg_slices(cap), kv.Hkv, kv.B);
  evict_init_kernel<<<units, kSelThreads, 0, s>>>(pv, budget, n_sink, n_recent, w);
  for (int pass = 0; pass < 3; ++pass)
    evict_hist_kernel<<<slices, kSelThreads, 0, s>>>(pv, scores, cap, budget, n_sink, n_recent, pass, w);
  evict_count_kernel<<<slices, kSelThreads, 0, s>>>(pv, scores, cap, budget, n_sink, n_recent, w);
  evict_write_kernel<<<slices, kSelThreads, 0, s>>>(pv, scores, cap, budget, n_sink, n_recent, w);
  const int xs = (top_k + kSelThreads - 1) / kSelThreads;
  list_to_sel_kernel<<<dim3(xs < 16 ? xs : 16, kv.Hkv, kv.B), kSelThreads, 0, s>>>(pv, top_k, budget, w, sel);
  return hipGetLastError();
}

size_t page_topk_list_bytes(const KVDev& kv) {
  return (size_t)kv.B * kv.Hkv * lg_stride(kv.max_pages, kv.max_pages) * sizeof(int32_t);
}

size_t token_topk_workspace_bytes(const KVDev& kv, int budget) {
  const int cap = kv.max_pages * kv.P;
  const int bud = (budget >= 1 && budget < cap) ? budget : cap;
  return (size_t)kv.B * lg_stride(cap, bud) * sizeof(int32_t);
}

bool h2o_evict_list_path(const KVDev& kv) { return kv.max_pages * kv.P > kEvFastMax; }

size_t h2o_evict_workspace_bytes(const KVDev& kv, int budget, int esize) {
  const int cap = kv.max_pages * kv.P;
  // up to kEvFastMax slots: optional per-sequence counters (zero between calls)
  if (cap <= kEvFastMax) return ((size_t)kv.B * sizeof(int) + 255) & ~(size_t)255;
  const int bud = (budget >= 1 && budget < cap) ? budget : cap;
  const int units = kv.B * kv.Hkv;
  // per-unit lists, then the low moves' scratch
  return low_scratch_offset(units, cap, bud) + (size_t)units * low_unit_bytes(bud, kv.D, esize);
}

}  // namespace spk
