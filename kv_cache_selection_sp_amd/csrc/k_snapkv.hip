// SnapKV prompt scoring from an observation window, and its pooling.
//
// "SparseEngine: Sparse-First Inference Engine", Appendix A.3, "SnapKV: Prompt
// Selection from an Observation Window": the prompt's last w positions form
// the observation window; every earlier position j collects the attention the
// window's queries give it, u(j) = sum over window queries of their softmax
// weight on j (each window query's softmax runs over its causal prefix); a
// one-dimensional max pooling of width kappa turns u into the selection score
// s(j).  Under GQA the score of a KV head sums the group's query heads.
//
// For one (sequence, KV head) the window queries of the G query heads are
// R = G * w rows.  A row's softmax normaliser needs every key up to its own
// position, so the work is two sweeps over the prompt's keys:
//   1. normalisers: workgroups over (key chunk, row slab, sequence x KV head)
//      form S^T = K . Q^T tiles with v_mfma_f32_16x16x32_bf16 (16 keys x 16
//      rows) and keep an online (max, sum) per row and lane over the chunk,
//      keys past a row's own position masked; the lanes and waves are merged
//      at the end, and a merge kernel folds the chunks into lse per row;
//   2. scores: the same tiles taken as S = Q . K^T (16 rows x 16 keys), so a
//      lane holds one key of four rows per block; p = 2^(s - lse) is summed
//      over the rows in registers, then across lanes and waves, giving u(j)
//      for every earlier position j < L - w.
// Keys are read in 16-key tiles, in stages of kStage tiles: each wave loads
// its share of a stage two stages ahead into registers (16 bytes per lane
// and piece, one 1 KB wave load per 32 dims of a tile) and writes it into one
// of two LDS buffers a stage before it is used; each wave owns 64 rows (four
// 16-row blocks) whose Q operands stay in registers and reads the shared
// tiles from LDS.  Everything is in the log2 domain:
// s = log2(e) * scale * (q . k).
// A pooling kernel sums the row slabs, takes the max over
// [j - kappa/2, j + kappa/2] clipped to the earlier positions and writes s(j),
// +inf at the sink positions.
#include "sp_internal.h"

namespace spk {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kSlab = 256;            // rows per workgroup (4 waves x 64)
constexpr int kStage = 2;             // 16-key tiles per LDS stage: two stages in flight in
                                      // registers cost 8 * KS VGPRs per lane, which keeps the
                                      // sweeps at three waves per SIMD (six tiles a stage: two)
constexpr int kMaxChunk = 1024;       // keys per workgroup: <= 64 pages (block ids in one
                                      // register per lane) and <= 64 tiles of column sums in LDS
constexpr int kMaxStages = (kMaxChunk / 16 + kStage - 1) / kStage;
constexpr int kTargetWG = 2048;       // workgroups a sweep aims for
constexpr int kPoolOut = 1024;        // pooled outputs per workgroup
constexpr int kMaxPoolHalf = 128;     // kappa <= 2 * kMaxPoolHalf + 1
constexpr float kMinState = -1e30f;   // running max before any key (finite: no inf - inf)
constexpr int kPassSlabs = 16;        // row slabs per pass at least
constexpr size_t kPassBytes = (size_t)256 << 20;   // column sums of one pass: as many slabs
                                      // as fit (one launch per sweep fills the chip in
                                      // whole rounds better than several small ones)
constexpr int kModeWindow = 0;        // SnapKV: u(j) for the earlier positions, pooled
constexpr int kModeChunk = 1;         // H2O prefill: u(j) for every slot, added to the scores

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Workgroup barrier that waits for this wave's LDS operations but not for its
// outstanding global loads, so the loads of later stages stay in flight across
// it (a __syncthreads would wait for them).
__device__ __forceinline__ void barrier_keep_loads() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt at their maxima
  asm volatile("s_barrier" ::: "memory");
}

__device__ __forceinline__ float swizzle_xor16(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), kSwizzleXor16));
}

// Sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 with the gfx950 row
// swaps (vector ALU; both lanes of a pair add the same two values in the same
// order, so every lane ends with the same bits).
__device__ __forceinline__ float sum_rows4(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void merge_state(float& m, float& l, float m2, float l2) {
  const float M = fmaxf(m, m2);
  l = l * fast_exp2(m - M) + l2 * fast_exp2(m2 - M);
  m = M;
}

struct SnapArgs {
  KVDev kv;
  const bf16_t* q;     // [B][w][Hq][D]
  int w, R;            // query positions (the last w slots) and rows R = G * w
  int row0, n_slab;    // this pass: rows [row0, row0 + n_slab * kSlab)
  int mode;            // kModeWindow (SnapKV) or kModeChunk (H2O prefill chunk)
  int first_pass;
  float c;             // log2(e) * scale
  int lp;              // log2 of the page size (16 or 32 tokens)
  int chunk1, n_chunk1, chunk2, n_chunk2;
  float2* ml;          // [B * Hkv][n_slab][n_chunk1][kSlab]: (max, sum) per chunk and row
  float* lse;          // [B * Hkv][n_slab * kSlab] (log2 domain; +inf for padding rows)
  float* up;           // [n_slab][B * Hkv][cap]: column sums per row slab of the pass
  float* scores;       // [B][Hkv][slot_cap]
  int slot_cap, half, n_sink;
};

// One wave's view of its rows and of the chunk it streams.
template <int D, int NRG>
struct SweepCtx {
  static constexpr int KS = D / 32;                  // MFMA k-steps (1 KB wave loads) per tile
  static constexpr int TB = 16 * D * 2;              // bytes of a 16-key tile
  static constexpr int NKG = kWaves / NRG;           // waves sharing a row group split the tiles
  static constexpr int LPS = kStage * KS / kWaves;   // 16-byte pieces per lane and stage
  static_assert(LPS * kWaves == kStage * KS, "stage loads divide over the waves");

  bf16x8_t qop[4][KS];   // this wave's 64 rows: Q[row][8 dims] per lane
  int blk_reg;           // block id of page (page0 + lane) of the chunk
  int page0;

  // Q operands of rows slab * kSlab + rg * 64 + rb * 16 + (lane & 15).  Rows
  // past R load row R - 1 (unconditional loads, no wait before the stage
  // loads): their normaliser states are never used and the score sweep gives
  // them lse = +inf, so they add 2^-inf = 0.
  __device__ __forceinline__ void load_q(const SnapArgs& A, int b, int h, int slab, int rg, int lane) {
    const int G = A.kv.G, Hq = A.kv.Hq, g = lane >> 4;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int row = A.row0 + slab * kSlab + rg * 64 + rb * 16 + (lane & 15);
      const int rc = row < A.R ? row : A.R - 1;
      const int i = rc / G, a = rc - i * G;
      const bf16_t* src = A.q + ((size_t)(b * A.w + i) * Hq + h * G + a) * D + 8 * g;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qop[rb][ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(src + 32 * ks));
      }
    }
  }

  // Block ids of the chunk's pages [page0, page0 + 64) (clamped to the chunk).
  __device__ __forceinline__ void load_blocks(const SnapArgs& A, int b, int k0, int k1, int lane) {
    page0 = k0 >> A.lp;
    const int last = (k1 - 1) >> A.lp;
    const int pg = min(page0 + lane, last);
    int blk = A.kv.block_table[(size_t)b * A.kv.max_pages + pg];
    blk_reg = (blk < 0 || blk >= A.kv.num_blocks) ? 0 : blk;   // invalid ids read block 0
  }

  // Loads of stage s (tiles [s * kStage, ...) of the chunk) into registers.
  // Page arithmetic with shifts (the page size is a power of two): a runtime
  // division and 64-bit page-base product per piece had made the scalar
  // instructions half as many as the vector ones.
  // this wave's LPS pieces of 16 bytes per lane, piece j = wid + kWaves * i
  // being dims [32 * (j % KS), +32) of tile j / KS (lane: chunk 4 * (j % KS)
  // + (lane >> 4), token lane & 15).  Pieces past the chunk load its last
  // tile again (their LDS slots are never read), so no load is conditional.
  __device__ __forceinline__ void fetch(const SnapArgs& A, u32x4_t (&r)[LPS], int h, int tile0, int s,
                                        int ntile, int wid, int lane) {
    const int lp = A.lp;
    const bf16_t* kpool = reinterpret_cast<const bf16_t*>(A.kv.k_pool);
    const size_t blk_stride = ((size_t)A.kv.Hkv * D) << lp;   // elements of one block (all heads)
    const bf16_t* head = kpool + (((size_t)h * D) << lp);
    const int g = lane >> 4, t = lane & 15;
#pragma unroll
    for (int i = 0; i < LPS; ++i) {
      const int j = wid + kWaves * i;
      const int q = j / KS, part = j - q * KS;
      const int tok = (tile0 + min(s * kStage + q, ntile - 1)) * 16;   // first token (one page)
      const int blk = __builtin_amdgcn_readlane(blk_reg, (tok >> lp) - page0);
      r[i] = *reinterpret_cast<const u32x4_t*>(head + (size_t)blk * blk_stride +
                                             ((((4 * part + g) << lp) + (tok & ((1 << lp) - 1)) + t) << 3));
    }
  }

  // The pieces of `fetch` into a stage buffer, in the MFMA operand order.
  __device__ __forceinline__ static void put(unsigned char* buf, const u32x4_t (&r)[LPS], int wid, int lane) {
#pragma unroll
    for (int i = 0; i < LPS; ++i) {
      const int j = wid + kWaves * i;
      const int q = j / KS, part = j - q * KS;
      *reinterpret_cast<u32x4_t*>(buf + q * TB + part * 1024 + lane * 16) = r[i];
    }
  }

  // Streams tiles [0, ntile) of the chunk and calls body(buf, s, tiles) once
  // per stage of kStage tiles.  Two register sets hold the next two stages
  // in flight (loaded two stages ahead, so a load's latency is spread over
  // two stages of work); a stage is written into one of two LDS buffers one
  // stage before it is computed.  Only LDS waits precede the barriers, so the
  // loads stay in flight across them, and each store into LDS waits (by the
  // compiler's count) for just the loads it writes.  The loads are issued
  // unconditionally, in the same order on every path (past the last stage
  // they re-read the chunk's last tile), so that this count stays exact.
  template <class Body>
  __device__ __forceinline__ void sweep(const SnapArgs& A, unsigned char* b0, unsigned char* b1, int h,
                                        int tile0, int ntile, int wid, int lane, Body&& body) {
    const int nstage = (ntile + kStage - 1) / kStage;
    u32x4_t ra[LPS], rb[LPS];
    fetch(A, ra, h, tile0, 0, ntile, wid, lane);
    fetch(A, rb, h, tile0, 1, ntile, wid, lane);
    put(b0, ra, wid, lane);
    fetch(A, ra, h, tile0, 2, ntile, wid, lane);
    barrier_keep_loads();
    // Stages past nstage leave through the breaks.  The compiler keeps this
    // a loop (its trip count is only bounded), so the write of rb at its top,
    // of loads issued in the previous iteration, waits for every load in
    // flight; stage loads straight into LDS with exact waits, and a rotated
    // loop whose writes each follow a younger stage's loads, measured no
    // faster.
    for (int s = 0; s < kMaxStages; s += 2) {
      if (s >= nstage) break;
      // stage s is in b0, stage s + 1 in rb, stage s + 2 in ra
      if (s + 1 < nstage) put(b1, rb, wid, lane);
      fetch(A, rb, h, tile0, s + 3, ntile, wid, lane);
      body(b0, s, min(kStage, ntile - s * kStage));
      barrier_keep_loads();
      if (s + 1 >= nstage) break;
      if (s + 2 < nstage) put(b0, ra, wid, lane);
      fetch(A, ra, h, tile0, s + 4, ntile, wid, lane);
      body(b1, s + 1, min(kStage, ntile - (s + 1) * kStage));
      barrier_keep_loads();
    }
  }

  __device__ __forceinline__ static void read_tile(const unsigned char* tb, int lane, bf16x8_t (&kop)[KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kop[ks] = *reinterpret_cast<const bf16x8_t*>(tb + (ks * 64 + lane) * 16);
  }

  // S^T = K . Q^T of one tile for the four row blocks: acc[rb][e] is row
  // (lane & 15) of block rb against key 4 * (lane >> 4) + e.
  __device__ __forceinline__ static void tile_st(const unsigned char* tb, int lane,
                                                 const bf16x8_t (&qop)[4][KS], float4_t (&acc)[4]) {
    bf16x8_t kop[KS];
    read_tile(tb, lane, kop);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      acc[rb] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[ks], qop[rb][ks], acc[rb], 0, 0, 0);
    }
  }

  // S = Q . K^T of one tile: acc[rb][e] is row 4 * (lane >> 4) + e of block rb
  // against key (lane & 15).
  __device__ __forceinline__ static void tile_s(const unsigned char* tb, int lane,
                                                const bf16x8_t (&qop)[4][KS], float4_t (&acc)[4]) {
    bf16x8_t kop[KS];
    read_tile(tb, lane, kop);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      acc[rb] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qop[rb][ks], kop[ks], acc[rb], 0, 0, 0);
    }
  }
};

// ------------------------------------------------------------ sweep 1: normalisers
template <int D, int NRG>
__global__ void __launch_bounds__(kThreads, 2) snap_lse_kernel(SnapArgs A) {
  using C = SweepCtx<D, NRG>;
  constexpr int TB = C::TB, NKG = C::NKG;
  __shared__ __align__(16) unsigned char buf0[kStage * TB];
  __shared__ __align__(16) unsigned char buf1[kStage * TB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wid % NRG, kg = wid / NRG;
  const int g = lane >> 4;
  const int u = blockIdx.z, b = u / A.kv.Hkv, h = u - b * A.kv.Hkv;
  const int slab = blockIdx.y, ck = blockIdx.x;
  const int cap = A.kv.max_pages * A.kv.P;
  const int L = clamp_len(A.kv.seq_lens[b], cap);
  const int w = A.w;
  const int k0 = ck * A.chunk1;
  // the slab's last row sees keys up to L - w + i_max; later chunks are skipped
  const int i_max = min(w - 1, (A.row0 + (slab + 1) * kSlab - 1) / A.kv.G);
  if (L < w || (A.mode == kModeWindow && L == w) || k0 >= L || k0 > L - w + i_max) return;
  // keys past the slab's last visible one (L - w + i_max) would only add zeros
  const int k1 = min(min(L, k0 + A.chunk1), L - w + i_max + 1);
  const int tile0 = k0 >> 4, ntile = (k1 - k0 + 15) >> 4;

  C cx;
  cx.load_blocks(A, b, k0, k1, lane);
  cx.load_q(A, b, h, slab, rg, lane);
  // keys visible to this lane's rows (S^T layout: row = lane & 15 of each block)
  int lim[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int row = A.row0 + slab * kSlab + rg * 64 + rb * 16 + (lane & 15);
    lim[rb] = L - w + row / A.kv.G;       // past R: beyond L, never stored
  }
  // m: the reference of the running sum l = sum 2^(s - m) (log2 domain,
  // s = c * q.k).  It need not be the maximum: a tile is summed against m as
  // it is, and only a tile whose partial sum exceeds 2^64 (or overflows: the
  // first tile, against kMinState) is redone against its own maximum, so no
  // tile's maximum is taken in the common case and l stays finite.
  float m[4], l[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) { m[rb] = kMinState; l[rb] = 0.f; }
  const float c = A.c;

  cx.sweep(A, buf0, buf1, h, tile0, ntile, wid, lane, [&](const unsigned char* buf, int s, int nq) {
    // software-pipelined: the MFMAs of the next tile are issued before the
    // softmax update of the current one, so the matrix core and the vector
    // ALU can work side by side.  The next tile is clamped to the stage (the
    // last step recomputes a tile and drops it): no branch around the MFMAs.
    auto mask = [&](float4_t (&acc)[4], int q) {
      const int key0 = (tile0 + s * kStage + q) * 16;
      if (key0 + 15 > L - w) {     // the tile reaches into the window: causal mask
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (key0 + 4 * g + e > lim[rb]) acc[rb][e] = -INFINITY;
      }
    };
    // Sums against the references as they are; only when a tile's sum
    // exceeds 2^64 is the tile redone against the larger of the reference and
    // its own maximum, the earlier sum rescaled.
    auto update = [&](float4_t (&acc)[4]) {
      float part_l[4];
      bool grow = false;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const float nm = -m[rb];
        part_l[rb] = (fast_exp2(fmaf(acc[rb][0], c, nm)) + fast_exp2(fmaf(acc[rb][1], c, nm))) +
                     (fast_exp2(fmaf(acc[rb][2], c, nm)) + fast_exp2(fmaf(acc[rb][3], c, nm)));
        grow |= part_l[rb] > 0x1p64f;
      }
      if (__ballot(grow)) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const float tm = fmaxf(fmaxf(acc[rb][0], acc[rb][1]), fmaxf(acc[rb][2], acc[rb][3]));
          const float mn = fmaxf(m[rb], tm * c), nm = -mn;
          part_l[rb] = (fast_exp2(fmaf(acc[rb][0], c, nm)) + fast_exp2(fmaf(acc[rb][1], c, nm))) +
                       (fast_exp2(fmaf(acc[rb][2], c, nm)) + fast_exp2(fmaf(acc[rb][3], c, nm)));
          l[rb] *= fast_exp2(m[rb] - mn);
          m[rb] = mn;
        }
      }
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) l[rb] += part_l[rb];
    };
    float4_t a0[4], a1[4];
    int q = kg;
    if (q < nq) C::tile_st(buf + q * TB, lane, cx.qop, a0);
    while (q < nq) {
      const int q1 = q + NKG;
      mask(a0, q);
      C::tile_st(buf + min(q1, nq - 1) * TB, lane, cx.qop, a1);
      update(a0);
      if (q1 >= nq) break;
      const int q2 = q1 + NKG;
      mask(a1, q1);
      C::tile_st(buf + min(q2, nq - 1) * TB, lane, cx.qop, a0);
      update(a1);
      q = q2;
    }
  });

  // lanes holding the same rows (lane, lane ^ 16, lane ^ 32, lane ^ 48)
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    merge_state(m[rb], l[rb], swizzle_xor16(m[rb]), swizzle_xor16(l[rb]));
    merge_state(m[rb], l[rb], __shfl_xor(m[rb], 32, 64), __shfl_xor(l[rb], 32, 64));
  }
  // waves holding the same rows (different key groups), through LDS
  float2* red = reinterpret_cast<float2*>(buf0);   // [NKG][NRG * 64]
  if (g == 0) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
      red[kg * (NRG * 64) + rg * 64 + rb * 16 + lane] = make_float2(m[rb], l[rb]);
  }
  __syncthreads();
  if (tid < NRG * 64) {
    float2 st = red[tid];
#pragma unroll
    for (int k = 1; k < NKG; ++k) {
      const float2 o = red[k * (NRG * 64) + tid];
      merge_state(st.x, st.y, o.x, o.y);
    }
    A.ml[(((size_t)u * A.n_slab + slab) * A.n_chunk1 + ck) * kSlab + tid] = st;
  }
}

// Fold the chunks of every row into lse (log2 domain); +inf past R.  Four
// groups of 256 threads take every fourth chunk (loads batched four deep),
// then LDS combines the groups.
constexpr int kMergeThreads = 4 * kSlab;
__global__ void __launch_bounds__(kMergeThreads) snap_merge_kernel(SnapArgs A) {
  __shared__ float2 part[4][kSlab];
  const int u = blockIdx.y, slab = blockIdx.x, tid = threadIdx.x;
  const int row = tid & (kSlab - 1), grp = tid >> 8;
  const int b = u / A.kv.Hkv;
  const int cap = A.kv.max_pages * A.kv.P;
  const int L = clamp_len(A.kv.seq_lens[b], cap);
  if (L < A.w || (A.mode == kModeWindow && L == A.w)) return;
  // the chunks the normaliser sweep ran for this slab (see snap_lse_kernel)
  const int i_max = min(A.w - 1, (A.row0 + (slab + 1) * kSlab - 1) / A.kv.G);
  const int nck = min(min(A.n_chunk1, (L + A.chunk1 - 1) / A.chunk1), (L - A.w + i_max) / A.chunk1 + 1);
  const float2* p = A.ml + ((size_t)u * A.n_slab + slab) * A.n_chunk1 * kSlab + row;
  float m = kMinState, l = 0.f;
  int k = grp;
  for (; k + 12 < nck; k += 16) {
    const float2 o0 = p[(size_t)k * kSlab], o1 = p[(size_t)(k + 4) * kSlab];
    const float2 o2 = p[(size_t)(k + 8) * kSlab], o3 = p[(size_t)(k + 12) * kSlab];
    merge_state(m, l, o0.x, o0.y);
    merge_state(m, l, o1.x, o1.y);
    merge_state(m, l, o2.x, o2.y);
    merge_state(m, l, o3.x, o3.y);
  }
  for (; k < nck; k += 4) {
    const float2 o = p[(size_t)k * kSlab];
    merge_state(m, l, o.x, o.y);
  }
  part[grp][row] = make_float2(m, l);
  __syncthreads();
  if (grp == 0) {
#pragma unroll
    for (int j = 1; j < 4; ++j) merge_state(m, l, part[j][row].x, part[j][row].y);
    const int r = slab * kSlab + row;
    A.lse[(size_t)u * A.n_slab * kSlab + r] = A.row0 + r < A.R ? m + fast_log2(l) : INFINITY;
  }
}

// ------------------------------------------------------------ sweep 2: scores
// CHUNK: the keys are every slot [0, L), the ones in the query range masked
// per row (causal); otherwise the earlier positions [0, L - w), all visible.
template <int D, int NRG, bool CHUNK>
__global__ void __launch_bounds__(kThreads, 2) snap_score_kernel(SnapArgs A) {
  using C = SweepCtx<D, NRG>;
  constexpr int TB = C::TB, NKG = C::NKG;
  __shared__ __align__(16) unsigned char buf0[kStage * TB];
  __shared__ __align__(16) unsigned char buf1[kStage * TB];
  __shared__ float part[(kMaxChunk / 16) * NRG * 16];   // [chunk tile][row group][key]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wid % NRG, kg = wid / NRG;
  const int g = lane >> 4;
  const int u = blockIdx.z, b = u / A.kv.Hkv, h = u - b * A.kv.Hkv;
  const int slab = blockIdx.y, ck = blockIdx.x;
  const int cap = A.kv.max_pages * A.kv.P;
  const int L = clamp_len(A.kv.seq_lens[b], cap);
  const int w = A.w;
  const int Le = CHUNK ? L : L - w;       // keys scored: [0, Le)
  const int k0 = ck * A.chunk2;
  const int i_max = min(w - 1, (A.row0 + (slab + 1) * kSlab - 1) / A.kv.G);
  if (L < w || Le <= 0 || k0 >= Le || (CHUNK && k0 > L - w + i_max)) return;
  // CHUNK: no row of the slab sees a key past L - w + i_max; those keys'
  // column sums are neither computed nor stored (the accumulation skips them)
  const int k1 = CHUNK ? min(min(Le, k0 + A.chunk2), L - w + i_max + 1) : min(Le, k0 + A.chunk2);
  const int tile0 = k0 >> 4, ntile = (k1 - k0 + 15) >> 4;

  C cx;
  cx.load_blocks(A, b, k0, k1, lane);
  cx.load_q(A, b, h, slab, rg, lane);
  // CHUNK: the last key each of this lane's rows sees (S layout: rows 4 * g + e)
  int lim[4][4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      lim[rb][e] = L - w + (A.row0 + slab * kSlab + rg * 64 + rb * 16 + 4 * g + e) / A.kv.G;
  // lse of this lane's rows (S layout: rows 4 * g + e of each block)
  float4_t nl[4];
  const float* lrow = A.lse + (size_t)u * A.n_slab * kSlab + slab * kSlab + rg * 64 + 4 * g;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) nl[rb] = -*reinterpret_cast<const float4_t*>(lrow + rb * 16);
  const float c = A.c;
  float* up = A.up + ((size_t)slab * A.kv.B * A.kv.Hkv + u) * cap;

  cx.sweep(A, buf0, buf1, h, tile0, ntile, wid, lane, [&](const unsigned char* buf, int s, int nq) {
    // software-pipelined as in the normaliser sweep
    auto update = [&](float4_t (&acc)[4], int q) {
      if (CHUNK) {
        const int key = (tile0 + s * kStage + q) * 16 + (lane & 15);
        if ((tile0 + s * kStage + q) * 16 + 15 > L - w) {   // the tile reaches the query range
#pragma unroll
          for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (key > lim[rb][e]) acc[rb][e] = -INFINITY;
        }
      }
      float sum = 0.f;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
        sum += (fast_exp2(fmaf(acc[rb][0], c, nl[rb][0])) + fast_exp2(fmaf(acc[rb][1], c, nl[rb][1]))) +
               (fast_exp2(fmaf(acc[rb][2], c, nl[rb][2])) + fast_exp2(fmaf(acc[rb][3], c, nl[rb][3])));
      sum = sum_rows4(sum);
      if (lane < 16) part[((s * kStage + q) * NRG + rg) * 16 + lane] = sum;
    };
    float4_t a0[4], a1[4];
    int q = kg;
    if (q < nq) C::tile_s(buf + q * TB, lane, cx.qop, a0);
    while (q < nq) {
      const int q1 = q + NKG;
      C::tile_s(buf + min(q1, nq - 1) * TB, lane, cx.qop, a1);
      update(a0, q);
      if (q1 >= nq) break;
      const int q2 = q1 + NKG;
      C::tile_s(buf + min(q2, nq - 1) * TB, lane, cx.qop, a0);
      update(a1, q1);
      q = q2;
    }
  });
  // Row groups summed in a fixed order, once per chunk: a store inside the
  // stage loop would be waited for with the next stage's loads.  Keys past the
  // earlier range are dropped.
  __syncthreads();
  for (int x = tid; x < k1 - k0; x += kThreads) {
    const int ti = x >> 4, t = x & 15;
    float v = part[(ti * NRG) * 16 + t];
#pragma unroll
    for (int r = 1; r < NRG; ++r) v += part[(ti * NRG + r) * 16 + t];
    up[k0 + x] = v;
  }
}

// ------------------------------------------------------------ pooling
__global__ void __launch_bounds__(kThreads) snap_pool_kernel(SnapArgs A) {
  __shared__ float su[kPoolOut + 2 * kMaxPoolHalf];
  const int u = blockIdx.y, tid = threadIdx.x;
  const int b = u / A.kv.Hkv;
  const int cap = A.kv.max_pages * A.kv.P;
  const int L = clamp_len(A.kv.seq_lens[b], cap);
  const int Le = L - A.w;
  const int j0 = blockIdx.x * kPoolOut;
  if (Le <= 0 || j0 >= Le) return;
  const int r = A.half;
  const size_t slab_stride = (size_t)A.kv.B * A.kv.Hkv * cap;
  const float* up = A.up + (size_t)u * cap;
  for (int x = tid; x < kPoolOut + 2 * r; x += kThreads) {
    const int j = j0 - r + x;
    float v = -INFINITY;
    if (j >= 0 && j < Le) {
      v = up[j];
      for (int sl = 1; sl < A.n_slab; ++sl) v += up[sl * slab_stride + j];
    }
    su[x] = v;
  }
  __syncthreads();
  float* out = A.scores + (size_t)u * A.slot_cap;
  for (int x = tid; x < kPoolOut; x += kThreads) {
    const int j = j0 + x;
    if (j < Le) {
      float mx = su[x];
      for (int d = 1; d <= 2 * r; ++d) mx = fmaxf(mx, su[x + d]);
      out[j] = j < A.n_sink ? INFINITY : mx;
    }
  }
}

// H2O prefill chunk: scores[j] = (j in the chunk and first pass ? 0 : scores[j])
// + the column sums of the pass's row slabs that have a row seeing slot j,
// for every slot j < L; slabs are added in ascending order.
__global__ void __launch_bounds__(kThreads) snap_accumulate_kernel(SnapArgs A) {
  const int u = blockIdx.y, b = u / A.kv.Hkv;
  const int cap = A.kv.max_pages * A.kv.P;
  const int L = clamp_len(A.kv.seq_lens[b], cap);
  const int j = blockIdx.x * kThreads + threadIdx.x;
  if (L < A.w || j >= L) return;
  const size_t slab_stride = (size_t)A.kv.B * A.kv.Hkv * cap;
  float add = 0.f;
  for (int sl = 0; sl < A.n_slab; ++sl) {
    // slab sl wrote the column sums of the keys its rows see: j <= L - w + i_max
    const int i_max = min(A.w - 1, (A.row0 + (sl + 1) * kSlab - 1) / A.kv.G);
    if (j <= L - A.w + i_max) add += A.up[sl * slab_stride + (size_t)u * cap + j];
  }
  float* srow = A.scores + (size_t)u * A.slot_cap;
  const float old = (A.first_pass && j >= L - A.w) ? 0.f : srow[j];
  srow[j] = old + add;
}

template <int D, int NRG, bool CHUNK>
hipError_t launch_sweeps(const SnapArgs& A, const SnapPlan& p, hipStream_t s) {
  const int units = A.kv.B * A.kv.Hkv;
  snap_lse_kernel<D, NRG><<<dim3(p.n_chunk1, A.n_slab, units), kThreads, 0, s>>>(A);
  snap_merge_kernel<<<dim3(A.n_slab, units), kMergeThreads, 0, s>>>(A);
  snap_score_kernel<D, NRG, CHUNK><<<dim3(p.n_chunk2, A.n_slab, units), kThreads, 0, s>>>(A);
  return hipGetLastError();
}

template <bool CHUNK>
hipError_t launch_sweeps_for(const SnapArgs& A, const SnapPlan& p, hipStream_t s) {
  if (A.kv.D == 64)
    return p.nrg == 1 ? launch_sweeps<64, 1, CHUNK>(A, p, s)
         : p.nrg == 2 ? launch_sweeps<64, 2, CHUNK>(A, p, s) : launch_sweeps<64, 4, CHUNK>(A, p, s);
  return p.nrg == 1 ? launch_sweeps<128, 1, CHUNK>(A, p, s)
       : p.nrg == 2 ? launch_sweeps<128, 2, CHUNK>(A, p, s) : launch_sweeps<128, 4, CHUNK>(A, p, s);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

SnapArgs make_args(const KVDev& kv, const SnapPlan& p, const void* q, int n_q, float scale, void* ws) {
  SnapArgs A{};
  A.kv = kv;
  A.q = static_cast<const bf16_t*>(q);
  A.w = n_q;
  A.R = kv.G * n_q;
  A.c = scale * 1.4426950408889634f;
  A.lp = kv.P == 32 ? 5 : 4;
  A.chunk1 = p.chunk1; A.n_chunk1 = p.n_chunk1;
  A.chunk2 = p.chunk2; A.n_chunk2 = p.n_chunk2;
  unsigned char* w = static_cast<unsigned char*>(ws);
  A.ml = reinterpret_cast<float2*>(w + p.ml_off);
  A.lse = reinterpret_cast<float*>(w + p.lse_off);
  A.up = reinterpret_cast<float*>(w + p.up_off);
  return A;
}

}  // namespace

SnapPlan plan_snapkv(const KVDev& kv, int n_obs) {
  SnapPlan p{};
  const long R = (long)kv.G * n_obs;
  const long slabs = (R + kSlab - 1) / kSlab;
  const long cap = (long)kv.max_pages * kv.P;
  const long units = (long)kv.B * kv.Hkv;
  // slabs per pass: every slab's column sums over the cache's capacity within
  // kPassBytes, and never fewer than kPassSlabs
  const long fit = (long)(kPassBytes / ((size_t)units * cap * sizeof(float)));
  const long per_pass = fit > kPassSlabs ? fit : kPassSlabs;
  p.n_slab = (int)(slabs < per_pass ? slabs : per_pass);
  p.n_pass = (int)((slabs + p.n_slab - 1) / p.n_slab);
  const long rows_slab = slabs == 1 ? R : kSlab;
  p.nrg = rows_slab <= 64 ? 1 : (rows_slab <= 128 ? 2 : 4);
  const long align = 128;             // chunks start on a page and a tile boundary
  auto chunking = [&](int& chunk, int& n_chunk) {
    long want = (kTargetWG + units * p.n_slab - 1) / (units * p.n_slab);
    long ck = (cap + want - 1) / want;
    ck = (ck + align - 1) / align * align;
    if (ck > kMaxChunk) ck = kMaxChunk;
    chunk = (int)ck;
    n_chunk = (int)((cap + ck - 1) / ck);
  };
  chunking(p.chunk1, p.n_chunk1);
  chunking(p.chunk2, p.n_chunk2);
  const size_t rows = (size_t)units * p.n_slab * kSlab;
  p.ml_off = 0;
  p.lse_off = align256(rows * p.n_chunk1 * sizeof(float2));
  p.up_off = p.lse_off + align256(rows * sizeof(float));
  p.ws_bytes = p.up_off + align256((size_t)p.n_slab * units * cap * sizeof(float));
  return p;
}

hipError_t launch_snapkv(const KVDev& kv, const SnapPlan& p, const void* q_obs, int n_obs,
                         float scale, int pool_kernel, int n_sink, float* scores, int slot_cap,
                         void* ws, hipStream_t s) {
  SnapArgs A = make_args(kv, p, q_obs, n_obs, scale, ws);
  A.mode = kModeWindow;
  A.row0 = 0;
  A.n_slab = p.n_slab;                 // one pass: G * n_obs <= kPassSlabs * kSlab rows
  A.first_pass = 1;
  A.scores = scores;
  A.slot_cap = slot_cap;
  A.half = pool_kernel / 2;
  A.n_sink = n_sink;
  hipError_t e = launch_sweeps_for<false>(A, p, s);
  if (e != hipSuccess) return e;
  const int cap = kv.max_pages * kv.P;
  snap_pool_kernel<<<dim3((cap + kPoolOut - 1) / kPoolOut, kv.B * kv.Hkv), kThreads, 0, s>>>(A);
  return hipGetLastError();
}

hipError_t launch_h2o_prefill_scores(const KVDev& kv, const SnapPlan& p, const void* q_chunk, int n_q,
                                     float scale, float* scores, int slot_cap, void* ws, hipStream_t s) {
  SnapArgs A = make_args(kv, p, q_chunk, n_q, scale, ws);
  A.mode = kModeChunk;
  A.scores = scores;
  A.slot_cap = slot_cap;
  const int cap = kv.max_pages * kv.P;
  const int slabs = (A.R + kSlab - 1) / kSlab;
  for (int pass = 0; pass < p.n_pass; ++pass) {
    A.row0 = pass * p.n_slab * kSlab;
    A.n_slab = min(p.n_slab, slabs - pass * p.n_slab);
    A.first_pass = pass == 0;
    hipError_t e = launch_sweeps_for<true>(A, p, s);
    if (e != hipSuccess) return e;
    snap_accumulate_kernel<<<dim3((cap + kThreads - 1) / kThreads, kv.B * kv.Hkv), kThreads, 0, s>>>(A);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

int snapkv_max_pool_kernel() { return 2 * kMaxPoolHalf + 1; }

}  // namespace spk
