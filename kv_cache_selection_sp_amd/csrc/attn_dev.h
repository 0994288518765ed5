// Device code of the paged decode attention (attn_kernel) as inline
// functions, shared by the attention launch and the fused decode step.  See
// k_attn.hip for the method, the work decomposition and the tile engines.
#pragma once
#include "lds_layout.h"
#include "sp_internal.h"

namespace spk {
namespace attndev {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kThreadsSmall = 256;   // workgroup sizes: 4 or 8 waves (chosen per call)
constexpr int kThreadsLarge = 512;
constexpr int kNumCU = 256;       // compute units of an MI355X
constexpr int kMinChunk = 8;      // fewest tiles given to one workgroup
constexpr int kTargetChunk = 64;  // preferred tiles per workgroup, while every CU keeps one
constexpr int kValuTasks = 8;     // (head, dim) outputs per thread: 16 * 128 / 256
constexpr int kMergeDirect = 4;   // up to this many records: one-pass merge in registers

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
constexpr int kRsrcFlags = 0x00020000;   // buffer resource word 3: raw 32-bit dwords
constexpr int kNonTemporal = 2;          // buffer load cache policy: non-temporal

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

struct AttnArgs {
  KVDev kv;
  const void* q;
  const int32_t* sel;   // NULL: dense mode
  const uint32_t* sel_mask;  // sparse mode, optional: per entry, bit t = token t of the page attended
  int top_k;
  float scale;
  float* out;
  float* lse;
  float* logits;
  int logit_cap;
  int n_wg;
  float* acc_scores;    // dense mode with logits, optional: H2O scores updated per unit
  int slot_cap;
  int n_new;
  int* counters;        // [units], zero between calls
  float* records;       // [n_wg + units][G][D + 2]
  // dense calls of more than kDenseLdsMax sequences: the tile prefix [B + 1]
  // and then the first sequence of each workgroup's range [n_wg], written by
  // dense_prefix_kernel before the attention
  const int* gpre = nullptr;
};

// The dynamic LDS layout (lds_layout, stage_bt) is in lds_layout.h.

// ============================================================== MFMA engine
template <int D, int P, bool LOGITS, int NT>
struct MfmaEngine {
  static constexpr bool kMfma = true;
  static constexpr bool kLogits = LOGITS;
  static constexpr int kThreads = NT;
  static constexpr int kWaves = NT / 64;
  static constexpr int KS = D / 32;   // 16x16x32 k-steps over the head dim
  static constexpr int NB = D / 16;   // 16-dim output tiles
  struct Buf {
    uint4 k[KS];                      // token `col`, 16-byte chunk 4ks+g
    uint2 v[NB];                      // dim 16nb+col, tokens 4g..4g+3
  };

  const bf16_t* kpool;
  const bf16_t* vpool;
  const int* lblk;
  const int* loff;
  const int* ltok;
  const int* lnv;
  float* wst;
  float* comb;
  int h, Hkv, G, lane, col, g, w;
  float scale, scale_log2;
  float* logit_head;                  // logits row of head `col` (LOGITS, col < G)
  bool coh_logits;                    // logits written through to the coherence point (split units)
  bool tok_mask = false;              // tiles carry token masks (selected tokens): skip the others' loads
  bf16x8_t qop[KS];
  float4_t o[NB];
  float m, l;

  __device__ void begin(const AttnArgs& A, int b, int hh) {
    h = hh;
    const bf16_t* q = static_cast<const bf16_t*>(A.q);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 u = {0u, 0u, 0u, 0u};
      if (col < G)
        u = *reinterpret_cast<const uint4*>(q + ((size_t)b * A.kv.Hq + h * G + col) * D + (4 * ks + g) * 8);
      qop[ks] = __builtin_bit_cast(bf16x8_t, u);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[nb] = float4_t{0.f, 0.f, 0.f, 0.f};
    m = -INFINITY;
    l = 0.f;
    logit_head = (LOGITS && col < G)
                     ? A.logits + ((size_t)b * A.kv.Hq + h * G + col) * A.logit_cap : nullptr;
  }

  // Loads of tile i of the list into bf.  The tile's K and V pages are
  // addressed through buffer resources built from wave-uniform page bases,
  // so every lane's offset is a constant.  A slot past the wave's last tile
  // (real == false) gets an empty resource: its loads return zeros without
  // touching memory, which keeps the number of loads in flight the same on
  // every path.  Non-temporal: every page is read once per call.  With
  // token masks (scattered selected tokens), a lane whose K token, or whose
  // four V tokens, are not selected loads from past the resource's end,
  // which also returns zeros without touching memory: such a token's K
  // chunks (16 bytes each, four tokens to a 64-byte line) are not fetched.
  // Its V shares 32-byte dim rows with the tile's other tokens, so V is
  // fetched whole for any selected token.
  __device__ __forceinline__ void issue(Buf& bf, int i, bool real) const {
    const int blk = __builtin_amdgcn_readfirstlane(lblk[i]);
    const int off = __builtin_amdgcn_readfirstlane(loff[i]);
    int kskip = 0, vskip = 0;
    if (tok_mask) {
      constexpr int kPast = 1 << 30;
      const unsigned vm = (unsigned)lnv[i];
      kskip = ((vm >> col) & 1u) ? 0 : kPast;
      vskip = ((vm >> (4 * g)) & 0xfu) ? 0 : kPast;
    }
    const size_t base = page_base(blk, h, Hkv, P, D);
    const int bytes = real ? P * D * 2 : 0;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(kpool + base), (short)0, bytes, kRsrcFlags);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(vpool + base), (short)0, bytes, kRsrcFlags);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      bf.k[ks] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                     rk, ((4 * ks + g) * P + col) * 16 + kskip, off * 16, kNonTemporal));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      bf.v[nb] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                     rv, ((16 * nb + col) * P + 4 * g) * 2 + vskip, off * 2, kNonTemporal));
  }

  __device__ __forceinline__ void process(const Buf& bf, int i) {
    const unsigned vm = (unsigned)lnv[i];      // tokens of the tile attended (bit t = token t)
    float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, bf.k[ks]), qop[ks],
                                                    acc, 0, 0, 0);
    float s[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = ((vm >> (4 * g + r)) & 1u) ? acc[r] * scale_log2 : -INFINITY;
    if constexpr (LOGITS) {
      if (logit_head != nullptr) {
        float* lr = logit_head + ltok[i] + 4 * g;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if ((vm >> (4 * g + r)) & 1u)
          {
            if (coh_logits)
              __hip_atomic_store(lr + r, acc[r] * scale, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else
              lr[r] = acc[r] * scale;
          }
      }
    }
    float mt = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m, mt);            // finite: the tile has a valid token
    const float alpha = fast_exp2(m - m_new);    // 0 on the first tile (m = -inf)
    m = m_new;
    float psum = 0.f;
    short4_t phi, plo;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = fast_exp2(s[r] - m_new);
      psum += p;
      const bf16_t hi = f32_to_bf16(p);
      phi[r] = (short)hi;
      plo[r] = (short)f32_to_bf16(p - to_f32(hi));
    }
    l = l * alpha + psum;
    // A tile with tokens left out (past the sequence's end, or not selected):
    // their slots may hold any bits, and a NaN or infinite V times p = 0
    // would still reach the output, so their V is zeroed.
    uint32_t vkeep0 = 0xffffffffu, vkeep1 = 0xffffffffu;
    if (__builtin_amdgcn_readfirstlane(vm) != 0xffffu) {
      const unsigned t4 = (vm >> (4 * g)) & 0xfu;
      vkeep0 = ((t4 & 1u) ? 0x0000ffffu : 0u) | ((t4 & 2u) ? 0xffff0000u : 0u);
      vkeep1 = ((t4 & 4u) ? 0x0000ffffu : 0u) | ((t4 & 8u) ? 0xffff0000u : 0u);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      o[nb] *= alpha;
      const short4_t va = __builtin_bit_cast(short4_t, make_uint2(bf.v[nb].x & vkeep0, bf.v[nb].y & vkeep1));
      o[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, phi, o[nb], 0, 0, 0);
      o[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, plo, o[nb], 0, 0, 0);
    }
  }

  // Wave w streams tiles w, w + kWaves, ... of the resolved list through a
  // ring of kRing register buffers: kRing - 1 tiles stay in flight while one
  // is processed.  Two are enough: a wider ring only lengthens the memory
  // queues (other requests of the same launch then wait behind them), and a
  // gather of the same tiles with two buffers per wave streams faster than
  // with three.  Every prefetch is issued unconditionally (past the end with
  // an empty resource, see issue), so the number of loads in flight is the
  // same on every path and each wait lets the younger tile stay queued.
  static constexpr int kRing = 2;
  __device__ void run(int cnt_in) {
    // wave-uniform values in scalar registers: the loop below is then a
    // scalar loop, which the wait-count analysis can follow
    const int cnt = __builtin_amdgcn_readfirstlane(cnt_in);
    if (w >= cnt) return;
    const int nw = (cnt - w + kWaves - 1) / kWaves;
    auto tile = [&](int j) { return j < nw ? w + j * kWaves : w; };
    // the scheduling barriers keep each stage where it is written, so the
    // buffers are filled in ring order and no third buffer is needed
    Buf b0, b1;
    issue(b0, tile(0), true);
    __builtin_amdgcn_sched_barrier(0);
    issue(b1, tile(1), nw > 1);
    __builtin_amdgcn_sched_barrier(0);
    for (int j = 0; j < nw; j += kRing) {
      process(b0, tile(j));
      __builtin_amdgcn_sched_barrier(0);
      issue(b0, tile(j + 2), j + 2 < nw);
      __builtin_amdgcn_sched_barrier(0);
      if (j + 1 < nw) process(b1, tile(j + 1));
      __builtin_amdgcn_sched_barrier(0);
      issue(b1, tile(j + 3), j + 3 < nw);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Combine the workgroup's wave states into comb (LDS).
  __device__ void finish() {
    constexpr int OSTR = D + 4;                      // rows 16-byte aligned for 4-float writes
    // l of this head summed over the four lane groups (lanes col, col + 16,
    // col + 32, col + 48): a row swap (swizzle) and a half swap (permute)
    float lsum = l;
    lsum += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(lsum), kSwizzleXor16));
    lsum += __shfl_xor(lsum, 32, 64);
    float* wo = wst;                                 // [w][a][OSTR]
    float* wm = wst + kWaves * G * OSTR;             // [w][a]
    float* wl = wm + kWaves * G;
    if (col < G) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        *reinterpret_cast<float4_t*>(wo + (w * G + col) * OSTR + 16 * nb + 4 * g) = o[nb];
      if (g == 0) {
        wm[w * G + col] = m;
        wl[w * G + col] = lsum;
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < G * D; i += kThreads) {
      const int a = i / D, d = i % D;
      // every wave's (m, l, acc) read at once, then combined without branches
      float mw[kWaves], lw[kWaves], ow[kWaves];
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        mw[ww] = wm[ww * G + a];
        lw[ww] = wl[ww * G + a];
        ow[ww] = wo[(ww * G + a) * OSTR + d];
      }
      float mstar = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) mstar = fmaxf(mstar, mw[ww]);
      float ov = 0.f, lv = 0.f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const float f = mw[ww] == -INFINITY ? 0.f : fast_exp2(mw[ww] - mstar);
        ov += f * ow[ww];
        lv += f * lw[ww];
      }
      comb[a * D + d] = ov;
      if (d == 0) {
        comb[G * D + a] = mstar;
        comb[G * D + G + a] = lv;
      }
    }
    __syncthreads();
  }
};

// ============================================================== VALU engine
template <typename T, int D, int P, bool LOGITS, int NT>
struct ValuEngine {
  static constexpr bool kMfma = false;
  static constexpr bool kLogits = LOGITS;
  static constexpr int kThreads = NT;
  static constexpr int kWaves = NT / 64;
  static constexpr int E = Chunk<T>::E;
  const T* kpool;
  const T* vpool;
  const int* lblk;
  const int* loff;
  const int* ltok;
  const int* lnv;
  float* wst;
  float* comb;
  int h, Hkv, G, lane, col, g, w;
  float scale, scale_log2;
  float* logit_rows;      // logits row of the group's first head (LOGITS)
  bool coh_logits;        // logits written through to the coherence point (split units)
  int logit_cap;
  float oacc[kValuTasks];

  // wst: qs[G][D], S[G][kTok + 1], m_run[G], l_run[G], alpha[G]
  __device__ float* qs() const { return wst; }
  __device__ float* S() const { return wst + G * D; }
  __device__ float* m_run() const { return wst + G * D + G * (kTok + 1); }
  __device__ float* l_run() const { return m_run() + G; }
  __device__ float* alph() const { return m_run() + 2 * G; }

  __device__ void begin(const AttnArgs& A, int b, int hh) {
    h = hh;
    const T* q = static_cast<const T*>(A.q);
    for (int i = threadIdx.x; i < G * D; i += kThreads)
      qs()[i] = to_f32(q[((size_t)b * A.kv.Hq + h * G) * D + i]);
    if ((int)threadIdx.x < G) {
      m_run()[threadIdx.x] = -INFINITY;
      l_run()[threadIdx.x] = 0.f;
    }
#pragma unroll
    for (int k = 0; k < kValuTasks; ++k) oacc[k] = 0.f;
    logit_cap = A.logit_cap;
    logit_rows = LOGITS ? A.logits + ((size_t)b * A.kv.Hq + h * G) * A.logit_cap : nullptr;
    __syncthreads();
  }

  __device__ void run(int cnt) {
    const int tid = threadIdx.x;
    constexpr int SS = kTok + 1;
    for (int i = 0; i < cnt; ++i) {
      const size_t base = page_base(lblk[i], h, Hkv, P, D);
      const T* kp = kpool + base;
      const T* vp = vpool + base;
      const int off = loff[i], tok0 = ltok[i];
      const unsigned vm = (unsigned)lnv[i];    // tokens of the tile attended (bit t = token t)
      for (int idx = tid; idx < G * kTok; idx += kThreads) {
        const int a = idx / kTok, t = idx % kTok;
        float z = -INFINITY;
        if ((vm >> t) & 1u) {
          float dot = 0.f;
          for (int c = 0; c < D / E; ++c) {
            union { uint4 u; T e[E]; } wv;
            wv.u = *reinterpret_cast<const uint4*>(kp + (size_t)(c * P + off + t) * E);
#pragma unroll
            for (int x = 0; x < E; ++x) dot = fmaf(qs()[a * D + c * E + x], to_f32(wv.e[x]), dot);
          }
          if constexpr (LOGITS)
          {
            float* lp = logit_rows + (size_t)a * logit_cap + tok0 + t;
            if (coh_logits) __hip_atomic_store(lp, dot * scale, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else *lp = dot * scale;
          }
          z = dot * scale_log2;
        }
        S()[a * SS + t] = z;
      }
      __syncthreads();
      if (tid < G) {
        float* Sa = S() + tid * SS;
        float mt = -INFINITY;
        for (int t = 0; t < kTok; ++t)
          if ((vm >> t) & 1u) mt = fmaxf(mt, Sa[t]);
        const float m_new = fmaxf(m_run()[tid], mt);
        const float al = fast_exp2(m_run()[tid] - m_new);
        float sum = 0.f;
        for (int t = 0; t < kTok; ++t) {
          const float p = ((vm >> t) & 1u) ? fast_exp2(Sa[t] - m_new) : 0.f;
          Sa[t] = p;
          sum += p;
        }
        l_run()[tid] = l_run()[tid] * al + sum;
        m_run()[tid] = m_new;
        alph()[tid] = al;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kValuTasks; ++k) {
        const int idx = tid + k * kThreads;
        if (idx < G * D) {
          const int a = idx / D, d = idx % D;
          const float* Sa = S() + a * SS;
          float ov = oacc[k] * alph()[a];
          const T* vrow = vp + (size_t)d * P + off;
          // the tile's kTok values of dim d, loaded together (all inside the
          // page); tokens left out are then skipped by a select, since their
          // slots may hold any bits and 0 * NaN would reach the output
          float vv[kTok];
#pragma unroll
          for (int t = 0; t < kTok; ++t) vv[t] = to_f32(vrow[t]);
#pragma unroll
          for (int t = 0; t < kTok; ++t) ov = ((vm >> t) & 1u) ? fmaf(Sa[t], vv[t], ov) : ov;
          oacc[k] = ov;
        }
      }
      __syncthreads();
    }
  }

  __device__ void finish() {
#pragma unroll
    for (int k = 0; k < kValuTasks; ++k) {
      const int idx = threadIdx.x + k * kThreads;
      if (idx < G * D) comb[idx] = oacc[k];
    }
    if ((int)threadIdx.x < G) {
      comb[G * D + threadIdx.x] = m_run()[threadIdx.x];
      comb[G * D + G + threadIdx.x] = l_run()[threadIdx.x];
    }
    __syncthreads();
  }
};

// The H2O score update of one (sequence b, KV head h) unit, by the workgroup
// that wrote its final lse: for slots j < L, the newest n_new start from
// zero, then s_j += sum over the group's heads a (in order) of
// exp(z_aj - lse_a).  The same expression, order and functions as
// h2o_accumulate_kernel, so both forms give identical scores.  Logits of the
// unit's other segments were stored through to the coherence point before
// their workgroups counted in, and are read the same way.
template <int NT>
__device__ __forceinline__ void accumulate_unit(const AttnArgs& A, int b, int h, int L, const float* s_lse,
                                                bool coherent) {
  constexpr int kMaxG = 16;
  constexpr int kHG = 8;                        // heads per load batch
  constexpr int kJ = 4;                         // slots per thread per batch, their loads issued together
  const KVDev& kv = A.kv;
  const int G = kv.G;
  const size_t ra0 = (size_t)b * kv.Hq + (size_t)h * G;
  float* srow = A.acc_scores + ((size_t)b * kv.Hkv + h) * A.slot_cap;
  auto ld = [&](const float* p) {
    return coherent ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : *p;
  };
  for (int j0 = 0; j0 < L; j0 += kJ * NT) {
    float s[kJ];
#pragma unroll
    for (int x = 0; x < kJ; ++x) {
      const int j = j0 + x * NT + (int)threadIdx.x;
      s[x] = (j >= L - A.n_new) ? 0.f : srow[min(j, L - 1)];
    }
    // the heads in order, eight at a time: the same additions in the same
    // order as the separate kernel
    for (int a0 = 0; a0 < G; a0 += kHG) {
      float z[kJ][kHG];
#pragma unroll
      for (int x = 0; x < kJ; ++x) {
        const int jc = min(j0 + x * NT + (int)threadIdx.x, L - 1);
#pragma unroll
        for (int aa = 0; aa < kHG; ++aa)
          z[x][aa] = a0 + aa < G ? ld(A.logits + (ra0 + a0 + aa) * A.logit_cap + jc) : 0.f;
      }
#pragma unroll
      for (int x = 0; x < kJ; ++x)
#pragma unroll
        for (int aa = 0; aa < kHG; ++aa)
          if (a0 + aa < G) s[x] += expf(z[x][aa] - s_lse[a0 + aa]);
    }
#pragma unroll
    for (int x = 0; x < kJ; ++x) {
      const int j = j0 + x * NT + (int)threadIdx.x;
      if (j < L) srow[j] = s[x];
    }
  }
  (void)kMaxG;
}

// ============================================================== kernel
template <typename Engine, int D, int P, typename T>
__device__ __forceinline__ void attn_block(const AttnArgs& A, const int wg) {
  constexpr int kThreads = Engine::kThreads;
  constexpr int kWaves = Engine::kWaves;
  extern __shared__ __align__(16) int smem[];
  __shared__ int wsum[kWaves + 1];
  __shared__ int s_last;
  __shared__ float s_lse[16];                  // the unit's lse per query head (fused H2O update)
  constexpr int TPP = P / kTok;                 // tiles per page
  const KVDev& kv = A.kv;
  const int G = kv.G, Hkv = kv.Hkv, B = kv.B, Hq = kv.Hq;
  const int tid = threadIdx.x;
  const bool sparse = A.sel != nullptr;
  const int cap = kv.max_pages * P;
  const int* gpre = A.gpre;                      // dense, more than kDenseLdsMax sequences
  const LdsLayout lay = lds_layout(gpre ? 0 : B, G, D, sparse, Engine::kMfma, kWaves, kv.max_pages);
  const bool lbt_on = stage_bt(sparse, kv.max_pages);
  int* lbt = smem + lay.lbt;                    // sparse: block-table row of the unit's sequence
  int* pre = smem + lay.pre;
  int* lens = smem + lay.lens;                  // dense: clamped lengths
  int* lblk = smem + lay.lblk;
  int* loff = smem + lay.loff;
  int* ltok = smem + lay.ltok;
  int* lnv = smem + lay.lnv;
  float* comb = reinterpret_cast<float*>(smem + lay.comb);

  // ---- tile totals (dense: per-sequence prefix, unit-major)
  const int tpu_sparse = A.top_k * TPP;
  int total;
  if (sparse) {
    total = B * Hkv * tpu_sparse;
  } else if (gpre) {
    total = gpre[B];
    for (int b = wg; b < B; b += A.n_wg) {
      if (gpre[b + 1] != gpre[b]) continue;
      for (int i = tid; i < Hq * D; i += kThreads) A.out[(size_t)b * Hq * D + i] = 0.f;
      if (A.lse != nullptr)
        for (int i = tid; i < Hq; i += kThreads) A.lse[(size_t)b * Hq + i] = -INFINITY;
    }
  } else {
    int carry = 0;
    for (int base = 0; base < B; base += kThreads) {
      const int b = base + tid;
      const int Lb = b < B ? clamp_len(kv.seq_lens[b], cap) : 0;
      const int t = Hkv * ((Lb + kTok - 1) / kTok);
      int tot;
      const int ex = block_exclusive_scan<kThreads>(t, wsum, &tot);
      if (b < B) { pre[b] = carry + ex; lens[b] = Lb; }
      carry += tot;
    }
    if (tid == 0) pre[B] = carry;
    __syncthreads();
    total = carry;
    // sequences without slots: zero output, lse = -inf
    for (int b = wg; b < B; b += A.n_wg) {
      if (pre[b + 1] != pre[b]) continue;
      for (int i = tid; i < Hq * D; i += kThreads) A.out[(size_t)b * Hq * D + i] = 0.f;
      if (A.lse != nullptr)
        for (int i = tid; i < Hq; i += kThreads) A.lse[(size_t)b * Hq + i] = -INFINITY;
    }
  }
  // chunk: the split over n_wg, raised toward kTargetChunk tiles as long as
  // that still gives every CU a workgroup (fewer, longer workgroups pay the
  // per-workgroup start-up and merge latency fewer times)
  int chunk = (total + A.n_wg - 1) / A.n_wg;
  const int per_cu = (total + kNumCU - 1) / kNumCU;
  const int want = per_cu < kTargetChunk ? per_cu : kTargetChunk;
  if (chunk < want) chunk = want;
  if (chunk < kMinChunk) chunk = kMinChunk;
  const int c0 = wg * chunk;
  if (c0 >= total) return;
  const int c1 = min(c0 + chunk, total);

  Engine eng;
  eng.kpool = reinterpret_cast<const T*>(kv.k_pool);
  eng.vpool = reinterpret_cast<const T*>(kv.v_pool);
  eng.lblk = lblk; eng.loff = loff; eng.ltok = ltok; eng.lnv = lnv;
  if constexpr (Engine::kMfma) eng.tok_mask = A.sel_mask != nullptr;
  eng.wst = reinterpret_cast<float*>(smem + lay.wst);
  eng.comb = comb;
  eng.Hkv = Hkv; eng.G = G;
  eng.lane = tid & 63; eng.col = eng.lane & 15; eng.g = eng.lane >> 4;
  eng.w = __builtin_amdgcn_readfirstlane(tid >> 6);
  eng.scale = A.scale;
  eng.scale_log2 = A.scale * kLog2e;

  // dense from the workspace prefix: the sequence holding the current tile,
  // walked forward from the range's first
  int gb = gpre ? gpre[B + 1 + wg] : 0;
  auto len_of = [&](int b) { return gpre ? clamp_len(kv.seq_lens[b], cap) : lens[b]; };
  for (int c = c0; c < c1;) {
    // unit holding tile c
    int b, h, start, n;
    if (sparse) {
      const int u = c / tpu_sparse;
      b = u / Hkv; h = u % Hkv; start = u * tpu_sparse; n = tpu_sparse;
    } else if (gpre) {
      while (gpre[gb + 1] <= c) ++gb;
      b = gb;
      const int p0 = gpre[b];
      const int tb = (gpre[b + 1] - p0) / Hkv;
      h = (c - p0) / tb;
      start = p0 + h * tb;
      n = tb;
    } else {
      int lo = 0, hi = B - 1;                   // last b with pre[b] <= c
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= c) lo = mid; else hi = mid - 1;
      }
      b = lo;
      const int tb = (pre[b + 1] - pre[b]) / Hkv;
      h = (c - pre[b]) / tb;
      start = pre[b] + h * tb;
      n = tb;
    }
    const int L_dense = sparse ? 0 : len_of(b);
    // Every workgroup streams exactly its range: a unit inside the range is
    // handled whole, a unit crossing a range boundary is split along the
    // ranges and merged.
    const bool whole = start >= c0 && start + n <= c1;
    if (whole && start < c0) {                  // started in the previous range
      c = start + n;
      continue;
    }
    const int seg_end = whole ? start + n : min(c1, start + n);
    const int u = b * Hkv + h;
    const int32_t* sel_row = sparse ? A.sel + (size_t)u * A.top_k : nullptr;
    const uint32_t* msk_row = (sparse && A.sel_mask) ? A.sel_mask + (size_t)u * A.top_k : nullptr;
    const int32_t* bt_row = kv.block_table + (size_t)b * kv.max_pages;

    // Sparse: the first resolution pass's selection entries (and token
    // masks) and the sequence length are loaded ahead of q and the
    // block-table row, and one wait covers them all, so the tile list costs
    // a single round trip.  Later passes (segments above kThreads tiles)
    // load their entries in the loop; the length does not change.
    const int t_first = c - start;
    int pf_page = 0, L_seq = 0;
    uint32_t pf_msk = 0xffffffffu;
    if (sparse) {
      const int t_end1 = min(seg_end - start, t_first + kList);
      const int ti_c = min(t_first + tid, t_end1 - 1);
      pf_page = sel_row[ti_c / TPP];
      if (msk_row) pf_msk = msk_row[ti_c / TPP];
      L_seq = kv.seq_lens[b];
    }
    eng.begin(A, b, h);
    // a split unit's logits are read by the workgroup that merges it, which
    // may sit on another XCD; a whole unit's only by this workgroup
    eng.coh_logits = !whole;
    if (lbt_on) {
      // the block-table row, copied into LDS by direct loads
      const int wv = tid >> 6, ln = tid & 63;
      for (int i = wv * 64; i < kv.max_pages; i += kThreads)
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(bt_row + min(i + ln, kv.max_pages - 1)),
                                         (__attribute__((address_space(3))) void*)(lbt + i), 4, 0, 0);
    }
    if (sparse) {
      __builtin_amdgcn_s_waitcnt(0);            // entries, length, q and the staged row
      // the loaded values are first used here: a use scheduled next to its
      // load (a readfirstlane of the length, the mask's low half) would
      // wait for that load on its own
      asm volatile("" : "+v"(pf_page), "+v"(pf_msk), "+v"(L_seq));
      __syncthreads();
      L_seq = clamp_len(L_seq, cap);
    }
    for (int t_lo = t_first; t_lo < seg_end - start; t_lo += kList) {
      const int t_hi = min(seg_end - start, t_lo + kList);
      // resolve tiles [t_lo, t_hi) of the unit, keeping the valid ones in order
      int cnt = 0;
      for (int base = t_lo; base < t_hi; base += kThreads) {
        const int ti = base + tid;
        const int ti_c = ti < t_hi ? ti : t_hi - 1;
        const int entry = ti_c / TPP, half = ti_c % TPP;
        int page = entry, L;
        uint32_t msk = 0xffffffffu;
        int blk = -1, tok0 = 0, nv = 0;
        if (sparse) {
          L = L_seq;
          if (base == t_first) {
            page = pf_page;
            msk = pf_msk;
          } else {
            page = sel_row[entry];
            if (msk_row) msk = msk_row[entry];
          }
        } else {
          L = L_dense;
        }
        const int n_pages = (L + P - 1) / P;
        if (ti < t_hi) {
          if (page >= 0 && page < n_pages) {
            tok0 = page * P + half * kTok;
            nv = min(kTok, L - tok0);
            // distinct load forms keep the LDS read a ds_read (merged into
            // one load of a selected pointer it would be a flat load)
            if (lbt_on) blk = lbt[page];
            else blk = __hip_atomic_load(bt_row + page, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (blk < 0 || blk >= kv.num_blocks) nv = 0;
          }
        }
        uint32_t vm = nv > 0 ? ((1u << nv) - 1u) : 0u;
        vm &= (msk >> (half * kTok)) & 0xffffu;
        const int ok = vm != 0 ? 1 : 0;
        int tot;
        const int pos = cnt + block_exclusive_scan<kThreads>(ok, wsum, &tot);
        if (ok) {
          lblk[pos] = blk;
          loff[pos] = tok0 % P;
          ltok[pos] = tok0;
          lnv[pos] = (int)vm;
        }
        cnt += tot;
      }
      __syncthreads();
      eng.run(cnt);
      __syncthreads();
    }
    eng.finish();

    // ---- epilogue: comb holds the workgroup's state for unit u
    const int wg_first = start / chunk, wg_last = whole ? wg_first : (start + n - 1) / chunk;
    const size_t rec_len = (size_t)G * (D + 2);
    if (wg_first == wg_last) {
      for (int i = tid; i < G * D; i += kThreads) {
        const float lv = comb[G * D + G + i / D];
        A.out[((size_t)b * Hq + h * G) * D + i] = lv > 0.f ? comb[i] / lv : 0.f;
      }
      if (A.lse != nullptr && tid < G) {
        const float lv = comb[G * D + G + tid];
        const float lz = lv > 0.f ? (comb[G * D + tid] + log2f(lv)) * kLn2 : -INFINITY;
        A.lse[(size_t)b * Hq + h * G + tid] = lz;
        s_lse[tid] = lz;
      }
      if constexpr (Engine::kLogits) {
        if (A.acc_scores != nullptr) {
          __syncthreads();
          accumulate_unit<kThreads>(A, b, h, L_dense, s_lse, !whole);
        }
      }
    } else {
      // Publish the record with device-scope stores (written through to the
      // point of coherence of all XCDs) and wait for them to complete before
      // counting in; the merging workgroup reads records with device-scope
      // loads.  Only the record and counter lines are synchronised, so no
      // L2 writeback or invalidation is needed.
      float* rec = A.records + (size_t)(wg + u) * rec_len;
      for (int i = tid; i < G * (D + 2); i += kThreads)
        __hip_atomic_store(rec + i, comb[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) s_last = atomicAdd(&A.counters[u], 1) == wg_last - wg_first;
      __syncthreads();
      auto rd = [&](int x, int i) {
        return __hip_atomic_load(A.records + (size_t)(x + u) * rec_len + i, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      };
      const int n_rec = wg_last + 1 - wg_first;
      if (s_last && n_rec <= kMergeDirect) {
        // Few records: every thread loads (m, l, acc) of all records for its
        // outputs at once (one round trip) and combines them in workgroup
        // order in registers.
        for (int i = tid; i < G * D; i += kThreads) {
          const int a = i / D;
          float mx[kMergeDirect], lx[kMergeDirect], ox[kMergeDirect];
#pragma unroll
          for (int x = 0; x < kMergeDirect; ++x) {
            if (x < n_rec) {
              mx[x] = rd(wg_first + x, G * D + a);
              lx[x] = rd(wg_first + x, G * D + G + a);
              ox[x] = rd(wg_first + x, i);
            }
          }
          float mstar = -INFINITY;
#pragma unroll
          for (int x = 0; x < kMergeDirect; ++x)
            if (x < n_rec) mstar = fmaxf(mstar, mx[x]);
          float ov = 0.f, lv = 0.f;
          if (mstar != -INFINITY) {
#pragma unroll
            for (int x = 0; x < kMergeDirect; ++x) {
              if (x < n_rec && mx[x] != -INFINITY) {
                const float f = fast_exp2(mx[x] - mstar);
                ov += f * ox[x];
                lv += f * lx[x];
              }
            }
          }
          A.out[((size_t)b * Hq + h * G) * D + i] = lv > 0.f ? ov / lv : 0.f;
          if (A.lse != nullptr && i % D == 0) {
            const float lz = lv > 0.f ? (mstar + log2f(lv)) * kLn2 : -INFINITY;
            A.lse[(size_t)b * Hq + h * G + a] = lz;
            s_lse[a] = lz;
          }
        }
        if (tid == 0) __hip_atomic_store(&A.counters[u], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if constexpr (Engine::kLogits) {
          if (A.acc_scores != nullptr) {
            __syncthreads();
            accumulate_unit<kThreads>(A, b, h, L_dense, s_lse, !whole);
          }
        }
      } else if (s_last) {
        // Merge the unit's records in workgroup order, kMergeBatch at a time:
        // (m, l) of the batch into LDS in one parallel pass, per-head
        // weights, then independent loads of the accumulators.
        float* mrg = reinterpret_cast<float*>(smem + lay.mrg);
        float* bm = mrg;                               // [kMergeBatch][G] m, then weights
        float* bl = mrg + kMergeBatch * G;             // [kMergeBatch][G] l
        float* m_run = mrg + 2 * kMergeBatch * G;      // [G]
        float* l_run = m_run + G;                      // [G]
        float* alpha = l_run + G;                      // [G]
        // comb (already published in this workgroup's record) becomes the
        // accumulator
        if (tid < G) { m_run[tid] = -INFINITY; l_run[tid] = 0.f; }
        for (int i = tid; i < G * D; i += kThreads) comb[i] = 0.f;
        for (int xb = wg_first; xb <= wg_last; xb += kMergeBatch) {
          const int nb = min(kMergeBatch, wg_last + 1 - xb);
          for (int i = tid; i < nb * G; i += kThreads) {
            bm[i] = rd(xb + i / G, G * D + i % G);
            bl[i] = rd(xb + i / G, G * D + G + i % G);
          }
          __syncthreads();
          if (tid < G) {
            float mb = -INFINITY;
            for (int x = 0; x < nb; ++x) mb = fmaxf(mb, bm[x * G + tid]);
            const float m_new = fmaxf(m_run[tid], mb);
            const float al = m_new == -INFINITY ? 1.f : fast_exp2(m_run[tid] - m_new);
            float lv = l_run[tid] * al;
            for (int x = 0; x < nb; ++x) {
              const float mx = bm[x * G + tid];
              const float f = mx == -INFINITY ? 0.f : fast_exp2(mx - m_new);
              bm[x * G + tid] = f;
              lv += f * bl[x * G + tid];
            }
            m_run[tid] = m_new;
            l_run[tid] = lv;
            alpha[tid] = al;
          }
          __syncthreads();
          for (int i = tid; i < G * D; i += kThreads) {
            const int a = i / D;
            float ov = comb[i] * alpha[a];
#pragma unroll 8
            for (int x = 0; x < nb; ++x) ov += bm[x * G + a] * rd(xb + x, i);
            comb[i] = ov;
          }
          __syncthreads();
        }
        for (int i = tid; i < G * D; i += kThreads) {
          const float lv = l_run[i / D];
          A.out[((size_t)b * Hq + h * G) * D + i] = lv > 0.f ? comb[i] / lv : 0.f;
        }
        if (A.lse != nullptr && tid < G) {
          const float lv = l_run[tid];
          const float lz = lv > 0.f ? (m_run[tid] + log2f(lv)) * kLn2 : -INFINITY;
          A.lse[(size_t)b * Hq + h * G + tid] = lz;
          s_lse[tid] = lz;
        }
        if (tid == 0) __hip_atomic_store(&A.counters[u], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if constexpr (Engine::kLogits) {
          if (A.acc_scores != nullptr) {
            __syncthreads();
            accumulate_unit<kThreads>(A, b, h, L_dense, s_lse, !whole);
          }
        }
      }
    }
    __syncthreads();
    c = seg_end;
  }
}

// ============================================================== fused step
// Attention phase of the fused Quest decode step.  The n workgroups that
// scored unit u attend over its selected tiles, workgroup c taking tiles
// [c * T / n, (c + 1) * T / n) of the unit's T = top_k * P / 16.
//  * Descriptors come from the unit's top-k workgroup of the same launch,
//    each tagged with the unit's epoch of this call; a workgroup polls its
//    descriptors until every one carries the epoch (a bounded wait).
//  * Split states: each workgroup writes its (m, l, acc) record and then the
//    record's tag (the epoch) through to the point of coherence, waits until
//    the tags of the unit's other records carry the epoch, and merges its
//    1/n share of the unit's output from all n records in workgroup order.
//    No arrival counter is needed, and the epochs leave nothing to reset for
//    the next call.
struct FusedAttnArgs {
  KVDev kv;
  const void* q;
  int top_k;
  float scale;
  float* out;
  float* lse;
  const uint64_t* desc;   // [units][top_k] (epoch << 32) | (block id << 6 | tokens), all ones: none
  float* records;         // [units][n][G][D + 2]
  uint32_t* tags;         // [units][n]
  int* err;               // set to 1 if a wait gave up
};

// Bounded waits of the fused step: about a second of polling before a wait
// gives up (it cannot time out while the launch is co-resident).
constexpr int kSpinMax = 1 << 20;

template <typename Engine, int D, int P, typename T>
__device__ __forceinline__ void fused_attend(const FusedAttnArgs& F, const int u, const int c, const int n,
                                             const uint32_t epoch) {
  constexpr int kThreads = Engine::kThreads;
  constexpr int kWaves = Engine::kWaves;
  constexpr int TPP = P / kTok;
  extern __shared__ __align__(16) int smem[];
  __shared__ int fwsum[kWaves + 1];
  const KVDev& kv = F.kv;
  const int G = kv.G, Hkv = kv.Hkv, Hq = kv.Hq;
  const int tid = threadIdx.x;
  const int b = u / Hkv, h = u % Hkv;
  const int n_tiles = F.top_k * TPP;
  const int t0 = (int)((long)c * n_tiles / n), t1 = (int)((long)(c + 1) * n_tiles / n);
  const LdsLayout lay = lds_layout(1, G, D, true, Engine::kMfma, kWaves, kv.max_pages, true);
  int* lblk = smem + lay.lblk;
  int* loff = smem + lay.loff;
  int* ltok = smem + lay.ltok;
  int* lnv = smem + lay.lnv;
  float* comb = reinterpret_cast<float*>(smem + lay.comb);
  const uint64_t* drow = F.desc + (size_t)u * F.top_k;

  AttnArgs A;
  A.kv = kv;
  A.q = F.q;
  A.logits = nullptr;
  A.logit_cap = 0;
  Engine eng;
  eng.kpool = reinterpret_cast<const T*>(kv.k_pool);
  eng.vpool = reinterpret_cast<const T*>(kv.v_pool);
  eng.lblk = lblk; eng.loff = loff; eng.ltok = ltok; eng.lnv = lnv;
  eng.wst = reinterpret_cast<float*>(smem + lay.wst);
  eng.comb = comb;
  eng.Hkv = Hkv; eng.G = G;
  eng.lane = tid & 63; eng.col = eng.lane & 15; eng.g = eng.lane >> 4;
  eng.w = __builtin_amdgcn_readfirstlane(tid >> 6);
  eng.scale = F.scale;
  eng.scale_log2 = F.scale * kLog2e;
  eng.begin(A, b, h);
  eng.coh_logits = false;

  for (int t_lo = t0; t_lo < t1; t_lo += kList) {
    const int t_hi = min(t1, t_lo + kList);
    int cnt = 0;
    for (int base = t_lo; base < t_hi; base += kThreads) {
      const int ti = base + tid;
      const bool mine = ti < t_hi;
      const uint64_t* dp = drow + (mine ? ti : t_hi - 1) / TPP;
      uint64_t d = __hip_atomic_load(dp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int it = 0;; ++it) {
        const int ok = !mine || (uint32_t)(d >> 32) == epoch;
        if (__syncthreads_and(ok)) break;
        if (it >= kSpinMax) {
          if (tid == 0) __hip_atomic_store(F.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
        if (!ok) d = __hip_atomic_load(dp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      const uint32_t dd = (uint32_t)d;
      const int half = (mine ? ti : 0) % TPP;
      int blk = -1, nv = 0;
      if (mine && dd != 0xffffffffu && (uint32_t)(d >> 32) == epoch) {
        blk = (int)(dd >> 6);
        nv = min(kTok, (int)(dd & 63u) - half * kTok);
        if (blk >= kv.num_blocks) nv = 0;
      }
      const uint32_t vm = nv > 0 ? ((1u << nv) - 1u) : 0u;
      const int ok = vm != 0 ? 1 : 0;
      int tot;
      const int pos = cnt + block_exclusive_scan<kThreads>(ok, fwsum, &tot);
      if (ok) {
        lblk[pos] = blk;
        loff[pos] = half * kTok;
        ltok[pos] = 0;
        lnv[pos] = (int)vm;
      }
      cnt += tot;
    }
    __syncthreads();
    eng.run(cnt);
    __syncthreads();
  }
  eng.finish();                                   // comb: acc [G][D], m [G], l [G]

  float* out = F.out + ((size_t)b * Hq + h * G) * D;
  float* lse = F.lse != nullptr ? F.lse + (size_t)b * Hq + h * G : nullptr;
  if (n == 1) {
    for (int i = tid; i < G * D; i += kThreads) {
      const float lv = comb[G * D + G + i / D];
      out[i] = lv > 0.f ? comb[i] / lv : 0.f;
    }
    if (lse != nullptr && tid < G) {
      const float lv = comb[G * D + G + tid];
      lse[tid] = lv > 0.f ? (comb[G * D + tid] + log2f(lv)) * kLn2 : -INFINITY;
    }
    return;
  }
  const size_t rec_len = (size_t)G * (D + 2);
  float* rec = F.records + ((size_t)u * n + c) * rec_len;
  for (int i = tid; i < G * (D + 2); i += kThreads)
    __hip_atomic_store(rec + i, comb[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);                  // the record is at the point of coherence
  __syncthreads();
  if (tid == 0) __hip_atomic_store(F.tags + (size_t)u * n + c, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Second half of the attention phase: once the tags of all n records of unit
// u carry the epoch (a bounded wait), workgroup c merges its share of the
// unit's output.  Nothing to do for an unsplit unit (n == 1: written by
// fused_attend).
template <typename Engine, int D>
__device__ __forceinline__ void fused_merge(const FusedAttnArgs& F, const int u, const int c, const int n,
                                            const uint32_t epoch) {
  constexpr int kThreads = Engine::kThreads;
  if (n == 1) return;
  extern __shared__ __align__(16) int smem[];
  const KVDev& kv = F.kv;
  const int G = kv.G, Hkv = kv.Hkv, Hq = kv.Hq;
  const int tid = threadIdx.x;
  const int b = u / Hkv, h = u % Hkv;
  const LdsLayout lay = lds_layout(1, G, D, true, Engine::kMfma, Engine::kWaves, kv.max_pages, true);
  float* comb = reinterpret_cast<float*>(smem + lay.comb);
  float* out = F.out + ((size_t)b * Hq + h * G) * D;
  float* lse = F.lse != nullptr ? F.lse + (size_t)b * Hq + h * G : nullptr;
  const size_t rec_len = (size_t)G * (D + 2);
  const uint32_t* tags = F.tags + (size_t)u * n;
  for (int it = 0;; ++it) {
    int ok = 1;
    for (int x = tid; x < n; x += kThreads)
      ok &= __hip_atomic_load(tags + x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch ? 1 : 0;
    if (__syncthreads_and(ok)) break;
    if (it >= kSpinMax) {
      if (tid == 0) __hip_atomic_store(F.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  // Workgroup c merges elements [e0, e1) of the unit's G x D output (and the
  // lse of every head whose first element it holds) from all n records, in
  // workgroup order, kMergeBatch records at a time: (m, l) of the batch's
  // heads into LDS, per-head weights, then independent loads of the
  // accumulators.  comb, already published in this workgroup's record,
  // becomes the accumulator of the range.
  const int ge = G * D;
  const int e0 = (int)((long)c * ge / n), e1 = (int)((long)(c + 1) * ge / n);
  if (e0 >= e1) return;
  const int a0 = e0 / D, na = (e1 - 1) / D - a0 + 1;   // heads of the range
  const float* recs = F.records + (size_t)u * n * rec_len;
  auto rd = [&](int x, int i) {
    return __hip_atomic_load(recs + (size_t)x * rec_len + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  float* mrg = reinterpret_cast<float*>(smem + lay.mrg);
  float* bm = mrg;                               // [kMergeBatch][na] m, then weights
  float* bl = mrg + kMergeBatch * na;            // [kMergeBatch][na] l
  float* m_run = mrg + 2 * kMergeBatch * G;      // [na]
  float* l_run = m_run + G;                      // [na]
  float* alpha = l_run + G;                      // [na]
  // the accumulators of this thread's first element in the first kPre
  // records, loaded with the first batch's (m, l) instead of after the two
  // barriers that turn those into weights: one round trip at the end of the
  // step instead of two
  constexpr int kPre = 8;
  const int i_pre = e0 + tid;
  float pre[kPre];
#pragma unroll
  for (int x = 0; x < kPre; ++x) pre[x] = (x < n && i_pre < e1) ? rd(x, i_pre) : 0.f;
  if (tid < na) { m_run[tid] = -INFINITY; l_run[tid] = 0.f; }
  for (int i = e0 + tid; i < e1; i += kThreads) comb[i - e0] = 0.f;
  for (int xb = 0; xb < n; xb += kMergeBatch) {
    const int nb = min(kMergeBatch, n - xb);
    for (int i = tid; i < nb * na; i += kThreads) {
      bm[i] = rd(xb + i / na, ge + a0 + i % na);
      bl[i] = rd(xb + i / na, ge + G + a0 + i % na);
    }
    __syncthreads();
    if (tid < na) {
      float mb = -INFINITY;
      for (int x = 0; x < nb; ++x) mb = fmaxf(mb, bm[x * na + tid]);
      const float m_new = fmaxf(m_run[tid], mb);
      const float al = m_new == -INFINITY ? 1.f : fast_exp2(m_run[tid] - m_new);
      float lv = l_run[tid] * al;
      for (int x = 0; x < nb; ++x) {
        const float mx = bm[x * na + tid];
        const float f = mx == -INFINITY ? 0.f : fast_exp2(mx - m_new);
        bm[x * na + tid] = f;
        lv += f * bl[x * na + tid];
      }
      m_run[tid] = m_new;
      l_run[tid] = lv;
      alpha[tid] = al;
    }
    __syncthreads();
    for (int i = e0 + tid; i < e1; i += kThreads) {
      const int a = i / D - a0;
      float ov = comb[i - e0] * alpha[a];
      int x0 = 0;
      if (xb == 0 && i == i_pre) {               // records 0 .. kPre - 1 from registers, same order
#pragma unroll
        for (int x = 0; x < kPre; ++x)
          if (x < nb) ov += bm[x * na + a] * pre[x];
        x0 = kPre;
      }
#pragma unroll 8
      for (int x = x0; x < nb; ++x) ov += bm[x * na + a] * rd(xb + x, i);
      comb[i - e0] = ov;
    }
    __syncthreads();
  }
  for (int i = e0 + tid; i < e1; i += kThreads) {
    const float lv = l_run[i / D - a0];
    out[i] = lv > 0.f ? comb[i - e0] / lv : 0.f;
  }
  if (lse != nullptr && tid < na && (a0 + tid) * D >= e0) {
    const float lv = l_run[tid];
    lse[a0 + tid] = lv > 0.f ? (m_run[tid] + log2f(lv)) * kLn2 : -INFINITY;
  }
}

}  // namespace attndev
}  // namespace spk
