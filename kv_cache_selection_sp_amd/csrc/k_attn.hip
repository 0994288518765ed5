// Split-K paged decode attention over selected pages (Quest) or all occupied
// slots (dense: H2O, evicted decode), plus the split merge.
//
// "SparseEngine: Sparse-First Inference Engine", Appendix A.1, "Attention over
// Selected Positions": attention over a nonempty selected set normalises over
// the selected positions only, dense decode being the full set; Appendix A.3,
// "Quest": attention uses the actual KV of the selected pages; Appendix A.1,
// "MHA, MQA, and GQA": query head a reads KV head a / G.
//
// Work unit: (sequence b, KV head h, split s).  A split covers pages_per_split
// consecutive entries of the page list (selection entries in Quest mode, logical
// pages in dense mode) and produces, for each of the G query heads of h, a
// partial softmax state (m, l, acc[D]) in the log2 domain:
//   m = max_j s_j,  l = sum_j 2^(s_j - m),  acc = sum_j 2^(s_j - m) v_j,
//   s_j = log2(e) * scale * (q . k_j).
// The merge combines the splits of a query head in fixed split order (so the
// result is deterministic) and writes out = acc / l and lse = ln 2 * (m + log2 l).
//
// Two kernels produce the partials:
//   * MFMA (bf16, G >= 2): the G heads sharing a KV head form a real
//     contraction.  Per 16-token tile, S^T[16 tok x 16 heads] = K . Q^T with
//     v_mfma_f32_16x16x32_bf16 (heads padded to 16), then O^T[16 dims x 16 heads]
//     += V^T . P^T with v_mfma_f32_16x16x16_bf16, P split into bf16 hi + lo so
//     the product keeps ~16 mantissa bits.  With tokens as the M dimension the
//     S^T accumulator lane layout (lane = head column, 4 tokens per lane group)
//     is exactly the B-operand layout PV needs, and the per-head running max
//     lives in the same lane column as that head's output accumulator, so the
//     online-softmax rescale needs no cross-lane traffic.  The chunk-tiled K
//     page and dim-major V page make every operand load a contiguous 1 KB
//     (K, dwordx4) or 512 B (V, dwordx2) run per wavefront instruction.
//   * VALU (fp32, or G == 1): plain per-(head, token) dot products through LDS.
#include "sp_internal.h"

namespace spk {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kAttnThreads = 256;
constexpr int kWaves = kAttnThreads / 64;

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

struct PageRef {
  int blk;      // physical block, -1 when the entry is skipped
  int nvalid;   // valid tokens on the page
  int logical;  // logical page index
};

// Entry `entry` of the (b, h) page list: a selection entry (Quest) or a
// logical page (dense).  Invalid entries resolve to blk = -1.
__device__ __forceinline__ PageRef resolve_page(const KVDev& kv, int b, const int32_t* sel_row,
                                                int top_k, int entry, int L, int n_pages) {
  PageRef r{-1, 0, -1};
  int p;
  if (sel_row != nullptr) {
    if (entry >= top_k) return r;
    p = sel_row[entry];
  } else {
    p = entry;
  }
  if (p < 0 || p >= n_pages) return r;
  const int blk = kv.block_table[(size_t)b * kv.max_pages + p];
  if (blk < 0 || blk >= kv.num_blocks) return r;
  r.blk = blk;
  r.nvalid = min(kv.P, L - p * kv.P);
  r.logical = p;
  return r;
}

// Partial record of (b, h, split, head-in-group): acc[D], m, l.
__device__ __forceinline__ float* partial_rec(float* partial, const KVDev& kv, int b, int h,
                                              int split, int n_splits, int a) {
  return partial + ((((size_t)b * kv.Hkv + h) * n_splits + split) * kv.G + a) * (size_t)(kv.D + 2);
}

// ============================================================== MFMA kernel
template <int D, int P>
struct MfmaPage {
  static constexpr int KS = D / 32;   // 16x16x32 k-steps over the head dim
  static constexpr int MB = P / 16;   // 16-token tiles per page
  static constexpr int NB = D / 16;   // 16-dim output tiles
  uint4 k[MB][KS];                    // K A-operands: token 16mb+col, chunk 4ks+g
  uint2 v[MB][NB];                    // V^T A-operands: dim 16nb+col, tokens 16mb+4g..+3
};

template <int D, int P>
__device__ __forceinline__ void load_page(MfmaPage<D, P>& pg, const bf16_t* kp, const bf16_t* vp,
                                          int col, int g) {
#pragma unroll
  for (int mb = 0; mb < MfmaPage<D, P>::MB; ++mb)
#pragma unroll
    for (int ks = 0; ks < MfmaPage<D, P>::KS; ++ks)
      pg.k[mb][ks] = *reinterpret_cast<const uint4*>(kp + (size_t)((4 * ks + g) * P + 16 * mb + col) * 8);
#pragma unroll
  for (int mb = 0; mb < MfmaPage<D, P>::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < MfmaPage<D, P>::NB; ++nb)
      pg.v[mb][nb] = *reinterpret_cast<const uint2*>(vp + (size_t)(16 * nb + col) * P + 16 * mb + 4 * g);
}

template <int D, int P>
struct MfmaState {
  float4_t o[D / 16];   // O^T tiles: lane holds dims 16nb+4g+r of head `col`
  float m;              // running max (log2 domain) of head `col`
  float l;              // this lane's share of the running denominator
};

template <int D, int P>
__device__ __forceinline__ void process_page(MfmaState<D, P>& st, const MfmaPage<D, P>& pg,
                                             const bf16x8_t (&qop)[D / 32], int nvalid,
                                             float scale_log2, float scale, float* logit_row,
                                             int col, int g) {
  constexpr int KS = D / 32, MB = P / 16, NB = D / 16;
  float s[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, pg.k[mb][ks]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop[ks], acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * mb + 4 * g + r;
      const bool ok = t < nvalid;
      s[mb][r] = ok ? acc[r] * scale_log2 : -INFINITY;
      if (logit_row != nullptr && ok) logit_row[t] = acc[r] * scale;
    }
  }
  float mt = -INFINITY;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) mt = fmaxf(mt, s[mb][r]);
  mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
  mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
  const float m_new = fmaxf(st.m, mt);        // finite: the page has >= 1 valid token
  const float alpha = fast_exp2(st.m - m_new);  // 0 on the first page (m = -inf)
  st.m = m_new;
  float psum = 0.f;
  short4_t phi[MB], plo[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = fast_exp2(s[mb][r] - m_new);
      psum += p;
      const bf16_t hi = f32_to_bf16(p);
      const bf16_t lo = f32_to_bf16(p - to_f32(hi));
      phi[mb][r] = (short)hi;
      plo[mb][r] = (short)lo;
    }
  }
  st.l = st.l * alpha + psum;
  if (alpha != 1.0f) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) st.o[nb] *= alpha;
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const short4_t va = __builtin_bit_cast(short4_t, pg.v[mb][nb]);
      st.o[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, phi[mb], st.o[nb], 0, 0, 0);
      st.o[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, plo[mb], st.o[nb], 0, 0, 0);
    }
  }
}

template <int D, int P>
__global__ void __launch_bounds__(kAttnThreads)
attn_mfma_kernel(KVDev kv, const bf16_t* __restrict__ q, const int32_t* __restrict__ sel,
                 int top_k, int pps, float scale, float* __restrict__ logits, int logit_cap,
                 float* __restrict__ partial, int n_splits) {
  constexpr int NB = D / 16, KS = D / 32;
  constexpr int OSTR = D + 1;                       // padded LDS row (bank spread)
  extern __shared__ float lds[];                    // [kWaves][G][OSTR] + m,l [kWaves][G]
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int G = kv.G;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int cap = kv.max_pages * kv.P;
  const int L = clamp_len(kv.seq_lens[b], cap);
  const int n_pages = (L + P - 1) / P;
  const bool sparse = sel != nullptr;
  const int e0 = split * pps;
  // dense mode: splits past the last page produce nothing (the merge knows)
  if (!sparse && e0 >= n_pages) return;
  const int e1 = min(e0 + pps, sparse ? top_k : n_pages);
  const int32_t* sel_row = sparse ? sel + ((size_t)b * kv.Hkv + h) * top_k : nullptr;

  // Q^T B-operand: head `col` of the group, chunk 4ks+g (8 dims); zero for col >= G.
  bf16x8_t qop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    uint4 u = {0u, 0u, 0u, 0u};
    if (col < G)
      u = *reinterpret_cast<const uint4*>(q + ((size_t)b * kv.Hq + h * G + col) * D + (4 * ks + g) * 8);
    qop[ks] = __builtin_bit_cast(bf16x8_t, u);
  }
  const float scale_log2 = scale * kLog2e;
  float* logit_base = (logits != nullptr && col < G)
                          ? logits + ((size_t)b * kv.Hq + h * G + col) * logit_cap : nullptr;

  MfmaState<D, P> st;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) st.o[nb] = float4_t{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;

  const bf16_t* kpool = reinterpret_cast<const bf16_t*>(kv.k_pool);
  const bf16_t* vpool = reinterpret_cast<const bf16_t*>(kv.v_pool);
  // Wave w takes entries e0 + w, e0 + w + 4, ...; the next page is loaded into
  // the other buffer while the current one is processed (static ping-pong so
  // both buffers stay in registers).
  MfmaPage<D, P> bufA, bufB;
  int e = e0 + w;
  PageRef cur = e < e1 ? resolve_page(kv, b, sel_row, top_k, e, L, n_pages) : PageRef{-1, 0, -1};
  if (cur.blk >= 0) {
    const size_t base = page_base(cur.blk, h, kv.Hkv, P, D);
    load_page<D, P>(bufA, kpool + base, vpool + base, col, g);
  }
  auto step = [&](MfmaPage<D, P>& now, MfmaPage<D, P>& next) {
    const int en = e + kWaves;
    const PageRef nxt = en < e1 ? resolve_page(kv, b, sel_row, top_k, en, L, n_pages) : PageRef{-1, 0, -1};
    if (nxt.blk >= 0) {
      const size_t base = page_base(nxt.blk, h, kv.Hkv, P, D);
      load_page<D, P>(next, kpool + base, vpool + base, col, g);
    }
    if (cur.blk >= 0) {
      float* lrow = logit_base ? logit_base + (size_t)cur.logical * P : nullptr;
      process_page<D, P>(st, now, qop, cur.nvalid, scale_log2, scale, lrow, col, g);
    }
    cur = nxt;
    e = en;
  };
  while (e < e1) {
    step(bufA, bufB);
    if (e >= e1) break;
    step(bufB, bufA);
  }
  // full denominator of head `col` across the four lane groups
  float lsum = st.l;
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);

  // combine the four waves
  float* lds_o = lds;                                  // [w][a][OSTR]
  float* lds_m = lds + (size_t)kWaves * G * OSTR;      // [w][a]
  float* lds_l = lds_m + kWaves * G;
  if (col < G) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) lds_o[((size_t)w * G + col) * OSTR + 16 * nb + 4 * g + r] = st.o[nb][r];
    if (g == 0) {
      lds_m[w * G + col] = st.m;
      lds_l[w * G + col] = lsum;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * D; i += kAttnThreads) {
    const int a = i / D, d = i % D;
    float mstar = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) mstar = fmaxf(mstar, lds_m[ww * G + a]);
    float o = 0.f, l = 0.f;
    if (mstar != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const float mw = lds_m[ww * G + a];
        if (mw == -INFINITY) continue;
        const float f = fast_exp2(mw - mstar);
        o += f * lds_o[((size_t)ww * G + a) * OSTR + d];
        l += f * lds_l[ww * G + a];
      }
    }
    float* rec = partial_rec(partial, kv, b, h, split, n_splits, a);
    rec[d] = o;
    if (d == 0) {
      rec[D] = mstar;
      rec[D + 1] = l;
    }
  }
}

// ============================================================== VALU kernel
constexpr int kValuMaxG = 16;
constexpr int kValuTasks = 8;   // >= kValuMaxG * 128 / kAttnThreads

template <typename T, int D, int P>
__global__ void __launch_bounds__(kAttnThreads)
attn_valu_kernel(KVDev kv, const T* __restrict__ q, const int32_t* __restrict__ sel, int top_k,
                 int pps, float scale, float* __restrict__ logits, int logit_cap,
                 float* __restrict__ partial, int n_splits) {
  constexpr int E = Chunk<T>::E;
  __shared__ float qs[kValuMaxG][D];
  __shared__ float S[kValuMaxG][P + 1];
  __shared__ float m_run[kValuMaxG], l_run[kValuMaxG], alpha[kValuMaxG];
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int G = kv.G, tid = threadIdx.x;
  const int cap = kv.max_pages * P;
  const int L = clamp_len(kv.seq_lens[b], cap);
  const int n_pages = (L + P - 1) / P;
  const bool sparse = sel != nullptr;
  const int e0 = split * pps;
  if (!sparse && e0 >= n_pages) return;
  const int e1 = min(e0 + pps, sparse ? top_k : n_pages);
  const int32_t* sel_row = sparse ? sel + ((size_t)b * kv.Hkv + h) * top_k : nullptr;

  for (int i = tid; i < G * D; i += kAttnThreads)
    qs[i / D][i % D] = to_f32(q[((size_t)b * kv.Hq + h * G + i / D) * D + i % D]);
  if (tid < G) { m_run[tid] = -INFINITY; l_run[tid] = 0.f; }
  float oacc[kValuTasks];
#pragma unroll
  for (int k = 0; k < kValuTasks; ++k) oacc[k] = 0.f;
  __syncthreads();

  const float scale_log2 = scale * kLog2e;
  const T* kpool = reinterpret_cast<const T*>(kv.k_pool);
  const T* vpool = reinterpret_cast<const T*>(kv.v_pool);
  for (int e = e0; e < e1; ++e) {
    const PageRef pr = resolve_page(kv, b, sel_row, top_k, e, L, n_pages);
    if (pr.blk < 0) continue;                       // uniform across the block
    const size_t base = page_base(pr.blk, h, kv.Hkv, P, D);
    const T* kp = kpool + base;
    const T* vp = vpool + base;
    for (int i = tid; i < G * P; i += kAttnThreads) {
      const int a = i / P, t = i % P;
      float z = -INFINITY;
      if (t < pr.nvalid) {
        float dot = 0.f;
        for (int c = 0; c < D / E; ++c) {
          union { uint4 u; T e[E]; } w;
          w.u = *reinterpret_cast<const uint4*>(kp + (size_t)(c * P + t) * E);
#pragma unroll
          for (int x = 0; x < E; ++x) dot = fmaf(qs[a][c * E + x], to_f32(w.e[x]), dot);
        }
        z = dot * scale;
        if (logits != nullptr)
          logits[((size_t)b * kv.Hq + h * G + a) * logit_cap + (size_t)pr.logical * P + t] = z;
        z = dot * scale_log2;
      }
      S[a][t] = z;
    }
    __syncthreads();
    if (tid < G) {
      float mt = -INFINITY;
      for (int t = 0; t < pr.nvalid; ++t) mt = fmaxf(mt, S[tid][t]);
      const float m_new = fmaxf(m_run[tid], mt);
      const float al = fast_exp2(m_run[tid] - m_new);
      float sum = 0.f;
      for (int t = 0; t < P; ++t) {
        const float p = t < pr.nvalid ? fast_exp2(S[tid][t] - m_new) : 0.f;
        S[tid][t] = p;
        sum += p;
      }
      l_run[tid] = l_run[tid] * al + sum;
      m_run[tid] = m_new;
      alpha[tid] = al;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kValuTasks; ++k) {
      const int idx = tid + k * kAttnThreads;
      if (idx < G * D) {
        const int a = idx / D, d = idx % D;
        float o = oacc[k] * alpha[a];
        const T* vrow = vp + (size_t)d * P;
        for (int t = 0; t < pr.nvalid; ++t) o = fmaf(S[a][t], to_f32(vrow[t]), o);
        oacc[k] = o;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < kValuTasks; ++k) {
    const int idx = tid + k * kAttnThreads;
    if (idx < G * D) {
      const int a = idx / D, d = idx % D;
      float* rec = partial_rec(partial, kv, b, h, split, n_splits, a);
      rec[d] = oacc[k];
      if (d == 0) {
        rec[D] = m_run[a];
        rec[D + 1] = l_run[a];
      }
    }
  }
}

// ============================================================== merge
template <int D>
__global__ void __launch_bounds__(D)
attn_merge_kernel(KVDev kv, const int32_t* __restrict__ sel, int pps, const float* __restrict__ partial,
                  int n_splits, float* __restrict__ out, float* __restrict__ lse) {
  const int a = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int G = kv.G, h = a / G, ai = a % G;
  const int L = clamp_len(kv.seq_lens[b], kv.max_pages * kv.P);
  const int n_pages = (L + kv.P - 1) / kv.P;
  // dense mode: only splits that own at least one page wrote a record
  const int active = sel != nullptr ? n_splits : min(n_splits, (n_pages + pps - 1) / pps);
  const size_t stride = (size_t)G * (D + 2);
  const float* rec0 = partial + (((size_t)b * kv.Hkv + h) * n_splits * G + ai) * (size_t)(D + 2);
  float mstar = -INFINITY;
  for (int s = 0; s < active; ++s) mstar = fmaxf(mstar, rec0[s * stride + D]);
  float o = 0.f, l = 0.f;
  if (mstar != -INFINITY) {
    for (int s = 0; s < active; ++s) {
      const float* rec = rec0 + s * stride;
      const float ms = rec[D];
      if (ms == -INFINITY) continue;
      const float f = fast_exp2(ms - mstar);
      o += f * rec[d];
      l += f * rec[D + 1];
    }
  }
  const bool any = l > 0.f;
  out[((size_t)b * kv.Hq + a) * D + d] = any ? o / l : 0.f;
  if (lse != nullptr && d == 0) lse[(size_t)b * kv.Hq + a] = any ? (mstar + log2f(l)) * kLn2 : -INFINITY;
}

template <int D, int P>
hipError_t attn_mfma_t(const KVDev& kv, const AttnPlan& plan, const void* q, const int32_t* sel,
                       int top_k, float scale, float* logits, int logit_cap, float* partial,
                       hipStream_t s) {
  dim3 grid(plan.n_splits, kv.Hkv, kv.B);
  const size_t lds = ((size_t)kWaves * kv.G * (D + 1) + 2 * kWaves * kv.G) * sizeof(float);
  attn_mfma_kernel<D, P><<<grid, kAttnThreads, lds, s>>>(
      kv, static_cast<const bf16_t*>(q), sel, top_k, plan.pages_per_split, scale, logits,
      logit_cap, partial, plan.n_splits);
  return hipGetLastError();
}

template <typename T, int D, int P>
hipError_t attn_valu_t(const KVDev& kv, const AttnPlan& plan, const void* q, const int32_t* sel,
                       int top_k, float scale, float* logits, int logit_cap, float* partial,
                       hipStream_t s) {
  dim3 grid(plan.n_splits, kv.Hkv, kv.B);
  attn_valu_kernel<T, D, P><<<grid, kAttnThreads, 0, s>>>(
      kv, static_cast<const T*>(q), sel, top_k, plan.pages_per_split, scale, logits, logit_cap,
      partial, plan.n_splits);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t attn_dispatch_p(const KVDev& kv, const AttnPlan& plan, const void* q,
                           const int32_t* sel, int top_k, float scale, float* logits,
                           int logit_cap, float* partial, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    if (plan.mfma) {
      if (kv.P == 16) return attn_mfma_t<D, 16>(kv, plan, q, sel, top_k, scale, logits, logit_cap, partial, s);
      return attn_mfma_t<D, 32>(kv, plan, q, sel, top_k, scale, logits, logit_cap, partial, s);
    }
  }
  if (kv.P == 16) return attn_valu_t<T, D, 16>(kv, plan, q, sel, top_k, scale, logits, logit_cap, partial, s);
  return attn_valu_t<T, D, 32>(kv, plan, q, sel, top_k, scale, logits, logit_cap, partial, s);
}

}  // namespace

AttnPlan plan_attention(const KVDev& kv, int dtype, bool sparse, int top_k) {
  AttnPlan p;
  p.mfma = (dtype == SP_BF16) && kv.G >= 2;
  const int n_work = sparse ? top_k : kv.max_pages;
  if (p.mfma) {
    int pps = kv.P == 16 ? 16 : 8;
    const long units = (long)kv.B * kv.Hkv;
    while (pps > 4 && units * ((n_work + pps - 1) / pps) < 1024) pps /= 2;
    p.pages_per_split = pps;
  } else {
    p.pages_per_split = 4;
  }
  p.n_splits = (n_work + p.pages_per_split - 1) / p.pages_per_split;
  if (p.n_splits < 1) p.n_splits = 1;
  p.ws_bytes = (size_t)kv.B * kv.Hkv * p.n_splits * kv.G * (kv.D + 2) * sizeof(float);
  return p;
}

hipError_t launch_attention(const KVDev& kv, int dtype, const AttnPlan& plan, const void* q,
                            const int32_t* sel, int top_k, float scale, float* out, float* lse,
                            float* logits, int logit_cap, void* ws, hipStream_t s) {
  float* partial = static_cast<float*>(ws);
  hipError_t e;
  if (dtype == SP_BF16)
    e = kv.D == 128 ? attn_dispatch_p<bf16_t, 128>(kv, plan, q, sel, top_k, scale, logits, logit_cap, partial, s)
                    : attn_dispatch_p<bf16_t, 64>(kv, plan, q, sel, top_k, scale, logits, logit_cap, partial, s);
  else
    e = kv.D == 128 ? attn_dispatch_p<float, 128>(kv, plan, q, sel, top_k, scale, logits, logit_cap, partial, s)
                    : attn_dispatch_p<float, 64>(kv, plan, q, sel, top_k, scale, logits, logit_cap, partial, s);
  if (e != hipSuccess) return e;
  dim3 grid(kv.Hq, kv.B);
  if (kv.D == 128)
    attn_merge_kernel<128><<<grid, 128, 0, s>>>(kv, sel, plan.pages_per_split, partial, plan.n_splits, out, lse);
  else
    attn_merge_kernel<64><<<grid, 64, 0, s>>>(kv, sel, plan.pages_per_split, partial, plan.n_splits, out, lse);
  return hipGetLastError();
}

}  // namespace spk
