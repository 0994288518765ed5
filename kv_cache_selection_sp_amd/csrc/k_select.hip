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
// Top-k: radix select (4 passes of 8-bit digits over order-preserving keys) in
// LDS finds the k-th largest key; pages above it are taken, and among pages
// equal to it the lowest indices, so ties go to the lower page.  A final
// index-ordered scan writes the chosen pages in ascending order.
#include "sp_internal.h"

namespace spk {
namespace {

constexpr int kScoreThreads = 256;
constexpr int kScorePagesPerBlock = 64;
constexpr int kTopkThreads = 1024;

template <typename T, int D>
__global__ void __launch_bounds__(kScoreThreads)
score_pages_kernel(KVDev kv, const T* __restrict__ q, const T* __restrict__ meta,
                   float* __restrict__ scores) {
  constexpr int E = Chunk<T>::E;
  constexpr int CPP = 2 * D / E;            // 16-byte chunks per page summary
  constexpr int PAGES_PER_ITER = kScoreThreads / CPP;
  static_assert(CPP <= 64 && (64 % CPP) == 0, "summary chunks must tile a wavefront");
  __shared__ float qsum[2][D];              // [0] = Qneg, [1] = Qpos

  const int b = blockIdx.z, h = blockIdx.y;
  const int P = kv.P, G = kv.G;
  const int L = clamp_len(kv.seq_lens[b], kv.max_pages * P);
  const int n_pages = (L + P - 1) / P;
  const int p0 = blockIdx.x * kScorePagesPerBlock;
  float* srow = scores + ((size_t)b * kv.Hkv + h) * kv.max_pages;

  for (int d = threadIdx.x; d < D; d += kScoreThreads) {
    float qp = 0.f, qn = 0.f;
    for (int a = 0; a < G; ++a) {
      const float x = to_f32(q[((size_t)b * kv.Hq + h * G + a) * D + d]);
      qp += x > 0.f ? x : 0.f;
      qn += x < 0.f ? x : 0.f;
    }
    qsum[0][d] = qn;
    qsum[1][d] = qp;
  }
  __syncthreads();

  const int j = threadIdx.x % CPP;          // chunk of the summary this lane reads
  const int row = j / (CPP / 2);            // 0: minimum row, 1: maximum row
  const int dim0 = (j % (CPP / 2)) * E;
  float w[E];
#pragma unroll
  for (int e = 0; e < E; ++e) w[e] = qsum[row][dim0 + e];

  const int sub = threadIdx.x / CPP;
  for (int it = 0; it < kScorePagesPerBlock; it += PAGES_PER_ITER) {
    const int p = p0 + it + sub;
    float part = 0.f;
    bool valid = p < n_pages;
    if (valid) {
      const int blk = kv.block_table[(size_t)b * kv.max_pages + p];
      valid = blk >= 0 && blk < kv.num_blocks;
      if (valid) {
        union { uint4 u; T e[E]; } m;
        m.u = *reinterpret_cast<const uint4*>(meta + ((size_t)blk * kv.Hkv + h) * 2 * D + j * E);
#pragma unroll
        for (int e = 0; e < E; ++e) part = fmaf(w[e], to_f32(m.e[e]), part);
      }
    }
#pragma unroll
    for (int o = CPP / 2; o >= 1; o >>= 1) part += __shfl_xor(part, o, 64);
    if (j == 0 && p < kv.max_pages) srow[p] = (p < n_pages) ? part : -INFINITY;
  }
}

__global__ void __launch_bounds__(kTopkThreads)
topk_pages_kernel(const float* __restrict__ scores, KVDev kv, int top_k, int32_t* __restrict__ sel) {
  extern __shared__ uint32_t keys[];        // [max_pages]
  __shared__ int hist[256];
  __shared__ int wsum[kTopkThreads / 64 + 1];
  __shared__ int s_digit, s_excl;

  const int b = blockIdx.y, h = blockIdx.x;
  const int P = kv.P;
  const int L = clamp_len(kv.seq_lens[b], kv.max_pages * P);
  const int N = (L + P - 1) / P;
  int32_t* out = sel + ((size_t)b * kv.Hkv + h) * top_k;
  const float* row = scores + ((size_t)b * kv.Hkv + h) * kv.max_pages;
  const int tid = threadIdx.x;

  if (top_k >= N) {                          // every page is selected
    for (int i = tid; i < top_k; i += kTopkThreads) out[i] = i < N ? i : -1;
    return;
  }
  for (int i = tid; i < N; i += kTopkThreads) keys[i] = float_key(row[i]);

  uint32_t prefix = 0, mask = 0;
  int krem = top_k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < N; i += kTopkThreads) {
      const uint32_t k = keys[i];
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255], 1);
    }
    __syncthreads();
    const int v = tid < 256 ? hist[255 - tid] : 0;   // bins from the top
    int total;
    const int excl = block_exclusive_scan<kTopkThreads>(v, wsum, &total);
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
  // prefix is now the k-th largest key; krem of the keys equal to it are taken
  // (the lowest indices).
  int eq_carry = 0, take_carry = 0;
  for (int base = 0; base < N; base += kTopkThreads) {
    const int i = base + tid;
    const uint32_t k = i < N ? keys[i] : 0u;
    const int gt = (i < N && k > prefix) ? 1 : 0;
    const int eq = (i < N && k == prefix) ? 1 : 0;
    int eq_tot, take_tot;
    const int eq_rank = eq_carry + block_exclusive_scan<kTopkThreads>(eq, wsum, &eq_tot);
    const int take = gt | (eq & (eq_rank < krem ? 1 : 0));
    const int pos = take_carry + block_exclusive_scan<kTopkThreads>(take, wsum, &take_tot);
    if (take) out[pos] = i;
    eq_carry += eq_tot;
    take_carry += take_tot;
  }
}

template <typename T, int D>
hipError_t select_t(const KVDev& kv, const void* q, const void* meta, int top_k, int32_t* sel,
                    float* scores, hipStream_t s) {
  dim3 g1((kv.max_pages + kScorePagesPerBlock - 1) / kScorePagesPerBlock, kv.Hkv, kv.B);
  score_pages_kernel<T, D><<<g1, kScoreThreads, 0, s>>>(
      kv, static_cast<const T*>(q), static_cast<const T*>(meta), scores);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(kv.Hkv, kv.B);
  topk_pages_kernel<<<g2, kTopkThreads, (size_t)kv.max_pages * sizeof(uint32_t), s>>>(
      scores, kv, top_k, sel);
  return hipGetLastError();
}

}  // namespace

size_t select_workspace_bytes(const KVDev& kv) {
  return (size_t)kv.B * kv.Hkv * kv.max_pages * sizeof(float);
}

hipError_t launch_select(const KVDev& kv, int dtype, const void* q, const void* page_meta,
                         int top_k, int32_t* sel, float* page_scores, void* ws, hipStream_t s) {
  float* scores = page_scores ? page_scores : static_cast<float*>(ws);
  if (dtype == SP_BF16) {
    if (kv.D == 128) return select_t<bf16_t, 128>(kv, q, page_meta, top_k, sel, scores, s);
    return select_t<bf16_t, 64>(kv, q, page_meta, top_k, sel, scores, s);
  }
  if (kv.D == 128) return select_t<float, 128>(kv, q, page_meta, top_k, sel, scores, s);
  return select_t<float, 64>(kv, q, page_meta, top_k, sel, scores, s);
}

}  // namespace spk
