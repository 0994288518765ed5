// Paged decode attention over selected pages (Quest) or all occupied slots
// (dense: H2O, evicted decode), with the split merge fused in.
//
// "SparseEngine: Sparse-First Inference Engine", Appendix A.1, "Attention over
// Selected Positions": attention over a nonempty selected set normalises over
// the selected positions only, dense decode being the full set; Appendix A.3,
// "Quest": attention uses the actual KV of the selected pages; Appendix A.1,
// "MHA, MQA, and GQA": query head a reads KV head a / G.
//
// Work decomposition.  The KV read by one (sequence b, KV head h) "unit" is
// cut into 16-token tiles: in Quest mode the tiles of the selected pages, in
// selection order (P/16 tiles per entry); in dense mode the tiles covering
// slots [0, seq_lens[b]).  The units' tiles are laid end to end (unit
// u = b * H_kv + h) and that range is cut into n_wg equal chunks, one per
// workgroup, so every workgroup streams the same number of tiles however
// ragged the lengths are.  Lengths are read on the device, so nothing here
// needs a host synchronisation.  A unit no longer than a chunk is handled
// whole by the workgroup whose range holds its first tile (no split, no
// merge); longer units are cut along the ranges.  For each unit segment it
// handles, a workgroup builds a softmax state per query head of the group,
// in the log2 domain:
//   m = max_j s_j,  l = sum_j 2^(s_j - m),  acc = sum_j 2^(s_j - m) v_j,
//   s_j = log2(e) * scale * (q . k_j).
// A segment that is a whole unit writes out = acc / l and
// lse = ln 2 * (m + log2 l) itself.  Otherwise its state goes to a workspace
// record, and the last of the unit's workgroups to finish (per-unit arrival
// counter) merges the unit's records in workgroup order, so the result does
// not depend on which workgroup arrives last.
//
// Tile engines:
//   * MFMA (bf16, G >= 2): the G heads sharing a KV head form a real
//     contraction.  Each wave streams its own tiles through a ring of register
//     buffers.  Per tile, S^T[16 tok x 16 heads] = K . Q^T with
//     v_mfma_f32_16x16x32_bf16 (heads padded to 16), then
//     O^T[16 dims x 16 heads] += V^T . P^T with v_mfma_f32_16x16x16_bf16, P
//     split into bf16 hi + lo so the product keeps ~16 mantissa bits.  With
//     tokens as the M dimension the S^T accumulator lane layout (lane = head
//     column, 4 tokens per lane group) is exactly the B-operand layout PV
//     needs, and a head's running max lives in the lanes that hold its output
//     accumulator, so the online-softmax rescale needs no cross-lane traffic.
//     The chunk-tiled K page and dim-major V page make every operand load a
//     contiguous 1 KB (K, dwordx4) or 512 B (V, dwordx2) run per wave
//     instruction.  The tile list is resolved into LDS first, so the load
//     pipeline never waits on a dependent global load.
//   * VALU (fp32, or G == 1): the workgroup walks its tiles one at a time,
//     one dot product per (head, token) thread, through LDS.
#include "attn_dev.h"

namespace spk {
namespace {
using namespace attndev;

// The dense tile prefix of a batch too large for LDS, and the sequence each
// workgroup's range starts in, for the attention launch that follows (one
// workgroup; the chunk is the attention's own).
constexpr int kPrefixThreads = 1024;
__global__ void __launch_bounds__(kPrefixThreads) dense_prefix_kernel(KVDev kv, int n_wg, int* __restrict__ gpre) {
  __shared__ int wsum[kPrefixThreads / 64 + 1];
  const int B = kv.B, Hkv = kv.Hkv, tid = threadIdx.x;
  const int cap = kv.max_pages * kv.P;
  int carry = 0;
  for (int base = 0; base < B; base += kPrefixThreads) {
    const int b = base + tid;
    const int Lb = b < B ? clamp_len(kv.seq_lens[b], cap) : 0;
    const int t = Hkv * ((Lb + kTok - 1) / kTok);
    int tot;
    const int ex = block_exclusive_scan<kPrefixThreads>(t, wsum, &tot);
    if (b < B) gpre[b] = carry + ex;
    carry += tot;
  }
  if (tid == 0) gpre[B] = carry;
  __syncthreads();                          // the prefix is visible to the whole workgroup
  const int total = carry;
  int chunk = (total + n_wg - 1) / n_wg;
  const int per_cu = (total + kNumCU - 1) / kNumCU;
  const int want = per_cu < kTargetChunk ? per_cu : kTargetChunk;
  if (chunk < want) chunk = want;
  if (chunk < kMinChunk) chunk = kMinChunk;
  int* wg_b = gpre + B + 1;
  // workgroup w starts at tile w * chunk, inside the one sequence whose
  // (non-empty) range holds it
  for (int b = tid; b < B; b += kPrefixThreads) {
    const int lo = gpre[b], hi = gpre[b + 1];
    for (int w = (lo + chunk - 1) / chunk; w * chunk < hi && w < n_wg; ++w) wg_b[w] = b;
  }
}

template <typename Engine, int D, int P, typename T>
__global__ void __launch_bounds__(Engine::kThreads)
attn_kernel(AttnArgs A) {
  attn_block<Engine, D, P, T>(A, blockIdx.x);
}

template <typename Engine, int D, int P, typename T>
hipError_t launch_t(const AttnArgs& A, const AttnPlan& plan, hipStream_t s) {
  attn_kernel<Engine, D, P, T><<<plan.n_wg, Engine::kThreads, plan.lds_bytes, s>>>(A);
  return hipGetLastError();
}

template <typename T, int D, int P, int NT>
hipError_t dispatch_engine(const AttnArgs& A, const AttnPlan& plan, hipStream_t s) {
  const bool logits = A.logits != nullptr;
  if constexpr (sizeof(T) == 2) {
    if (plan.mfma) {
      return logits ? launch_t<MfmaEngine<D, P, true, NT>, D, P, T>(A, plan, s)
                    : launch_t<MfmaEngine<D, P, false, NT>, D, P, T>(A, plan, s);
    }
  }
  return logits ? launch_t<ValuEngine<T, D, P, true, NT>, D, P, T>(A, plan, s)
                : launch_t<ValuEngine<T, D, P, false, NT>, D, P, T>(A, plan, s);
}

template <typename T, int D, int P>
hipError_t dispatch_threads(const AttnArgs& A, const AttnPlan& plan, hipStream_t s) {
  return plan.threads == kThreadsLarge ? dispatch_engine<T, D, P, kThreadsLarge>(A, plan, s)
                                       : dispatch_engine<T, D, P, kThreadsSmall>(A, plan, s);
}

template <typename T>
hipError_t dispatch_shape(const AttnArgs& A, const AttnPlan& plan, hipStream_t s) {
  const KVDev& kv = A.kv;
  if (kv.D == 128) return kv.P == 16 ? dispatch_threads<T, 128, 16>(A, plan, s)
                                     : dispatch_threads<T, 128, 32>(A, plan, s);
  return kv.P == 16 ? dispatch_threads<T, 64, 16>(A, plan, s) : dispatch_threads<T, 64, 32>(A, plan, s);
}

}  // namespace

AttnPlan plan_attention(const KVDev& kv, int dtype, bool sparse, int top_k) {
  AttnPlan p;
  p.mfma = (dtype == SP_BF16) && kv.G >= 2;
  const long units = (long)kv.B * kv.Hkv;
  const long tpp = kv.P / kTok;
  const long tiles_max = units * (sparse ? (long)top_k * tpp : (long)kv.max_pages * tpp);
  p.tiles_max = tiles_max;
  // Workgroup shape: with at least kTargetChunk tiles per CU and few units,
  // one 8-wave workgroup per CU (two waves per SIMD, about 8 tiles per wave);
  // otherwise 4-wave workgroups, so that short calls still spread over every
  // CU and many short units keep each wave's tile stream long.  The kernel
  // raises the chunk toward kTargetChunk from the actual lengths.
  p.threads = (p.mfma && tiles_max >= (long)kNumCU * kTargetChunk && units < 4L * kNumCU)
                  ? kThreadsLarge : kThreadsSmall;
  const long per_cu_wgs = p.threads == kThreadsLarge ? 1 : (p.mfma ? 2 : 4);
  const long wg_cap = (long)kNumCU * per_cu_wgs;   // one round of resident workgroups
  const long by_target = (tiles_max + kTargetChunk - 1) / kTargetChunk;
  const long by_min = (tiles_max + kMinChunk - 1) / kMinChunk;
  const long floor_cu = by_min < kNumCU ? by_min : kNumCU;
  long n_wg = by_target > floor_cu ? by_target : floor_cu;
  if (n_wg > wg_cap) n_wg = wg_cap;
  if (n_wg < 1) n_wg = 1;
  p.n_wg = (int)n_wg;
  p.counter_bytes = ((size_t)units * sizeof(int) + 255) & ~(size_t)255;
  p.ws_bytes = p.counter_bytes + (size_t)(n_wg + units) * kv.G * (kv.D + 2) * sizeof(float);
  // dense batches beyond what LDS holds: the tile prefix and the workgroups'
  // first sequences after the records
  p.global_prefix = !sparse && kv.B > kDenseLdsMax;
  if (p.global_prefix) p.ws_bytes += ((size_t)(kv.B + 1 + n_wg) * sizeof(int) + 255) & ~(size_t)255;
  p.lds_bytes = (size_t)lds_layout(p.global_prefix ? 0 : kv.B, kv.G, kv.D, sparse, p.mfma, p.threads / 64,
                                   kv.max_pages).total * 4;
  return p;
}

hipError_t launch_attention(const KVDev& kv, int dtype, const AttnPlan& plan, const void* q,
                            const int32_t* sel, const uint32_t* sel_mask, int top_k, float scale,
                            float* out, float* lse, float* logits, int logit_cap, void* ws,
                            hipStream_t s, float* acc_scores, int slot_cap, int n_new) {
  return launch_attention_split(kv, dtype, plan, q, sel, sel_mask, top_k, scale, out, lse, logits, logit_cap,
                                static_cast<int*>(ws),
                                reinterpret_cast<float*>(static_cast<char*>(ws) + plan.counter_bytes), s,
                                acc_scores, slot_cap, n_new);
}

hipError_t launch_attention_split(const KVDev& kv, int dtype, const AttnPlan& plan, const void* q,
                                  const int32_t* sel, const uint32_t* sel_mask, int top_k, float scale,
                                  float* out, float* lse, float* logits, int logit_cap, int* counters,
                                  float* records, hipStream_t s, float* acc_scores, int slot_cap, int n_new) {
  AttnArgs A;
  A.acc_scores = acc_scores;
  A.slot_cap = slot_cap;
  A.n_new = n_new;
  A.kv = kv;
  A.q = q;
  A.sel = sel;
  A.sel_mask = sel_mask;
  A.top_k = top_k;
  A.scale = scale;
  A.out = out;
  A.lse = lse;
  A.logits = logits;
  A.logit_cap = logit_cap;
  A.n_wg = plan.n_wg;
  A.counters = counters;
  A.records = records;
  if (plan.global_prefix) {
    int* gpre = reinterpret_cast<int*>(records + (size_t)(plan.n_wg + kv.B * kv.Hkv) * kv.G * (kv.D + 2));
    dense_prefix_kernel<<<1, kPrefixThreads, 0, s>>>(kv, plan.n_wg, gpre);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    A.gpre = gpre;
  }
  if (dtype == SP_BF16) return dispatch_shape<bf16_t>(A, plan, s);
  return dispatch_shape<float>(A, plan, s);
}

}  // namespace spk
