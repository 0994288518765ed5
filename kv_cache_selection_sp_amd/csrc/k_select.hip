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
//
// The launch runs 8-wave workgroups, about one per CU.  Beyond 5120 pages
// (runs of 10 keys over 512 threads) it only scores, and its last workgroup
// per unit leaves the sequence's page count.  Up to kRowsMaxRun * 1024 pages
// a second launch then runs the same top-k over each unit's score row with
// 1024 threads (runs half as long: the radix passes and the scans are
// per-thread work over the run); beyond that the list path's threshold search
// (k_h2o.hip) picks each unit's pages with the sink pages and the recent
// pages kept as its leading and trailing entries, in seven launches whose
// slices spread the row over many workgroups.  All three give the same
// selection.
#include "select_dev.h"

namespace spk {
namespace {
using namespace seldev;

constexpr int kSelThreads = 512;        // 8-wave workgroups
constexpr int kSelWgTarget = 256;       // about one workgroup per CU
constexpr int kInSelectMaxPages = 5120; // beyond, the separate top-k launch is as fast or faster

template <typename T, int D, int RM, int GM>
__global__ void __launch_bounds__(kSelThreads)
select_kernel(KVDev kv, const T* __restrict__ q, const T* __restrict__ meta, float* __restrict__ scores,
              int chunk, int n_chunks, int top_k, int n_sink, int n_recent, int32_t* __restrict__ sel,
              int* __restrict__ counters, AppendIn ap) {
  select_block<T, D, RM, GM, false, kSelThreads>(kv, q, meta, scores, chunk, n_chunks, top_k, n_sink, n_recent,
                                                   sel, counters, ap, SelFused(), blockIdx.x);
}

constexpr int kRowsThreads = 1024;
constexpr int kRowsMaxRun = 32;       // keys per thread (48 would spill at 1024 threads)

// The top-k of one unit's score row by 1024 threads (score rows of every
// unit written by the select launch before, the page counts per sequence).
template <int RM>
__global__ void __launch_bounds__(kRowsThreads)
topk_rows_kernel(const float* __restrict__ scores, const int32_t* __restrict__ n_pages, int Hkv, int max_pages,
                 int top_k, int n_sink, int n_recent, int32_t* __restrict__ sel) {
  __shared__ int hist[kBins];
  __shared__ uint32_t cand[kCand];
  __shared__ int sh[8 + 2 * (kRowsThreads / 64)];
  __shared__ int wsum[2][kRowsThreads / 64 + 1];
  const int u = blockIdx.x, b = u / Hkv;
  TopkLds tl;
  tl.hist = hist;
  tl.cand = cand;
  tl.sh = sh;
  tl.wsum = wsum[0];
  tl.wsum2 = wsum[1];
  topk_unit<RM, false, kRowsThreads>(scores + (size_t)u * max_pages, n_pages[b], top_k, n_sink, n_recent,
                                     sel + (size_t)u * top_k, tl, Resolve());
}

template <typename T, int D, int RM>
void select_launch(const KVDev& kv, const T* q, const T* meta, float* scores, int chunk, int n_chunks,
                   int top_k, const SelectOpts& o, int32_t* sel, int* counters, hipStream_t s) {
  const dim3 grid(kv.B * kv.Hkv * n_chunks);
  const size_t lds = select_lds_bytes(kv.G, D, kSelThreads);
  if (o.group_max) {
    constexpr int GM = sizeof(T) == 2 ? 2 : 1;
    select_kernel<T, D, RM, GM><<<grid, kSelThreads, lds, s>>>(kv, q, meta, scores, chunk, n_chunks, top_k,
                                                                 o.n_sink, o.n_recent, sel, counters, o.ap);
  } else {
    select_kernel<T, D, RM, 0><<<grid, kSelThreads, lds, s>>>(kv, q, meta, scores, chunk, n_chunks, top_k,
                                                                o.n_sink, o.n_recent, sel, counters, o.ap);
  }
}

template <typename T, int D>
hipError_t select_t(const KVDev& kv, const void* q, const void* meta, int top_k, const SelectOpts& o,
                    int32_t* sel, float* scores, int* counters, void* list_ws, hipStream_t s) {
  int chunk, n_chunks;
  select_chunks<T, D, kSelThreads>(kv, &chunk, &n_chunks, kSelWgTarget);
  const T* qt = static_cast<const T*>(q);
  const T* mt = static_cast<const T*>(meta);
  if (kv.max_pages > kInSelectMaxPages) {
    int32_t* n_pages = static_cast<int32_t*>(list_ws);
    select_launch<T, D, 0>(kv, qt, mt, scores, chunk, n_chunks, top_k, o, n_pages, counters, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int R2 = (kv.max_pages + kRowsThreads - 1) / kRowsThreads;
    const int units = kv.B * kv.Hkv;
    if (R2 <= 8)
      topk_rows_kernel<8><<<units, kRowsThreads, 0, s>>>(scores, n_pages, kv.Hkv, kv.max_pages, top_k, o.n_sink,
                                                         o.n_recent, sel);
    else if (R2 <= 16)
      topk_rows_kernel<16><<<units, kRowsThreads, 0, s>>>(scores, n_pages, kv.Hkv, kv.max_pages, top_k, o.n_sink,
                                                          o.n_recent, sel);
    else if (R2 <= kRowsMaxRun)
      topk_rows_kernel<kRowsMaxRun><<<units, kRowsThreads, 0, s>>>(scores, n_pages, kv.Hkv, kv.max_pages, top_k,
                                                                  o.n_sink, o.n_recent, sel);
    else
      return launch_page_topk_list(kv, scores, n_pages, top_k, o.n_sink, o.n_recent, sel,
                                   static_cast<char*>(list_ws) + list_counts_bytes(kv), s);
    return hipGetLastError();
  }
  // register run of the top-k: ceil(max_pages / 512) <= 10 keys per thread
  if (kv.max_pages <= 8 * kSelThreads)
    select_launch<T, D, 8>(kv, qt, mt, scores, chunk, n_chunks, top_k, o, sel, counters, s);
  else
    select_launch<T, D, 16>(kv, qt, mt, scores, chunk, n_chunks, top_k, o, sel, counters, s);
  return hipGetLastError();
}

}  // namespace

// the page counts of the list top-k, one per sequence
size_t list_counts_bytes(const KVDev& kv) { return ((size_t)kv.B * sizeof(int32_t) + 255) & ~(size_t)255; }

size_t select_list_bytes(const KVDev& kv) {
  if (kv.max_pages <= kInSelectMaxPages) return 0;
  if (kv.max_pages <= kRowsMaxRun * kRowsThreads) return list_counts_bytes(kv);
  return list_counts_bytes(kv) + page_topk_list_bytes(kv);
}

// per-unit arrival counters, then per-sequence ones (fused append)
size_t select_counter_bytes(const KVDev& kv) {
  return ((size_t)kv.B * (kv.Hkv + 1) * sizeof(int) + 255) & ~(size_t)255;
}

// counters, the scores (when the caller passes none), then the list top-k's
// page counts and lists (above the register top-k's page count)
size_t select_workspace_bytes(const KVDev& kv) {
  const size_t list = select_list_bytes(kv);
  if (list == 0) return select_counter_bytes(kv) + (size_t)kv.B * kv.Hkv * kv.max_pages * sizeof(float);
  return select_counter_bytes(kv) + select_scores_bytes(kv) + list;
}

size_t select_scores_bytes(const KVDev& kv) {
  return ((size_t)kv.B * kv.Hkv * kv.max_pages * sizeof(float) + 255) & ~(size_t)255;
}

hipError_t launch_select(const KVDev& kv, int dtype, const void* q, const void* page_meta,
                         int top_k, const SelectOpts& o, int32_t* sel, float* page_scores, void* ws,
                         hipStream_t s) {
  char* w = static_cast<char*>(ws);
  float* scores = page_scores ? page_scores : reinterpret_cast<float*>(w + select_counter_bytes(kv));
  return launch_select_split(kv, dtype, q, page_meta, top_k, o, sel, scores, static_cast<int*>(ws),
                             w + select_counter_bytes(kv) + select_scores_bytes(kv), s);
}

hipError_t launch_select_split(const KVDev& kv, int dtype, const void* q, const void* page_meta, int top_k,
                               const SelectOpts& o, int32_t* sel, float* scores, int* counters, void* list_ws,
                               hipStream_t s) {
  if (dtype == SP_BF16) {
    if (kv.D == 128) return select_t<bf16_t, 128>(kv, q, page_meta, top_k, o, sel, scores, counters, list_ws, s);
    return select_t<bf16_t, 64>(kv, q, page_meta, top_k, o, sel, scores, counters, list_ws, s);
  }
  if (kv.D == 128) return select_t<float, 128>(kv, q, page_meta, top_k, o, sel, scores, counters, list_ws, s);
  return select_t<float, 64>(kv, q, page_meta, top_k, o, sel, scores, counters, list_ws, s);
}

}  // namespace spk
