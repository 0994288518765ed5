// One Quest decode step of one layer in a single launch: the decode token's
// append and page-summary fold, the page scoring and per-KV-head top-k, and
// the attention over the selected pages.
//
// "SparseEngine: Sparse-First Inference Engine", Appendix A.3, "Quest:
// Query-Dependent Page Selection" (new keys update the extrema of their
// pages; pages are ranked by an estimate that upper-bounds every token's
// logit; attention uses the actual KV of the selected pages) and Appendix
// A.1, "Attention over Selected Positions" (softmax normalised over the
// selected positions only).  The results are those of sp_append_select_pages
// followed by sp_sparse_decode_attn.
//
// The launch is one resident round of workgroups: for bf16 caches 8-wave
// workgroups, one per CU (the unit's top-k, which runs in one workgroup, then
// has runs half as long as with 4 waves); for fp32 caches 4-wave workgroups,
// two per CU.  Each first scores one
// chunk of one (sequence, KV head) unit's page summaries exactly as the
// selection launch does (the last workgroup of a unit runs its top-k), then
// the n workgroups that scored a unit attend over an equal share of that
// unit's selected tiles.  A unit's attention cannot start before its
// selection exists, so the top-k workgroup writes a resolved descriptor per
// selected page -- (block id << 6) | tokens of the page -- through to the
// point of coherence of all XCDs, tagged with the unit's epoch of this call
// (every workgroup of the unit read the previous epoch in its prologue, before
// counting in, so before the top-k raises it); the attention workgroups poll
// their descriptors until they carry the epoch, so no block-table lookup or
// length load sits before the first tile load.  The appended token's K and V
// are also written through, since a workgroup on another XCD may read that
// page.  The split states are merged by epoch-tagged records: every
// workgroup of the unit writes its record and tag, waits for the others' and
// merges its own share of the unit's output, so nothing needs resetting after
// the call.
//
// Against the two launches this removes one launch and its gap, the
// attention's start-up overlaps the other units' selection, and the merge
// needs no arrival counter.  Every wait is on workgroups of the same launch
// whose own waits are on earlier steps of the same chain (scoring and top-k
// never wait), and the launch is only used when the runtime reports that
// every workgroup is resident at once; otherwise the entry point runs the two
// launches.  A wait that is not released within about a second sets the
// workspace's error word and gives up instead of hanging.
#include "attn_dev.h"
#include "select_dev.h"

namespace spk {
namespace {

// Both phases' workgroup size and the launch's workgroup count (about one
// resident round): bf16 caches take one 8-wave workgroup per CU, which halves
// the runs of the unit's top-k (the step's serial phase); fp32 caches (tiny
// VALU-engine tiles, latency-bound) keep two 4-wave workgroups per CU, which
// measured faster for them.
template <typename T>
struct StepShape {
  static constexpr int kThreads = sizeof(T) == 2 ? 512 : 256;
  static constexpr int kWgTarget = sizeof(T) == 2 ? 256 : 512;
  static constexpr int kMaxPages = 24 * kThreads;   // top-k runs of at most 24 keys per thread
};

template <typename T, int D, int P, int RM, bool GMAX, typename Engine>
__global__ void __launch_bounds__(StepShape<T>::kThreads)
quest_step_kernel(KVDev kv, const T* __restrict__ q, const T* __restrict__ meta, float* __restrict__ scores,
                  int chunk, int n_chunks, int top_k, int n_sink, int n_recent, int32_t* __restrict__ sel,
                  int* __restrict__ sel_counters, AppendIn ap, seldev::SelFused fz, attndev::FusedAttnArgs F) {
  constexpr int kStepThreads = StepShape<T>::kThreads;
  static_assert(Engine::kThreads == kStepThreads, "both phases run on the same workgroup");
  __shared__ uint32_t s_epoch;
  seldev::select_block<T, D, RM, GMAX ? (sizeof(T) == 2 ? 2 : 1) : 0, true, kStepThreads>(kv, q, meta, scores, chunk, n_chunks, top_k, n_sink, n_recent, sel,
                                             sel_counters, ap, fz, blockIdx.x, &s_epoch);
  __syncthreads();   // the dynamic LDS passes from the scoring to the attention
  const uint32_t epoch = s_epoch;
  const int u = blockIdx.x / n_chunks, c = blockIdx.x % n_chunks;
  attndev::fused_attend<Engine, D, P, T>(F, u, c, n_chunks, epoch);
  attndev::fused_merge<Engine, D>(F, u, c, n_chunks, epoch);
}

// Workspace of the fused step (bytes, 256-aligned areas):
//   select counters | attention counters | unit epochs | error word
//   | page scores | descriptors | record tags
//   | split records
// (one tag and one record per workgroup; the attention counters and the
// record area also serve the two-launch form).  A workspace serves calls of
// one descriptor shape and top_k.
struct StepLayout {
  size_t sel_ctr, att_ctr, epoch, err, scores, desc, tags, records, list, total;
};
inline size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }
StepLayout step_layout(const KVDev& kv, int top_k, int grid, int two_launch_records) {
  const size_t units = (size_t)kv.B * kv.Hkv;
  StepLayout l;
  size_t off = 0;
  l.sel_ctr = off; off += up256((size_t)kv.B * (kv.Hkv + 1) * sizeof(int));
  l.att_ctr = off; off += up256(units * sizeof(int));
  l.epoch = off;   off += up256(units * sizeof(uint32_t));
  l.err = off;     off += 256;
  l.scores = off;  off += up256(units * kv.max_pages * sizeof(float));
  l.desc = off;    off += up256(units * (size_t)top_k * sizeof(uint64_t));
  l.tags = off;    off += up256((size_t)grid * sizeof(uint32_t));
  const size_t recs = (size_t)(grid > two_launch_records ? grid : two_launch_records);
  l.records = off; off += up256(recs * kv.G * (kv.D + 2) * sizeof(float));
  l.list = off;    off += up256(select_list_bytes(kv));   // the list top-k's (two launches only)
  l.total = off;
  return l;
}

// Grid of the fused launch: the scoring chunks of every unit.
template <typename T, int D>
int step_grid(const KVDev& kv, int* chunk, int* n_chunks) {
  seldev::select_chunks<T, D, StepShape<T>::kThreads>(kv, chunk, n_chunks, StepShape<T>::kWgTarget);
  return kv.B * kv.Hkv * *n_chunks;
}

template <typename T, int D>
size_t step_lds_bytes(const KVDev& kv, bool mfma) {
  constexpr int kStepThreads = StepShape<T>::kThreads;
  const size_t s = seldev::select_lds_bytes(kv.G, D, kStepThreads);
  const size_t a = (size_t)attndev::lds_layout(kv.B, kv.G, D, true, mfma, kStepThreads / 64, kv.max_pages, true)
                       .total * 4;
  return s > a ? s : a;
}

// Resident workgroups of a kernel on the current device (0 if unknown).
int resident_wgs(const void* fn, int threads, size_t lds) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds) != hipSuccess) return 0;
  return cus * per_cu;
}

// With query set, only decides whether the single launch fits (*fused).
template <typename T, int D, int P, int RM, bool GMAX>
hipError_t step_launch(const KVDev& kv, const T* q, const T* meta, int top_k, const SelectOpts& o, int32_t* sel,
                       float* page_scores, float scale, float* out, float* lse, void* ws, hipStream_t s,
                       bool* fused, bool query) {
  constexpr int kStepThreads = StepShape<T>::kThreads;
  int chunk, n_chunks;
  const int grid = step_grid<T, D>(kv, &chunk, &n_chunks);
  const bool mfma = sizeof(T) == 2 && kv.G >= 2;
  const size_t lds = step_lds_bytes<T, D>(kv, mfma);
  using EngM = attndev::MfmaEngine<D, P, false, kStepThreads>;   // instantiated for bf16 only
  using EngV = attndev::ValuEngine<T, D, P, false, kStepThreads>;
  const void* fn = reinterpret_cast<const void*>(&quest_step_kernel<T, D, P, RM, GMAX, EngV>);
  if constexpr (sizeof(T) == 2) {
    if (mfma) fn = reinterpret_cast<const void*>(&quest_step_kernel<T, D, P, RM, GMAX, EngM>);
  }
  if (resident_wgs(fn, kStepThreads, lds) < grid) {
    *fused = false;
    return hipSuccess;
  }
  *fused = true;
  if (query) return hipSuccess;
  const StepLayout l = step_layout(kv, top_k, grid, 0);
  char* w = static_cast<char*>(ws);
  int* sel_counters = reinterpret_cast<int*>(w + l.sel_ctr);
  float* scores = page_scores ? page_scores : reinterpret_cast<float*>(w + l.scores);
  seldev::SelFused fz;
  fz.desc = reinterpret_cast<uint64_t*>(w + l.desc);
  fz.epoch = reinterpret_cast<uint32_t*>(w + l.epoch);
  attndev::FusedAttnArgs A;
  A.kv = kv;
  A.q = q;
  A.top_k = top_k;
  A.scale = scale;
  A.out = out;
  A.lse = lse;
  A.desc = fz.desc;
  A.records = reinterpret_cast<float*>(w + l.records);
  A.tags = reinterpret_cast<uint32_t*>(w + l.tags);
  A.err = reinterpret_cast<int*>(w + l.err);
  bool launched = false;
  if constexpr (sizeof(T) == 2) {
    if (mfma) {
      quest_step_kernel<T, D, P, RM, GMAX, EngM><<<grid, kStepThreads, lds, s>>>(
          kv, q, meta, scores, chunk, n_chunks, top_k, o.n_sink, o.n_recent, sel, sel_counters, o.ap, fz, A);
      launched = true;
    }
  }
  if (!launched)
    quest_step_kernel<T, D, P, RM, GMAX, EngV><<<grid, kStepThreads, lds, s>>>(
        kv, q, meta, scores, chunk, n_chunks, top_k, o.n_sink, o.n_recent, sel, sel_counters, o.ap, fz, A);
  return hipGetLastError();
}

// The fused launch covers up to 24 * 512 = 12 288 pages per sequence for
// bf16 caches, 24 * 256 = 6144 for fp32 (top-k runs of 8, 16 or 24 keys per
// thread), with the sum over the group, and with the maximum over the group
// for bf16 and 128-dimension heads; other selections take the two launches.

template <typename T, int D, int P, bool GMAX>
hipError_t step_rm(const KVDev& kv, const T* qt, const T* mt, int top_k, const SelectOpts& o, int32_t* sel,
                   float* page_scores, float scale, float* out, float* lse, void* ws, hipStream_t s, bool* fused,
                   bool query) {
  constexpr int kStepThreads = StepShape<T>::kThreads;
  const int R = (kv.max_pages + kStepThreads - 1) / kStepThreads;
  if (R <= 8)
    return step_launch<T, D, P, 8, GMAX>(kv, qt, mt, top_k, o, sel, page_scores, scale, out, lse, ws, s, fused,
                                         query);
  if (R <= 16)
    return step_launch<T, D, P, 16, GMAX>(kv, qt, mt, top_k, o, sel, page_scores, scale, out, lse, ws, s, fused,
                                          query);
  return step_launch<T, D, P, 24, GMAX>(kv, qt, mt, top_k, o, sel, page_scores, scale, out, lse, ws, s, fused,
                                        query);
}

template <typename T, int D, int P>
hipError_t step_t(const KVDev& kv, const void* q, const void* meta, int top_k, const SelectOpts& o, int32_t* sel,
                  float* page_scores, float scale, float* out, float* lse, void* ws, hipStream_t s, bool* fused,
                  bool query) {
  const T* qt = static_cast<const T*>(q);
  const T* mt = static_cast<const T*>(meta);
  *fused = false;
  if (kv.max_pages > StepShape<T>::kMaxPages) return hipSuccess;
  if (o.group_max) {
    if constexpr (sizeof(T) == 2 && D == 128)
      return step_rm<T, D, P, true>(kv, qt, mt, top_k, o, sel, page_scores, scale, out, lse, ws, s, fused, query);
    return hipSuccess;
  }
  return step_rm<T, D, P, false>(kv, qt, mt, top_k, o, sel, page_scores, scale, out, lse, ws, s, fused, query);
}

template <typename T>
hipError_t step_shape(const KVDev& kv, const void* q, const void* meta, int top_k, const SelectOpts& o,
                      int32_t* sel, float* page_scores, float scale, float* out, float* lse, void* ws,
                      hipStream_t s, bool* fused, bool query) {
  if (kv.D == 128)
    return kv.P == 16
               ? step_t<T, 128, 16>(kv, q, meta, top_k, o, sel, page_scores, scale, out, lse, ws, s, fused, query)
               : step_t<T, 128, 32>(kv, q, meta, top_k, o, sel, page_scores, scale, out, lse, ws, s, fused, query);
  return kv.P == 16 ? step_t<T, 64, 16>(kv, q, meta, top_k, o, sel, page_scores, scale, out, lse, ws, s, fused, query)
                    : step_t<T, 64, 32>(kv, q, meta, top_k, o, sel, page_scores, scale, out, lse, ws, s, fused, query);
}

int step_grid_of(const KVDev& kv, int dtype) {
  int chunk = 0, n_chunks = 0;
  if (dtype == SP_BF16)
    return kv.D == 128 ? step_grid<bf16_t, 128>(kv, &chunk, &n_chunks) : step_grid<bf16_t, 64>(kv, &chunk, &n_chunks);
  return kv.D == 128 ? step_grid<float, 128>(kv, &chunk, &n_chunks) : step_grid<float, 64>(kv, &chunk, &n_chunks);
}

}  // namespace

size_t quest_step_error_offset(const KVDev& kv) { return step_layout(kv, 1, 1, 0).err; }

hipError_t quest_step_single_launch(const KVDev& kv, int dtype, bool group_max, bool* single) {
  SelectOpts o;
  o.group_max = group_max;
  return dtype == SP_BF16
             ? step_shape<bf16_t>(kv, nullptr, nullptr, 1, o, nullptr, nullptr, 0.f, nullptr, nullptr, nullptr,
                                  nullptr, single, true)
             : step_shape<float>(kv, nullptr, nullptr, 1, o, nullptr, nullptr, 0.f, nullptr, nullptr, nullptr,
                                 nullptr, single, true);
}

size_t quest_step_workspace_bytes(const KVDev& kv, int dtype, int top_k) {
  // records for the fused grid or for the two-launch form's attention plan,
  // whichever is larger
  const AttnPlan ap = plan_attention(kv, dtype, true, top_k);
  return step_layout(kv, top_k, step_grid_of(kv, dtype), ap.n_wg + kv.B * kv.Hkv).total;
}

hipError_t launch_quest_step(const KVDev& kv, int dtype, const void* q, const void* page_meta, int top_k,
                             const SelectOpts& o, int32_t* sel, float* page_scores, float scale, float* out,
                             float* lse, void* ws, hipStream_t s, bool* fused) {
  hipError_t e =
      dtype == SP_BF16
          ? step_shape<bf16_t>(kv, q, page_meta, top_k, o, sel, page_scores, scale, out, lse, ws, s, fused, false)
          : step_shape<float>(kv, q, page_meta, top_k, o, sel, page_scores, scale, out, lse, ws, s, fused, false);
  if (e != hipSuccess || *fused) return e;
  // not every workgroup of the fused launch can be resident: the two
  // launches, on the same workspace (select counters and scores, then the
  // attention's counters and records)
  const AttnPlan plan = plan_attention(kv, dtype, true, top_k);
  const StepLayout l = step_layout(kv, top_k, step_grid_of(kv, dtype), plan.n_wg + kv.B * kv.Hkv);
  char* w = static_cast<char*>(ws);
  // the select launch expects counters followed by its scores in one block
  // when page_scores is NULL; give it the scores area explicitly instead
  e = launch_select_split(kv, dtype, q, page_meta, top_k, o, sel,
                          page_scores ? page_scores : reinterpret_cast<float*>(w + l.scores),
                          reinterpret_cast<int*>(w + l.sel_ctr), w + l.list, s);
  if (e != hipSuccess) return e;
  return launch_attention_split(kv, dtype, plan, q, sel, nullptr, top_k, scale, out, lse, nullptr, 0,
                                reinterpret_cast<int*>(w + l.att_ctr), reinterpret_cast<float*>(w + l.records), s);
}

}  // namespace spk
