// C ABI entry points: host-side argument checks, workspace sizing, error text
// and dispatch to the kernel launchers.  Nothing here touches the device until
// every check has passed, so the checks can run on a machine without a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "sp_internal.h"

namespace {

thread_local std::string g_err;

sp_status fail(sp_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

sp_status hip_fail(hipError_t e, const char* where) {
  return fail(SP_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int64_t capacity(const sp_paged_kv* kv) { return (int64_t)kv->max_pages_per_seq * kv->page_size; }

sp_status check_kv(const sp_paged_kv* kv) {
  g_err.clear();
  if (kv == nullptr) return fail(SP_ERR_NULL_PTR, "kv descriptor is NULL");
  if (!kv->k_pool || !kv->v_pool || !kv->block_table || !kv->seq_lens)
    return fail(SP_ERR_NULL_PTR, "kv: k_pool, v_pool, block_table and seq_lens must be non-NULL");
  if (kv->batch < 1 || kv->num_q_heads < 1 || kv->num_kv_heads < 1 || kv->max_pages_per_seq < 1 ||
      kv->num_blocks < 1)
    return fail(SP_ERR_BAD_SHAPE, "kv: batch, heads, max_pages_per_seq and num_blocks must be >= 1");
  if (kv->num_q_heads % kv->num_kv_heads != 0)
    return fail(SP_ERR_BAD_SHAPE, "kv: num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                kv->num_q_heads, kv->num_kv_heads);
  if (kv->num_q_heads / kv->num_kv_heads > 16)
    return fail(SP_ERR_UNSUPPORTED, "kv: group size %d > 16", kv->num_q_heads / kv->num_kv_heads);
  if (kv->dtype != SP_F32 && kv->dtype != SP_BF16)
    return fail(SP_ERR_UNSUPPORTED, "kv: dtype %d (need SP_F32 or SP_BF16)", kv->dtype);
  if (kv->head_dim != 64 && kv->head_dim != 128)
    return fail(SP_ERR_UNSUPPORTED, "kv: head_dim %d (need 64 or 128)", kv->head_dim);
  if (kv->page_size != 16 && kv->page_size != 32)
    return fail(SP_ERR_UNSUPPORTED, "kv: page_size %d (need 16 or 32)", kv->page_size);
  if (capacity(kv) > (int64_t)1 << 30)
    return fail(SP_ERR_BAD_SHAPE, "kv: max_pages_per_seq * page_size exceeds 2^30 slots");
  if ((int64_t)kv->batch * kv->max_pages_per_seq > ((int64_t)1 << 31) - 1)
    return fail(SP_ERR_BAD_SHAPE, "kv: block table larger than 2^31 entries");
  if (!aligned(kv->k_pool, 16) || !aligned(kv->v_pool, 16))
    return fail(SP_ERR_MISALIGNED, "kv: k_pool and v_pool must be 16-byte aligned");
  if (!aligned(kv->block_table, 4) || !aligned(kv->seq_lens, 4))
    return fail(SP_ERR_MISALIGNED, "kv: block_table and seq_lens must be 4-byte aligned");
  return SP_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

sp_status sp_build_page_meta(const sp_paged_kv* kv, const void* k_new, const void* v_new,
                             int32_t n_new, void* page_meta, const int32_t* pos_new,
                             int32_t* slot_pos, int32_t slot_cap, void* stream) {
  sp_status st = check_kv(kv);
  if (st != SP_OK) return st;
  if (n_new < 0) return fail(SP_ERR_BAD_SHAPE, "n_new = %d < 0", n_new);
  if (page_meta != nullptr && !aligned(page_meta, 16))
    return fail(SP_ERR_MISALIGNED, "page_meta must be 16-byte aligned");
  const spk::KVDev d = spk::to_dev(kv);
  if (n_new == 0) {
    if (k_new != nullptr || v_new != nullptr)
      return fail(SP_ERR_BAD_SHAPE, "rebuild mode (n_new = 0) takes k_new = v_new = NULL");
    if (page_meta == nullptr) return fail(SP_ERR_NULL_PTR, "rebuild mode needs page_meta");
    hipError_t e = spk::launch_rebuild_meta(d, kv->dtype, page_meta, as_stream(stream));
    return e == hipSuccess ? SP_OK : hip_fail(e, "sp_build_page_meta(rebuild)");
  }
  if (k_new == nullptr || v_new == nullptr)
    return fail(SP_ERR_NULL_PTR, "append mode needs k_new and v_new");
  if (!aligned(k_new, 16) || !aligned(v_new, 16))
    return fail(SP_ERR_MISALIGNED, "k_new and v_new must be 16-byte aligned");
  if (pos_new != nullptr && !aligned(pos_new, 4)) return fail(SP_ERR_MISALIGNED, "pos_new must be 4-byte aligned");
  if (slot_pos != nullptr) {
    if (!aligned(slot_pos, 4)) return fail(SP_ERR_MISALIGNED, "slot_pos must be 4-byte aligned");
    if (slot_cap < capacity(kv))
      return fail(SP_ERR_BAD_SHAPE, "slot_cap %d below the capacity %lld", slot_cap,
                  (long long)capacity(kv));
  }
  hipError_t e = spk::launch_append(d, kv->dtype, k_new, v_new, n_new, page_meta, pos_new,
                                    slot_pos, slot_cap, as_stream(stream));
  return e == hipSuccess ? SP_OK : hip_fail(e, "sp_build_page_meta(append)");
}

namespace {
// Checks of the page selection's arguments (every selection entry point).
sp_status select_checks(const sp_paged_kv* kv, const void* q, const void* page_meta, int32_t top_k,
                        int32_t n_sink, int32_t n_recent, int32_t group_reduce, int32_t* sel_pages,
                        float* page_scores) {
  sp_status st = check_kv(kv);
  if (st != SP_OK) return st;
  if (!q || !page_meta || !sel_pages) return fail(SP_ERR_NULL_PTR, "q, page_meta and sel_pages are required");
  if (top_k < 1) return fail(SP_ERR_BAD_SHAPE, "top_k = %d < 1", top_k);
  if (n_sink < 0 || n_recent < 0 || (int64_t)n_sink + n_recent > top_k)
    return fail(SP_ERR_BAD_SHAPE, "need 0 <= n_sink, 0 <= n_recent, n_sink + n_recent <= top_k (got %d, %d, %d)",
                n_sink, n_recent, top_k);
  if (group_reduce != SP_GROUP_SUM && group_reduce != SP_GROUP_MAX)
    return fail(SP_ERR_BAD_SHAPE, "group_reduce = %d is neither SP_GROUP_SUM nor SP_GROUP_MAX", group_reduce);
  if (!aligned(q, 16) || !aligned(page_meta, 16))
    return fail(SP_ERR_MISALIGNED, "q and page_meta must be 16-byte aligned");
  if (!aligned(sel_pages, 4) || (page_scores && !aligned(page_scores, 4)))
    return fail(SP_ERR_MISALIGNED, "sel_pages and page_scores must be 4-byte aligned");
  return SP_OK;
}

// Checks of the decode append's arguments.
sp_status append_checks(const sp_paged_kv* kv, const void* k_new, const void* v_new, const int32_t* pos_new,
                        int32_t* slot_pos, int32_t slot_cap) {
  if (k_new == nullptr || v_new == nullptr) return fail(SP_ERR_NULL_PTR, "k_new and v_new are required");
  if (!aligned(k_new, 16) || !aligned(v_new, 16))
    return fail(SP_ERR_MISALIGNED, "k_new and v_new must be 16-byte aligned");
  if (pos_new != nullptr && !aligned(pos_new, 4)) return fail(SP_ERR_MISALIGNED, "pos_new must be 4-byte aligned");
  if (slot_pos != nullptr) {
    if (!aligned(slot_pos, 4)) return fail(SP_ERR_MISALIGNED, "slot_pos must be 4-byte aligned");
    if (slot_cap < capacity(kv))
      return fail(SP_ERR_BAD_SHAPE, "slot_cap %d below the capacity %lld", slot_cap,
                  (long long)capacity(kv));
  }
  return SP_OK;
}

sp_status select_impl(const char* who, const sp_paged_kv* kv, const void* q, const void* page_meta,
                      int32_t top_k, int32_t n_sink, int32_t n_recent, int32_t group_reduce,
                      int32_t* sel_pages, float* page_scores, void* workspace, size_t workspace_bytes,
                      void* stream, const spk::AppendIn& ap = spk::AppendIn()) {
  sp_status st = select_checks(kv, q, page_meta, top_k, n_sink, n_recent, group_reduce, sel_pages, page_scores);
  if (st != SP_OK) return st;
  const spk::KVDev d = spk::to_dev(kv);
  const size_t need = spk::select_workspace_bytes(d);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(SP_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 16)) return fail(SP_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  spk::SelectOpts o;
  o.n_sink = n_sink;
  o.n_recent = n_recent;
  o.group_max = group_reduce == SP_GROUP_MAX;
  o.ap = ap;
  hipError_t e = spk::launch_select(d, kv->dtype, q, page_meta, top_k, o, sel_pages, page_scores,
                                    workspace, as_stream(stream));
  return e == hipSuccess ? SP_OK : hip_fail(e, who);
}
}  // namespace

sp_status sp_select_pages(const sp_paged_kv* kv, const void* q, const void* page_meta,
                          int32_t top_k, int32_t* sel_pages, float* page_scores,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return select_impl("sp_select_pages", kv, q, page_meta, top_k, 0, 0, SP_GROUP_SUM, sel_pages,
                     page_scores, workspace, workspace_bytes, stream);
}

sp_status sp_select_pages_ex(const sp_paged_kv* kv, const void* q, const void* page_meta,
                             int32_t top_k, int32_t n_sink, int32_t n_recent, int32_t group_reduce,
                             int32_t* sel_pages, float* page_scores, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return select_impl("sp_select_pages_ex", kv, q, page_meta, top_k, n_sink, n_recent, group_reduce,
                     sel_pages, page_scores, workspace, workspace_bytes, stream);
}

sp_status sp_append_select_pages(const sp_paged_kv* kv, const void* k_new, const void* v_new,
                                 const int32_t* pos_new, int32_t* slot_pos, int32_t slot_cap,
                                 void* page_meta, const void* q, int32_t top_k, int32_t n_sink,
                                 int32_t n_recent, int32_t group_reduce, int32_t* sel_pages,
                                 float* page_scores, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  sp_status st = check_kv(kv);
  if (st != SP_OK) return st;
  st = append_checks(kv, k_new, v_new, pos_new, slot_pos, slot_cap);
  if (st != SP_OK) return st;
  spk::AppendIn ap;
  ap.k_new = k_new;
  ap.v_new = v_new;
  ap.pos_new = pos_new;
  ap.slot_pos = slot_pos;
  ap.slot_cap = slot_cap;
  return select_impl("sp_append_select_pages", kv, q, page_meta, top_k, n_sink, n_recent, group_reduce,
                     sel_pages, page_scores, workspace, workspace_bytes, stream, ap);
}

}  // extern "C"

namespace {
// Checks shared by sp_sparse_decode_attn and its allocation-free form; on
// success *plan holds the launch plan.
sp_status attn_checks(const sp_paged_kv* kv, const void* q, const int32_t* sel_pages, int32_t top_k,
                      float scale, float* out, float* lse, float* logits, int32_t logit_cap,
                      spk::AttnPlan* plan) {
  sp_status st = check_kv(kv);
  if (st != SP_OK) return st;
  if (!q || !out) return fail(SP_ERR_NULL_PTR, "q and out are required");
  if (!aligned(q, 16)) return fail(SP_ERR_MISALIGNED, "q must be 16-byte aligned");
  if (!aligned(out, 4) || (lse && !aligned(lse, 4)) || (logits && !aligned(logits, 4)) ||
      (sel_pages && !aligned(sel_pages, 4)))
    return fail(SP_ERR_MISALIGNED, "out, lse, logits and sel_pages must be 4-byte aligned");
  if (!isfinite(scale)) return fail(SP_ERR_BAD_SHAPE, "scale is not finite");
  const bool sparse = sel_pages != nullptr;
  if (sparse && top_k < 1) return fail(SP_ERR_BAD_SHAPE, "top_k = %d < 1", top_k);
  if (logits != nullptr) {
    if (sparse) return fail(SP_ERR_UNSUPPORTED, "logits are produced in dense mode only");
    if (logit_cap < capacity(kv))
      return fail(SP_ERR_BAD_SHAPE, "logit_cap %d below the capacity %lld", logit_cap,
                  (long long)capacity(kv));
  }
  const spk::KVDev d = spk::to_dev(kv);
  *plan = spk::plan_attention(d, kv->dtype, sparse, sparse ? top_k : 0);
  if (plan->tiles_max > (long)INT32_MAX - 65536)
    return fail(SP_ERR_UNSUPPORTED, "too many 16-token tiles in one call (%ld)", plan->tiles_max);
  if (plan->lds_bytes > 65536)
    return fail(SP_ERR_UNSUPPORTED, "shape needs %zu bytes of LDS per workgroup", plan->lds_bytes);
  return SP_OK;
}

// ---- the allocation-free attention's scratch: one array per device, looked
// up once per device (hipGetSymbolAddress) and then used only through that
// device address.  The host-side name `scratch` is not a device address and
// is never passed to a kernel or a copy.
static __device__ __align__(256) unsigned char scratch[SP_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

__global__ void zero_words_kernel(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// The current device's scratch address; on the device's first call the
// counter area is cleared by a fill kernel on `s` (stream-ordered before the
// caller's launch, and capturable, unlike a memset).
sp_status scratch_for_current_device(void** out, hipStream_t s) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "sp_sparse_decode_attn_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SP_ERR_UNSUPPORTED, "device %d is outside the %d devices the scratch table covers", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol,
                      "sp_sparse_decode_attn_noalloc: hipGetSymbolAddress(scratch)");
    const int words = (int)(SP_NOALLOC_COUNTER_BYTES / 4);
    zero_words_kernel<<<(words + 255) / 256, 256, 0, s>>>(static_cast<uint32_t*>(p), words);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "sp_sparse_decode_attn_noalloc: clearing the counters");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SP_OK;
}
}  // namespace

extern "C" {

sp_status sp_sparse_decode_attn(const sp_paged_kv* kv, const void* q, const int32_t* sel_pages,
                                int32_t top_k, float scale, float* out, float* lse,
                                float* logits, int32_t logit_cap, void* workspace,
                                size_t workspace_bytes, void* stream) {
  spk::AttnPlan plan;
  sp_status st = attn_checks(kv, q, sel_pages, top_k, scale, out, lse, logits, logit_cap, &plan);
  if (st != SP_OK) return st;
  if (workspace == nullptr || workspace_bytes < plan.ws_bytes)
    return fail(SP_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", plan.ws_bytes,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 16)) return fail(SP_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  const bool sparse = sel_pages != nullptr;
  hipError_t e = spk::launch_attention(spk::to_dev(kv), kv->dtype, plan, q, sel_pages, nullptr,
                                       sparse ? top_k : 0, scale, out, lse, logits, logit_cap, workspace,
                                       as_stream(stream));
  return e == hipSuccess ? SP_OK : hip_fail(e, "sp_sparse_decode_attn");
}

sp_status sp_sparse_decode_attn_noalloc(const sp_paged_kv* kv, const void* q, const int32_t* sel_pages,
                                        int32_t top_k, float scale, float* out, float* lse,
                                        float* logits, int32_t logit_cap, void* stream) {
  spk::AttnPlan plan;
  sp_status st = attn_checks(kv, q, sel_pages, top_k, scale, out, lse, logits, logit_cap, &plan);
  if (st != SP_OK) return st;
  const size_t units = (size_t)kv->batch * kv->num_kv_heads;
  const size_t rec_bytes = plan.ws_bytes - plan.counter_bytes;
  if (units * sizeof(int) > SP_NOALLOC_COUNTER_BYTES ||
      rec_bytes > (size_t)SP_NOALLOC_SCRATCH_BYTES - SP_NOALLOC_COUNTER_BYTES)
    return fail(SP_ERR_UNSUPPORTED,
                "shape needs %zu counter bytes and %zu record bytes; the allocation-free form holds %u and %u "
                "(use sp_sparse_decode_attn with a workspace)",
                units * sizeof(int), rec_bytes, SP_NOALLOC_COUNTER_BYTES,
                SP_NOALLOC_SCRATCH_BYTES - SP_NOALLOC_COUNTER_BYTES);
  void* base = nullptr;
  st = scratch_for_current_device(&base, as_stream(stream));
  if (st != SP_OK) return st;
  const bool sparse = sel_pages != nullptr;
  hipError_t e = spk::launch_attention_split(
      spk::to_dev(kv), kv->dtype, plan, q, sel_pages, nullptr, sparse ? top_k : 0, scale, out, lse, logits,
      logit_cap, static_cast<int*>(base),
      reinterpret_cast<float*>(static_cast<char*>(base) + SP_NOALLOC_COUNTER_BYTES), as_stream(stream));
  return e == hipSuccess ? SP_OK : hip_fail(e, "sp_sparse_decode_attn_noalloc");
}

sp_status sp_quest_decode_step(const sp_paged_kv* kv, const void* k_new, const void* v_new,
                               const int32_t* pos_new, int32_t* slot_pos, int32_t slot_cap,
                               void* page_meta, const void* q, int32_t top_k, int32_t n_sink,
                               int32_t n_recent, int32_t group_reduce, float scale, int32_t* sel_pages,
                               float* page_scores, float* out, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream) {
  sp_status st = select_checks(kv, q, page_meta, top_k, n_sink, n_recent, group_reduce, sel_pages, page_scores);
  if (st != SP_OK) return st;
  spk::AppendIn ap;
  if (k_new != nullptr || v_new != nullptr) {
    st = append_checks(kv, k_new, v_new, pos_new, slot_pos, slot_cap);
    if (st != SP_OK) return st;
    ap.k_new = k_new;
    ap.v_new = v_new;
    ap.pos_new = pos_new;
    ap.slot_pos = slot_pos;
    ap.slot_cap = slot_cap;
  }
  spk::AttnPlan plan;
  st = attn_checks(kv, q, sel_pages, top_k, scale, out, lse, nullptr, 0, &plan);
  if (st != SP_OK) return st;
  if (kv->num_blocks >= (1 << 25))
    return fail(SP_ERR_UNSUPPORTED, "num_blocks %d >= 2^25 (block ids travel in 26-bit descriptors)",
                kv->num_blocks);
  const spk::KVDev d = spk::to_dev(kv);
  const size_t need = spk::quest_step_workspace_bytes(d, kv->dtype, top_k);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(SP_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 16)) return fail(SP_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  spk::SelectOpts o;
  o.n_sink = n_sink;
  o.n_recent = n_recent;
  o.group_max = group_reduce == SP_GROUP_MAX;
  o.ap = ap;
  bool fused = false;
  hipError_t e = spk::launch_quest_step(d, kv->dtype, q, page_meta, top_k, o, sel_pages, page_scores, scale, out,
                                        lse, workspace, as_stream(stream), &fused);
  return e == hipSuccess ? SP_OK : hip_fail(e, "sp_quest_decode_step");
}

size_t sp_quest_step_error_offset(const sp_paged_kv* kv) {
  if (check_kv(kv) != SP_OK) return 0;
  return spk::quest_step_error_offset(spk::to_dev(kv));
}

sp_status sp_quest_step_single_launch(const sp_paged_kv* kv, int32_t group_reduce, int32_t* single_launch) {
  sp_status st = check_kv(kv);
  if (st != SP_OK) return st;
  if (!single_launch) return fail(SP_ERR_NULL_PTR, "single_launch is required");
  if (group_reduce != SP_GROUP_SUM && group_reduce != SP_GROUP_MAX)
    return fail(SP_ERR_BAD_SHAPE, "group_reduce %d is neither SP_GROUP_SUM nor SP_GROUP_MAX", group_reduce);
  bool single = false;
  hipError_t e = spk::quest_step_single_launch(spk::to_dev(kv), kv->dtype, group_reduce == SP_GROUP_MAX, &single);
  if (e != hipSuccess) return hip_fail(e, "sp_quest_step_single_launch");
  *single_launch = single ? 1 : 0;
  return SP_OK;
}

sp_status sp_decode_attn_accumulate(const sp_paged_kv* kv, const void* q, float scale, float* out,
                                    float* lse, float* logits, int32_t logit_cap, int32_t n_new,
                                    float* scores, int32_t slot_cap, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  sp_status st = check_kv(kv);
  if (st != SP_OK) return st;
  if (!q || !out || !lse || !logits || !scores)
    return fail(SP_ERR_NULL_PTR, "q, out, lse, logits and scores are required");
  if (!aligned(q, 16)) return fail(SP_ERR_MISALIGNED, "q must be 16-byte aligned");
  if (!aligned(out, 4) || !aligned(lse, 4) || !aligned(logits, 4) || !aligned(scores, 4))
    return fail(SP_ERR_MISALIGNED, "out, lse, logits and scores must be 4-byte aligned");
  if (!isfinite(scale)) return fail(SP_ERR_BAD_SHAPE, "scale is not finite");
  if (n_new < 0) return fail(SP_ERR_BAD_SHAPE, "n_new = %d < 0", n_new);
  if (logit_cap < capacity(kv) || slot_cap < capacity(kv))
    return fail(SP_ERR_BAD_SHAPE, "logit_cap %d / slot_cap %d below the capacity %lld", logit_cap,
                slot_cap, (long long)capacity(kv));
  const spk::KVDev d = spk::to_dev(kv);
  const spk::AttnPlan plan = spk::plan_attention(d, kv->dtype, false, 0);
  if (plan.tiles_max > (long)INT32_MAX - 65536)
    return fail(SP_ERR_UNSUPPORTED, "too many 16-token tiles in one call (%ld)", plan.tiles_max);
  if (plan.lds_bytes > 65536)
    return fail(SP_ERR_UNSUPPORTED, "shape needs %zu bytes of LDS per workgroup", plan.lds_bytes);
  if (workspace == nullptr || workspace_bytes < plan.ws_bytes)
    return fail(SP_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", plan.ws_bytes,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 16)) return fail(SP_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  hipError_t e = spk::launch_attention(d, kv->dtype, plan, q, nullptr, nullptr, 0, scale, out, lse, logits,
                                       logit_cap, workspace, as_stream(stream), scores, slot_cap, n_new);
  return e == hipSuccess ? SP_OK : hip_fail(e, "sp_decode_attn_accumulate");
}

sp_status sp_sparse_decode_attn_masked(const sp_paged_kv* kv, const void* q, const int32_t* sel_pages,
                                       const uint32_t* sel_mask, int32_t top_k, float scale, float* out,
                                       float* lse, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  sp_status st = check_kv(kv);
  if (st != SP_OK) return st;
  if (!q || !out || !sel_pages || !sel_mask)
    return fail(SP_ERR_NULL_PTR, "q, out, sel_pages and sel_mask are required");
  if (!aligned(q, 16)) return fail(SP_ERR_MISALIGNED, "q must be 16-byte aligned");
  if (!aligned(out, 4) || (lse && !aligned(lse, 4)) || !aligned(sel_pages, 4) || !aligned(sel_mask, 4))
    return fail(SP_ERR_MISALIGNED, "out, lse, sel_pages and sel_mask must be 4-byte aligned");
  if (!isfinite(scale)) return fail(SP_ERR_BAD_SHAPE, "scale is not finite");
  if (top_k < 1) return fail(SP_ERR_BAD_SHAPE, "top_k = %d < 1", top_k);
  const spk::KVDev d = spk::to_dev(kv);
  const spk::AttnPlan plan = spk::plan_attention(d, kv->dtype, true, top_k);
  if (plan.tiles_max > (long)INT32_MAX - 65536)
    return fail(SP_ERR_UNSUPPORTED, "too many 16-token tiles in one call (%ld)", plan.tiles_max);
  if (plan.lds_bytes > 65536)
    return fail(SP_ERR_UNSUPPORTED, "shape needs %zu bytes of LDS per workgroup", plan.lds_bytes);
  if (workspace == nullptr || workspace_bytes < plan.ws_bytes)
    return fail(SP_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", plan.ws_bytes,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 16)) return fail(SP_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  hipError_t e = spk::launch_attention(d, kv->dtype, plan, q, sel_pages, sel_mask, top_k, scale, out, lse,
                                       nullptr, 0, workspace, as_stream(stream));
  return e == hipSuccess ? SP_OK : hip_fail(e, "sp_sparse_decode_attn_masked");
}

sp_status sp_h2o_accumulate(const sp_paged_kv* kv, const float* logits, const float* lse,
                            int32_t logit_cap, int32_t n_new, float* scores, int32_t slot_cap,
                            void* stream) {
  sp_status st = check_kv(kv);
  if (st != SP_OK) return st;
  if (!logits || !lse || !scores) return fail(SP_ERR_NULL_PTR, "logits, lse and scores are required");
  if (n_new < 0) return fail(SP_ERR_BAD_SHAPE, "n_new = %d < 0", n_new);
  if (logit_cap < capacity(kv) || slot_cap < capacity(kv))
    return fail(SP_ERR_BAD_SHAPE, "logit_cap %d / slot_cap %d below the capacity %lld", logit_cap,
                slot_cap, (long long)capacity(kv));
  if (!aligned(logits, 4) || !aligned(lse, 4) || !aligned(scores, 4))
    return fail(SP_ERR_MISALIGNED, "logits, lse and scores must be 4-byte aligned");
  hipError_t e = spk::launch_h2o_accumulate(spk::to_dev(kv), logits, lse, logit_cap, n_new, scores,
                                            slot_cap, as_stream(stream));
  return e == hipSuccess ? SP_OK : hip_fail(e, "sp_h2o_accumulate");
}

sp_status sp_h2o_evict_compact(const sp_paged_kv* kv, float* scores, int32_t* slot_pos,
                               int32_t slot_cap, int32_t budget, int32_t recent_window,
                               void* workspace, size_t workspace_bytes, void* stream) {
  sp_status st = check_kv(kv);
  if (st != SP_OK) return st;
  if (!scores) return fail(SP_ERR_NULL_PTR, "scores is required");
  if (budget < 1) return fail(SP_ERR_BAD_SHAPE, "budget = %d < 1", budget);
  if (recent_window < 0 || recent_window > budget)
    return fail(SP_ERR_BAD_SHAPE, "recent_window = %d outside [0, budget = %d]", recent_window, budget);
  if (slot_cap < capacity(kv))
    return fail(SP_ERR_BAD_SHAPE, "slot_cap %d below the capacity %lld", slot_cap,
                (long long)capacity(kv));
  if (!aligned(scores, 4) || (slot_pos && !aligned(slot_pos, 4)))
    return fail(SP_ERR_MISALIGNED, "scores and slot_pos must be 4-byte aligned");
  const spk::KVDev d = spk::to_dev(kv);
  const size_t need = spk::h2o_evict_workspace_bytes(d, budget, kv->dtype == SP_BF16 ? 2 : 4);
  void* ws = workspace;
  if (spk::h2o_evict_list_path(d)) {
    if (workspace == nullptr || workspace_bytes < need)
      return fail(SP_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 16)) return fail(SP_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  } else if (workspace == nullptr || workspace_bytes < need) {
    ws = nullptr;                  // optional here: without it the length update is a second launch
  } else if (!aligned(workspace, 16)) {
    return fail(SP_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  }
  hipError_t e = spk::launch_h2o_evict(d, kv->dtype, scores, slot_pos, slot_cap, budget,
                                       recent_window, ws, as_stream(stream));
  return e == hipSuccess ? SP_OK : hip_fail(e, "sp_h2o_evict_compact");
}

sp_status sp_snapkv_scores(const sp_paged_kv* kv, const void* q_obs, int32_t n_obs, float scale,
                           int32_t pool_kernel, int32_t n_sink, float* scores, int32_t slot_cap,
                           void* workspace, size_t workspace_bytes, void* stream) {
  sp_status st = check_kv(kv);
  if (st != SP_OK) return st;
  if (!q_obs || !scores) return fail(SP_ERR_NULL_PTR, "q_obs and scores are required");
  if (kv->dtype != SP_BF16) return fail(SP_ERR_UNSUPPORTED, "SnapKV scoring needs a bf16 cache");
  const int G = kv->num_q_heads / kv->num_kv_heads;
  if (n_obs < 1 || (int64_t)G * n_obs > 4096)
    return fail(SP_ERR_BAD_SHAPE, "n_obs = %d: need 1 <= n_obs and G * n_obs <= 4096 (G = %d)", n_obs, G);
  if (!isfinite(scale) || !(scale > 0.f)) return fail(SP_ERR_BAD_SHAPE, "scale must be finite and > 0");
  if (pool_kernel < 1 || pool_kernel > spk::snapkv_max_pool_kernel())
    return fail(SP_ERR_BAD_SHAPE, "pool_kernel = %d outside [1, %d]", pool_kernel,
                spk::snapkv_max_pool_kernel());
  if (n_sink < 0) return fail(SP_ERR_BAD_SHAPE, "n_sink = %d < 0", n_sink);
  if ((int64_t)kv->batch * kv->num_kv_heads > 65535)
    return fail(SP_ERR_UNSUPPORTED, "batch * num_kv_heads = %lld > 65535",
                (long long)kv->batch * kv->num_kv_heads);
  if (slot_cap < capacity(kv))
    return fail(SP_ERR_BAD_SHAPE, "slot_cap %d below the capacity %lld", slot_cap,
                (long long)capacity(kv));
  if (!aligned(q_obs, 16)) return fail(SP_ERR_MISALIGNED, "q_obs must be 16-byte aligned");
  if (!aligned(scores, 4)) return fail(SP_ERR_MISALIGNED, "scores must be 4-byte aligned");
  const spk::KVDev d = spk::to_dev(kv);
  const spk::SnapPlan plan = spk::plan_snapkv(d, n_obs);
  if (workspace == nullptr || workspace_bytes < plan.ws_bytes)
    return fail(SP_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", plan.ws_bytes,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 16)) return fail(SP_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  hipError_t e = spk::launch_snapkv(d, plan, q_obs, n_obs, scale, pool_kernel, n_sink, scores, slot_cap,
                                    workspace, as_stream(stream));
  return e == hipSuccess ? SP_OK : hip_fail(e, "sp_snapkv_scores");
}

sp_status sp_h2o_prefill_scores(const sp_paged_kv* kv, const void* q_chunk, int32_t n_q, float scale,
                                float* scores, int32_t slot_cap, void* workspace,
                                size_t workspace_bytes, void* stream) {
  sp_status st = check_kv(kv);
  if (st != SP_OK) return st;
  if (!q_chunk || !scores) return fail(SP_ERR_NULL_PTR, "q_chunk and scores are required");
  if (kv->dtype != SP_BF16) return fail(SP_ERR_UNSUPPORTED, "prefill scoring needs a bf16 cache");
  if (n_q < 1 || n_q > 65536) return fail(SP_ERR_BAD_SHAPE, "n_q = %d outside [1, 65536]", n_q);
  if (!isfinite(scale) || !(scale > 0.f)) return fail(SP_ERR_BAD_SHAPE, "scale must be finite and > 0");
  if ((int64_t)kv->batch * kv->num_kv_heads > 65535)
    return fail(SP_ERR_UNSUPPORTED, "batch * num_kv_heads = %lld > 65535",
                (long long)kv->batch * kv->num_kv_heads);
  if (slot_cap < capacity(kv))
    return fail(SP_ERR_BAD_SHAPE, "slot_cap %d below the capacity %lld", slot_cap,
                (long long)capacity(kv));
  if (!aligned(q_chunk, 16)) return fail(SP_ERR_MISALIGNED, "q_chunk must be 16-byte aligned");
  if (!aligned(scores, 4)) return fail(SP_ERR_MISALIGNED, "scores must be 4-byte aligned");
  const spk::KVDev d = spk::to_dev(kv);
  const spk::SnapPlan plan = spk::plan_snapkv(d, n_q);
  if (workspace == nullptr || workspace_bytes < plan.ws_bytes)
    return fail(SP_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", plan.ws_bytes,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 16)) return fail(SP_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  hipError_t e = spk::launch_h2o_prefill_scores(d, plan, q_chunk, n_q, scale, scores, slot_cap, workspace,
                                                as_stream(stream));
  return e == hipSuccess ? SP_OK : hip_fail(e, "sp_h2o_prefill_scores");
}

sp_status sp_omnikv_select(const sp_paged_kv* kv, const void* q, int32_t top_b, int32_t* sel_pages,
                           uint32_t* sel_mask, int32_t k_pages, float* token_scores, int32_t slot_cap,
                           void* workspace, size_t workspace_bytes, void* stream) {
  sp_status st = check_kv(kv);
  if (st != SP_OK) return st;
  if (!q || !sel_pages || !sel_mask || !token_scores)
    return fail(SP_ERR_NULL_PTR, "q, sel_pages, sel_mask and token_scores are required");
  if (kv->dtype != SP_BF16) return fail(SP_ERR_UNSUPPORTED, "OmniKV scoring needs a bf16 cache");
  if (kv->num_q_heads > spk::omnikv_max_q_heads())
    return fail(SP_ERR_UNSUPPORTED, "num_q_heads = %d > %d", kv->num_q_heads, spk::omnikv_max_q_heads());
  if (kv->num_q_heads / kv->num_kv_heads > spk::omnikv_max_group())
    return fail(SP_ERR_UNSUPPORTED, "more than %d query heads per KV head", spk::omnikv_max_group());
  if (top_b < 1) return fail(SP_ERR_BAD_SHAPE, "top_b = %d < 1", top_b);
  const int need_pages = top_b < kv->max_pages_per_seq ? top_b : kv->max_pages_per_seq;
  if (k_pages < need_pages)
    return fail(SP_ERR_BAD_SHAPE, "k_pages = %d below min(top_b, max_pages) = %d", k_pages, need_pages);
  if (slot_cap < capacity(kv))
    return fail(SP_ERR_BAD_SHAPE, "slot_cap %d below the capacity %lld", slot_cap,
                (long long)capacity(kv));
  if (!aligned(q, 16)) return fail(SP_ERR_MISALIGNED, "q must be 16-byte aligned");
  if (!aligned(sel_pages, 4) || !aligned(sel_mask, 4) || !aligned(token_scores, 4))
    return fail(SP_ERR_MISALIGNED, "sel_pages, sel_mask and token_scores must be 4-byte aligned");
  const spk::KVDev d = spk::to_dev(kv);
  const size_t need = spk::token_topk_workspace_bytes(d, top_b);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(SP_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 16)) return fail(SP_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  hipError_t e = spk::launch_omnikv_select(d, q, top_b, sel_pages, sel_mask, k_pages, token_scores, slot_cap,
                                           workspace, as_stream(stream));
  return e == hipSuccess ? SP_OK : hip_fail(e, "sp_omnikv_select");
}

size_t sp_workspace_bytes(int32_t op, const sp_paged_kv* kv, int32_t top_k) {
  if (check_kv(kv) != SP_OK) return 0;
  const spk::KVDev d = spk::to_dev(kv);
  switch (op) {
    case SP_OP_SELECT_PAGES:
      return spk::select_workspace_bytes(d);
    case SP_OP_DECODE_ATTN:
      return spk::plan_attention(d, kv->dtype, top_k > 0, top_k > 0 ? top_k : 0).ws_bytes;
    case SP_OP_H2O_EVICT:
      return spk::h2o_evict_workspace_bytes(d, top_k, kv->dtype == SP_BF16 ? 2 : 4);
    case SP_OP_SNAPKV_SCORES:
    case SP_OP_H2O_PREFILL:
      return top_k >= 1 ? spk::plan_snapkv(d, top_k).ws_bytes : 0;
    case SP_OP_OMNIKV_SELECT:
      return top_k >= 1 ? spk::token_topk_workspace_bytes(d, top_k) : 0;
    case SP_OP_QUEST_STEP:
      return top_k >= 1 ? spk::quest_step_workspace_bytes(d, kv->dtype, top_k) : 0;
    default:
      return 0;
  }
}

const char* sp_status_str(int32_t status) {
  switch (status) {
    case SP_OK: return "SP_OK";
    case SP_ERR_NULL_PTR: return "SP_ERR_NULL_PTR";
    case SP_ERR_BAD_SHAPE: return "SP_ERR_BAD_SHAPE";
    case SP_ERR_UNSUPPORTED: return "SP_ERR_UNSUPPORTED";
    case SP_ERR_MISALIGNED: return "SP_ERR_MISALIGNED";
    case SP_ERR_WORKSPACE: return "SP_ERR_WORKSPACE";
    case SP_ERR_HIP: return "SP_ERR_HIP";
  }
  return "SP_ERR_UNKNOWN";
}

const char* sp_last_error(void) { return g_err.c_str(); }

int32_t sp_version(void) { return 100; }

}  // extern "C"
