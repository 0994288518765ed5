// KV append fused with the Quest page-summary fold, and the full summary
// rebuild.
//
// "SparseEngine: Sparse-First Inference Engine", Appendix A.3, "Quest:
// Query-Dependent Page Selection": every page stores the per-channel minimum
// and maximum of its keys, and new keys update the extrema of their page, so
// the summaries persist beside the KV.  Appendix A.2, "Logical Positions and
// Physical Blocks": slot s of a sequence is on logical page s / P, resolved to
// a physical block through the block table.
//
// min/max of representable values is exact, so the summaries are stored in the
// KV dtype and an incremental fold equals a rebuild bit for bit.
#include "sp_internal.h"

namespace spk {
namespace {

constexpr int kAppendThreads = 256;
constexpr int kSmallAppend = 16;   // appends of at most this many tokens take the one-launch path

// One workgroup per (logical page touched by the new tokens, KV head,
// sequence).  blockIdx.x enumerates the pages [L0 / P, (L0 + n_new - 1) / P]
// where L0 = seq_lens[b] before the append.
template <typename T>
__global__ void __launch_bounds__(kAppendThreads)
append_fold_kernel(KVDev kv, const T* __restrict__ k_new, const T* __restrict__ v_new, int n_new,
                   T* __restrict__ meta, const int32_t* __restrict__ pos_new,
                   int32_t* __restrict__ slot_pos, int slot_cap) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int P = kv.P, D = kv.D, Hkv = kv.Hkv;
  const int cap = kv.max_pages * P;
  const int L0 = clamp_len(kv.seq_lens[b], cap);
  const int page = L0 / P + (int)blockIdx.x;
  const int s_lo = max(L0, page * P);
  const int s_hi = min(min(L0 + n_new, (page + 1) * P), cap);
  if (s_lo >= s_hi) return;
  const int blk = kv.block_table[(size_t)b * kv.max_pages + page];
  if (blk < 0 || blk >= kv.num_blocks) return;
  const int nt = s_hi - s_lo;
  T* kp = reinterpret_cast<T*>(kv.k_pool) + page_base(blk, h, Hkv, P, D);
  T* vp = reinterpret_cast<T*>(kv.v_pool) + page_base(blk, h, Hkv, P, D);
  const size_t tok_stride = (size_t)Hkv * D;   // k_new[b][t][h][d]
  const T* kn = k_new + ((size_t)b * n_new) * tok_stride + (size_t)h * D;
  const T* vn = v_new + ((size_t)b * n_new) * tok_stride + (size_t)h * D;
  const int t0 = s_lo - L0;   // index of the first new token landing on this page

  // K: 16-byte chunks (token, chunk) -> consecutive threads write consecutive
  // tokens of one chunk row, which are adjacent in the chunk-tiled page.
  constexpr int E = Chunk<T>::E;
  const int nchunk = D / E;
  for (int i = threadIdx.x; i < nt * nchunk; i += kAppendThreads) {
    const int tt = i % nt, c = i / nt;
    const uint4 val = *reinterpret_cast<const uint4*>(kn + (size_t)(t0 + tt) * tok_stride + c * E);
    const int slot_in_page = s_lo - page * P + tt;
    *reinterpret_cast<uint4*>(kp + (size_t)(c * P + slot_in_page) * E) = val;
  }
  // V: dim-major page, element (t, d) at d * P + t.
  for (int i = threadIdx.x; i < nt * D; i += kAppendThreads) {
    const int tt = i % nt, d = i / nt;
    vp[v_off(s_lo - page * P + tt, d, P)] = vn[(size_t)(t0 + tt) * tok_stride + d];
  }
  // Page summary: start afresh when the page's first slot is among the new
  // tokens, else fold into the stored extrema.
  if (meta != nullptr) {
    T* mrow = meta + ((size_t)blk * Hkv + h) * 2 * D;
    const bool fresh = (s_lo == page * P);
    for (int d = threadIdx.x; d < D; d += kAppendThreads) {
      float mn, mx;
      int tt = 0;
      if (fresh) {
        mn = mx = to_f32(kn[(size_t)t0 * tok_stride + d]);
        tt = 1;
      } else {
        mn = to_f32(mrow[d]);
        mx = to_f32(mrow[D + d]);
      }
      for (; tt < nt; ++tt) {
        const float x = to_f32(kn[(size_t)(t0 + tt) * tok_stride + d]);
        mn = x < mn ? x : mn;
        mx = x > mx ? x : mx;
      }
      mrow[d] = from_f32<T>(mn);
      mrow[D + d] = from_f32<T>(mx);
    }
  }
  if (slot_pos != nullptr) {
    const int base = pos_new ? pos_new[b] : L0;
    int32_t* sp = slot_pos + ((size_t)b * Hkv + h) * slot_cap;
    for (int tt = threadIdx.x; tt < nt; tt += kAppendThreads) sp[s_lo + tt] = base + t0 + tt;
  }
}

// Small appends (decode: a few tokens per sequence): one workgroup per
// sequence writes every KV head's tokens, folds the summaries and then bumps
// seq_lens[b] itself, so the append is a single launch.  A task is one
// (KV head, 16-byte chunk of the head dim); it loads the new keys and values
// of its chunk and the stored summary of the first touched page together,
// then writes the pool and the folded summaries.  At most two pages are
// touched (n_new <= 16 <= P), and the second one always starts afresh.  All
// threads read the old length before the barrier that precedes the update.
template <typename T>
__global__ void __launch_bounds__(kAppendThreads)
append_small_kernel(KVDev kv, const T* __restrict__ k_new, const T* __restrict__ v_new, int n_new,
                    T* __restrict__ meta, const int32_t* __restrict__ pos_new,
                    int32_t* __restrict__ slot_pos, int slot_cap) {
  constexpr int E = Chunk<T>::E;
  const int b = blockIdx.x;
  const int P = kv.P, D = kv.D, Hkv = kv.Hkv;
  const int cap = kv.max_pages * P;
  const int L0 = clamp_len(kv.seq_lens[b], cap);
  const int nt = min(n_new, cap - L0);            // tokens that fit
  const int32_t* bt_row = kv.block_table + (size_t)b * kv.max_pages;
  const int pg0 = L0 / P;
  const int blk0 = nt > 0 ? bt_row[pg0] : -1;
  const int blk1 = (nt > 0 && (L0 + nt - 1) / P != pg0) ? bt_row[pg0 + 1] : -1;
  const bool ok0 = blk0 >= 0 && blk0 < kv.num_blocks, ok1 = blk1 >= 0 && blk1 < kv.num_blocks;
  const size_t tok_stride = (size_t)Hkv * D;      // k_new[b][t][h][d]
  const T* kn = k_new + (size_t)b * n_new * tok_stride;
  const T* vn = v_new + (size_t)b * n_new * tok_stride;
  const int nchunk = D / E;
  T* kpool = reinterpret_cast<T*>(kv.k_pool);
  T* vpool = reinterpret_cast<T*>(kv.v_pool);
  for (int task = threadIdx.x; task < Hkv * nchunk; task += kAppendThreads) {
    const int h = task / nchunk, c = task % nchunk;
    union U { uint4 u; T e[E]; };
    // stored summary of the first page, when it already holds tokens
    U mn0, mx0;
    const bool fold0 = meta != nullptr && ok0 && (L0 % P) != 0;
    T* mrow0 = ok0 && meta ? meta + ((size_t)blk0 * Hkv + h) * 2 * D + c * E : nullptr;
    T* mrow1 = ok1 && meta ? meta + ((size_t)blk1 * Hkv + h) * 2 * D + c * E : nullptr;
    if (fold0) {
      mn0.u = *reinterpret_cast<const uint4*>(mrow0);
      mx0.u = *reinterpret_cast<const uint4*>(mrow0 + D);
    }
    float mn[E], mx[E];
    bool have = false;                 // mn/mx hold the page being folded
    int cur_pg = pg0;
    for (int t = 0; t < nt; ++t) {
      const int s = L0 + t, pg = s / P, off = s % P;
      U kk, vv;
      kk.u = *reinterpret_cast<const uint4*>(kn + (size_t)t * tok_stride + (size_t)h * D + c * E);
      vv.u = *reinterpret_cast<const uint4*>(vn + (size_t)t * tok_stride + (size_t)h * D + c * E);
      const bool okp = pg == pg0 ? ok0 : ok1;
      const int blk = pg == pg0 ? blk0 : blk1;
      if (okp) {
        const size_t base = page_base(blk, h, Hkv, P, D);
        *reinterpret_cast<uint4*>(kpool + base + (size_t)(c * P + off) * E) = kk.u;
#pragma unroll
        for (int e = 0; e < E; ++e) vpool[base + v_off(off, c * E + e, P)] = vv.e[e];
      }
      if (meta != nullptr) {
        if (pg != cur_pg && have) {              // page change: write the first page back
          U a, z;
#pragma unroll
          for (int e = 0; e < E; ++e) { a.e[e] = from_f32<T>(mn[e]); z.e[e] = from_f32<T>(mx[e]); }
          if (mrow0) { *reinterpret_cast<uint4*>(mrow0) = a.u; *reinterpret_cast<uint4*>(mrow0 + D) = z.u; }
          have = false;
        }
        cur_pg = pg;
        if (!have) {
          if (pg == pg0 && fold0) {
#pragma unroll
            for (int e = 0; e < E; ++e) { mn[e] = to_f32(mn0.e[e]); mx[e] = to_f32(mx0.e[e]); }
          } else {
#pragma unroll
            for (int e = 0; e < E; ++e) mn[e] = mx[e] = to_f32(kk.e[e]);
          }
          have = true;
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float x = to_f32(kk.e[e]);
          mn[e] = x < mn[e] ? x : mn[e];
          mx[e] = x > mx[e] ? x : mx[e];
        }
      }
    }
    if (meta != nullptr && have) {
      U a, z;
#pragma unroll
      for (int e = 0; e < E; ++e) { a.e[e] = from_f32<T>(mn[e]); z.e[e] = from_f32<T>(mx[e]); }
      T* mrow = cur_pg == pg0 ? mrow0 : mrow1;
      if (mrow) { *reinterpret_cast<uint4*>(mrow) = a.u; *reinterpret_cast<uint4*>(mrow + D) = z.u; }
    }
  }
  if (slot_pos != nullptr) {
    const int base = pos_new ? pos_new[b] : L0;
    for (int i = threadIdx.x; i < nt * Hkv; i += kAppendThreads) {
      const int h = i % Hkv, t = i / Hkv;
      slot_pos[((size_t)b * Hkv + h) * slot_cap + L0 + t] = base + t;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) kv.seq_lens[b] = L0 + nt;
}

__global__ void bump_lens_kernel(int32_t* seq_lens, int B, int n_new, int cap) {
  for (int b = blockIdx.x * blockDim.x + threadIdx.x; b < B; b += gridDim.x * blockDim.x) {
    const int L = clamp_len(seq_lens[b], cap);
    seq_lens[b] = min(L + n_new, cap);
  }
}

// Rebuild: one thread per (page, 16-byte key chunk); it scans the page's valid
// tokens of its chunk (contiguous in the chunk-tiled layout).
template <typename T>
__global__ void __launch_bounds__(256)
rebuild_meta_kernel(KVDev kv, T* __restrict__ meta) {
  constexpr int E = Chunk<T>::E;
  const int b = blockIdx.z, h = blockIdx.y;
  const int P = kv.P, D = kv.D, Hkv = kv.Hkv;
  const int nchunk = D / E;
  const int pages_per_block = 256 / nchunk;
  const int page = blockIdx.x * pages_per_block + threadIdx.x / nchunk;
  const int c = threadIdx.x % nchunk;
  const int L = clamp_len(kv.seq_lens[b], kv.max_pages * P);
  if (page * P >= L) return;
  const int blk = kv.block_table[(size_t)b * kv.max_pages + page];
  if (blk < 0 || blk >= kv.num_blocks) return;
  const int nt = min(P, L - page * P);
  const T* kp = reinterpret_cast<const T*>(kv.k_pool) + page_base(blk, h, Hkv, P, D) + (size_t)c * P * E;
  float mn[E], mx[E];
  for (int t = 0; t < nt; ++t) {
    union { uint4 u; T e[E]; } w;
    w.u = *reinterpret_cast<const uint4*>(kp + (size_t)t * E);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float x = to_f32(w.e[e]);
      mn[e] = (t == 0 || x < mn[e]) ? x : mn[e];
      mx[e] = (t == 0 || x > mx[e]) ? x : mx[e];
    }
  }
  T* mrow = meta + ((size_t)blk * Hkv + h) * 2 * D + c * E;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    mrow[e] = from_f32<T>(mn[e]);
    mrow[D + e] = from_f32<T>(mx[e]);
  }
}

template <typename T>
hipError_t append_t(const KVDev& kv, const void* k_new, const void* v_new, int n_new,
                    void* meta, const int32_t* pos_new, int32_t* slot_pos, int slot_cap,
                    hipStream_t s) {
  if (n_new <= kSmallAppend) {
    append_small_kernel<T><<<kv.B, kAppendThreads, 0, s>>>(
        kv, static_cast<const T*>(k_new), static_cast<const T*>(v_new), n_new,
        static_cast<T*>(meta), pos_new, slot_pos, slot_cap);
    return hipGetLastError();
  }
  const int pages_touched = (n_new + kv.P - 1) / kv.P + 1;
  dim3 grid(pages_touched, kv.Hkv, kv.B);
  append_fold_kernel<T><<<grid, kAppendThreads, 0, s>>>(
      kv, static_cast<const T*>(k_new), static_cast<const T*>(v_new), n_new,
      static_cast<T*>(meta), pos_new, slot_pos, slot_cap);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  bump_lens_kernel<<<1, 256, 0, s>>>(kv.seq_lens, kv.B, n_new, kv.max_pages * kv.P);
  return hipGetLastError();
}

template <typename T>
hipError_t rebuild_t(const KVDev& kv, void* meta, hipStream_t s) {
  const int nchunk = kv.D / Chunk<T>::E;
  const int ppb = 256 / nchunk;
  dim3 grid((kv.max_pages + ppb - 1) / ppb, kv.Hkv, kv.B);
  rebuild_meta_kernel<T><<<grid, 256, 0, s>>>(kv, static_cast<T*>(meta));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const KVDev& kv, int dtype, const void* k_new, const void* v_new,
                         int n_new, void* page_meta, const int32_t* pos_new, int32_t* slot_pos,
                         int slot_cap, hipStream_t s) {
  if (dtype == SP_BF16)
    return append_t<bf16_t>(kv, k_new, v_new, n_new, page_meta, pos_new, slot_pos, slot_cap, s);
  return append_t<float>(kv, k_new, v_new, n_new, page_meta, pos_new, slot_pos, slot_cap, s);
}

hipError_t launch_rebuild_meta(const KVDev& kv, int dtype, void* page_meta, hipStream_t s) {
  if (dtype == SP_BF16) return rebuild_t<bf16_t>(kv, page_meta, s);
  return rebuild_t<float>(kv, page_meta, s);
}

}  // namespace spk
