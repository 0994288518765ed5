// Host check of the LDS layouts in kv_cache_selection_sp_amd/csrc/lds_layout.h
// against the direct global-to-LDS load loops that fill them, for every shape
// the entry points accept.  Each loop is restated here: wave w stages words
// [i, i + 64) for i = 64 w, 64 w + threads, ... while i < n (one dword per
// lane, whatever the number of useful lanes).  Exit status 0 when every
// loop's writes stay inside its region and the regions are disjoint and in
// order.
#include <cstdio>

#include "lds_layout.h"

namespace {

int g_bad = 0;
long g_checked = 0;

// Largest word index written by the loop, plus one (0 when n <= 0).
int loop_extent(int n, int threads) {
  int end = 0;
  for (int w = 0; w < threads / 64; ++w)
    for (int i = w * 64; i < n; i += threads)
      if (i + 64 > end) end = i + 64;
  return end;
}

void expect(bool ok, const char* what, int a, int b, int c, int d) {
  ++g_checked;
  if (!ok && g_bad++ < 20) std::printf("FAIL %s (%d, %d, %d, %d)\n", what, a, b, c, d);
}

void check_attention() {
  using namespace spk::attndev;
  const int thread_opts[2] = {256, 512};
  for (int t = 0; t < 2; ++t)
    for (int mfma = 0; mfma < 2; ++mfma)
      for (int G = 1; G <= 16; ++G)
        for (int D = 64; D <= 128; D += 64)
          for (int resolved = 0; resolved < 2; ++resolved)
            // sparse calls: the block-table row is staged for max_pages <= kLbtMax
            for (int mp = 1; mp <= 12288; mp += (mp < 256 ? 1 : 61)) {
              const int threads = thread_opts[t];
              const LdsLayout L = lds_layout(1, G, D, true, mfma, threads / 64, mp, resolved);
              const int region = L.lblk - L.lbt;
              if (stage_bt(true, mp, resolved)) {
                expect(region >= loop_extent(mp, threads), "attention block-table row", threads, G, D, mp);
                expect(region % 64 == 0, "attention block-table region a multiple of 64", threads, G, D, mp);
              } else {
                expect(region == 0, "attention: no row staged", threads, G, D, mp);
              }
              expect(L.lbt <= L.lblk && L.lblk < L.loff && L.loff < L.ltok && L.ltok < L.lnv && L.lnv < L.wst &&
                         L.wst <= L.comb && L.comb < L.mrg && L.mrg < L.total,
                     "attention regions in order", threads, G, D, mp);
            }
  // dense calls (no direct loads): the length prefix and lengths before the lists
  for (int B = 1; B <= 2048; ++B) {
    const LdsLayout L = lds_layout(B, 4, 128, false, true, 8, 512);
    expect(L.lens - L.pre >= B + 1 && L.lbt - L.lens >= B && L.lbt == L.lblk, "attention dense prefix", B, 0, 0, 0);
  }
}

void check_eviction() {
  using namespace spk::evlds;
  const int kThreads = 256, kFastMax = 8192;
  for (int P = 16; P <= 32; P += 16)
    for (int mp = 1; mp * P <= kFastMax; ++mp) {
      const int cap = mp * P;
      const EvLayout L = ev_layout(cap, mp);
      // candidate scores: nc = L - window words, 1 <= nc <= cap
      expect(L.srcmap - L.keys >= loop_extent(cap, kThreads), "eviction keys", P, mp, cap, 0);
      for (int nc = 1; nc <= cap; nc += (nc < 512 ? 1 : 37))
        expect(L.srcmap - L.keys >= loop_extent(nc, kThreads), "eviction keys (nc)", P, mp, nc, 0);
      expect(L.hist - L.lbt >= loop_extent(mp, kThreads), "eviction block-table row", P, mp, cap, 0);
      expect(L.keys == 0 && L.keys < L.srcmap && L.srcmap < L.lbt && L.lbt < L.hist && L.hist < L.cand &&
                 L.cand < L.sh && L.sh < L.total,
             "eviction regions in order", P, mp, cap, 0);
      expect(L.srcmap - L.keys >= cap && 2 * (L.lbt - L.srcmap) >= cap, "eviction keys and 16-bit map hold cap",
             P, mp, cap, 0);
      expect(L.total * 4 <= 64 * 1024, "eviction fast path within 64 KiB of LDS", P, mp, L.total * 4, 0);
    }
}

}  // namespace

int main() {
  check_attention();
  check_eviction();
  std::printf("%ld checks, %d failed\n", g_checked, g_bad);
  return g_bad == 0 ? 0 : 1;
}
