// LDS layouts (in 4-byte words) of the kernels that stage data with direct
// global-to-LDS loads, written as plain C++ so that a host-only checker can
// verify them for every shape the entry points accept.
//
// A direct load of 4 bytes per lane writes one dword per lane of the 64-lane
// wave, at the wave's LDS base + 4 * lane, whatever the number of useful
// lanes.  A loop that stages n words with each wave starting at a multiple of
// 64 therefore writes up to lds_direct_words(n) words, and every region such
// a loop fills is sized at least that (a region sized n would let the last
// wave's tail overwrite the next region).
#pragma once

#if defined(__HIPCC__)
#define SPK_HD __host__ __device__
#else
#define SPK_HD
#endif

namespace spk {

constexpr int kLdsWave = 64;   // lanes written by one direct load
SPK_HD constexpr int lds_direct_words(int n) { return (n + kLdsWave - 1) / kLdsWave * kLdsWave; }

// ------------------------------------------------------------ attention
namespace attndev {
constexpr int kTok = 16;          // tokens per tile
constexpr int kList = 512;        // tiles resolved into LDS per batch
constexpr int kMergeBatch = 32;   // split records merged per LDS pass
// Sparse calls stage the block-table row of the unit's sequence in LDS (one
// direct-load loop over max_pages words) when it holds at most kLbtMax pages.
constexpr int kLbtMax = 8192;
// Dense calls keep the per-sequence tile prefix and lengths in LDS for up to
// kDenseLdsMax sequences; larger batches take them from a workspace area
// (lds_layout is then given B = 0).
constexpr int kDenseLdsMax = 2048;

struct LdsLayout {
  int pre, lens, lbt, lblk, loff, ltok, lnv, wst, comb, mrg, total;
};
// Resolved (fused-step) calls read block ids from their descriptors instead.
SPK_HD inline bool stage_bt(bool sparse, int max_pages, bool resolved = false) {
  return sparse && !resolved && max_pages <= kLbtMax;
}
SPK_HD inline LdsLayout lds_layout(int B, int G, int D, bool sparse, bool mfma, int kWaves, int max_pages,
                                   bool resolved = false) {
  LdsLayout s;
  int off = 0;
  s.pre = off;  off += sparse ? 0 : ((B + 1 + 3) & ~3);
  s.lens = off; off += sparse ? 0 : ((B + 3) & ~3);
  s.lbt = off;  off += stage_bt(sparse, max_pages, resolved) ? lds_direct_words(max_pages) : 0;
  s.lblk = off; off += kList;
  s.loff = off; off += kList;
  s.ltok = off; off += kList;
  s.lnv = off;  off += kList;
  s.wst = off;
  off += mfma ? (kWaves * G * (D + 4) + 2 * kWaves * G)
              : (G * D + G * (kTok + 1) + 3 * G);
  off = (off + 3) & ~3;
  s.comb = off; off += G * D + 2 * G;
  s.mrg = off;  off += 2 * kMergeBatch * G + 3 * G;
  s.total = off;
  return s;
}
}  // namespace attndev

// ------------------------------------------------------------ fast eviction
namespace evlds {
constexpr int kEvBins = 1 << 11;  // radix bins of the threshold search
constexpr int kEvCand = 64;       // boundary-bin candidates counted by one wave
// Two direct-load loops: the candidate scores (nc <= cap words) into keys and
// the block-table row (max_pages words) into lbt.
struct EvLayout { int keys, srcmap, lbt, hist, cand, sh, total; };
SPK_HD inline EvLayout ev_layout(int cap, int max_pages) {
  EvLayout l;
  int off = 0;
  l.keys = off;   off += (cap + 255) & ~255;              // a multiple of 256 >= lds_direct_words(cap)
  l.srcmap = off; off += ((cap + 1) / 2 + 3) & ~3;        // uint16 slot indices
  l.lbt = off;    off += lds_direct_words(max_pages);
  l.hist = off;   off += kEvBins;
  l.cand = off;   off += kEvCand;
  l.sh = off;     off += 16;
  l.total = off;
  return l;
}
}  // namespace evlds

}  // namespace spk
