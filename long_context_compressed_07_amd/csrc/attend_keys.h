// The key list of one query, shared by the attention kernels.
//
// CSA (deepseek.csdn.net "一文搞懂 DeepSeek" V4 改进一): the k selected entries (slots holding -1
// are skipped) followed by the raw rows of the positions max(0, pos - window + 1) .. pos, with no
// de-duplication. HCA (same section; yudonglee.me "DeepSeek-V4 详解" 2.3 Step 2): every visible
// entry, j < n_vis(pos) for the m'-fold store, and no window. Token selection (hongke120.com
// 2.2 item 3; yudonglee.me 2.2 Steps 3-4: the selected blocks' original tokens are attended):
// slot s holding block j contributes the m raw rows of positions j m .. j m + m - 1, in order,
// then the window; all rows come from the raw store.
#pragma once

#include "common.h"

namespace csa {

struct KeyList {
  int64_t b;            // sequence
  int64_t pos;          // absolute position of the query
  const int32_t* sel;   // selected entry slots of this query (CSA) or nullptr (HCA)
  int64_t n_sel;        // number of entry slots (k for CSA, n_vis for HCA)
  int64_t ent_rows;     // rows of the entry store (selected slots at or past it are skipped)
  int64_t wlo;          // first window position
  int64_t n_win;        // window rows
  int64_t w_row0;       // raw-store row of position wlo: (wlo - pos0) mod rows
  int64_t raw_rows;     // rows of the raw store (the ring length)
  int64_t tok_m;        // token selection: tokens per selected block (0: the slots are entries)
  int64_t tok_base;     // token selection: raw row of position p is p + tok_base (= -pos0)
  int64_t total;
};

// Selection slot of key kk (kk < n_sel): kk itself, or its block's slot in token selection.
__device__ __forceinline__ int64_t sel_index(const KeyList& kl, int64_t kk) {
  return kl.tok_m > 0 ? kk / kl.tok_m : kk;
}

// Raw-store row of absolute position p: the store is a ring, row (p - pos0) mod rows. A store that
// holds every position from pos0 on (rows >= the positions it covers) is the special case where
// no wrap happens.
__device__ __forceinline__ int64_t ring_row(int64_t p, int64_t pos0, int64_t rows) {
  const int64_t r = (p - pos0) % rows;
  return r < 0 ? r + rows : r;
}

__device__ __forceinline__ KeyList make_key_list(const AttendArgs& a, int qi) {
  KeyList kl;
  kl.b = a.Q.seq[qi];
  kl.pos = a.Q.pos[qi];
  kl.tok_m = a.tok_m;
  kl.tok_base = 0;
  if (!a.dense) {
    kl.sel = a.idx + (int64_t)qi * a.k;
    kl.n_sel = a.tok_m > 0 ? (int64_t)a.k * a.tok_m : a.k;
  } else {
    kl.sel = nullptr;
    kl.n_sel = n_visible(kl.pos, a.m, a.ent.rows);
  }
  kl.ent_rows = a.ent.rows;
  if (a.window > 0 && a.raw.c != nullptr && a.raw.rows > 0) {
    kl.wlo = kl.pos - a.window + 1 > 0 ? kl.pos - a.window + 1 : 0;
    kl.n_win = kl.pos - kl.wlo + 1;
    kl.raw_rows = a.raw.rows;
    kl.w_row0 = ring_row(kl.wlo, a.raw.pos0 != nullptr ? a.raw.pos0[kl.b] : 0, a.raw.rows);
  } else {
    kl.wlo = 0;
    kl.n_win = 0;
    kl.raw_rows = 1;
    kl.w_row0 = 0;
  }
  if (a.tok_m > 0) {
    kl.raw_rows = a.raw.rows;
    kl.tok_base = -(a.raw.pos0 != nullptr ? a.raw.pos0[kl.b] : 0);
  }
  kl.total = kl.n_sel + kl.n_win;
  return kl;
}

// Row of key kk in its store (src = 0: entries, 1: raw); -1 for an empty selection slot (or one
// naming a row past the entry store).
__device__ __forceinline__ int64_t key_row(const AttendArgs& a, const KeyList& kl, int64_t kk,
                                           int& src) {
  if (kk < kl.n_sel) {
    if (kl.tok_m > 0) {
      src = 1;
      const int64_t blk = kl.sel[kk / kl.tok_m];
      const int64_t r = blk * kl.tok_m + kk % kl.tok_m + kl.tok_base;
      return blk >= 0 && r >= 0 && r < kl.raw_rows ? r : -1;
    }
    src = 0;
    if (kl.sel == nullptr) return kk;
    const int64_t r = kl.sel[kk];
    return r < kl.ent_rows ? r : -1;
  }
  src = 1;
  const int64_t r = kl.w_row0 + (kk - kl.n_sel);
  return r < kl.raw_rows ? r : r - kl.raw_rows;
}

}  // namespace csa
