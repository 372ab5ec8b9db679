// The key list of one query, shared by the attention kernels.
//
// CSA (deepseek.csdn.net "一文搞懂 DeepSeek" V4 改进一): the k selected entries (slots holding -1
// are skipped) followed by the raw rows of the positions max(0, pos - window + 1) .. pos, with no
// de-duplication. HCA (same section; yudonglee.me "DeepSeek-V4 详解" 2.3 Step 2): every visible
// entry, j < n_vis(pos) for the m'-fold store, and no window.
#pragma once

#include "common.h"

namespace csa {

struct KeyList {
  int64_t b;            // sequence
  int64_t pos;          // absolute position of the query
  const int32_t* sel;   // selected entry slots of this query (CSA) or nullptr (HCA)
  int64_t n_sel;        // number of entry slots (k for CSA, n_vis for HCA)
  int64_t wlo;          // first window position
  int64_t n_win;        // window rows
  int64_t raw_base;     // absolute position of raw row 0 of this sequence
  int64_t total;
};

__device__ __forceinline__ KeyList make_key_list(const AttendArgs& a, int qi) {
  KeyList kl;
  kl.b = a.Q.seq[qi];
  kl.pos = a.Q.pos[qi];
  if (!a.dense) {
    kl.sel = a.idx + (int64_t)qi * a.k;
    kl.n_sel = a.k;
  } else {
    kl.sel = nullptr;
    kl.n_sel = n_visible(kl.pos, a.m, a.ent.rows);
  }
  if (a.window > 0 && a.raw.c != nullptr) {
    kl.wlo = kl.pos - a.window + 1 > 0 ? kl.pos - a.window + 1 : 0;
    kl.n_win = kl.pos - kl.wlo + 1;
    kl.raw_base = a.raw.pos0 != nullptr ? a.raw.pos0[kl.b] : 0;
  } else {
    kl.wlo = 0;
    kl.n_win = 0;
    kl.raw_base = 0;
  }
  kl.total = kl.n_sel + kl.n_win;
  return kl;
}

// Row of key kk in its store (src = 0: entries, 1: raw); -1 for an empty selection slot.
__device__ __forceinline__ int64_t key_row(const AttendArgs& a, const KeyList& kl, int64_t kk,
                                           int& src) {
  if (kk < kl.n_sel) {
    src = 0;
    return kl.sel != nullptr ? (int64_t)kl.sel[kk] : kk;
  }
  src = 1;
  return kl.wlo + (kk - kl.n_sel) - kl.raw_base;
}

}  // namespace csa
