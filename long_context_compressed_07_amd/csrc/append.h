// Arguments of the decode-time cache append (append.hip; C entry point csa_cache_append).
#pragma once
#include "csa_internal.h"

namespace csa {

struct AppendArgs {
  const void* x_new;        // [B][d] new token rows, in_dtype
  const void* g_new;        // [B][d] their gates
  int in_dtype;             // CSA_F32 or CSA_BF16
  const float* bias;        // [m]
  int m;
  int B;
  const int64_t* pos;       // [B] absolute position of each sequence's new token (device)
  int d_c, d_r;
  float* stage_x;           // [B][m][d] fp32 staging ring of the block being filled
  float* stage_g;
  OutStore ent;             // entry store (rows = entries per sequence)
  OutStore raw;             // raw store, a ring of rows per sequence (c == null: none)
  const int64_t* raw_pos0;  // [B] ring offset: position p goes to row (p - pos0) mod rows; null: 0
};

hipError_t launch_append(const AppendArgs& a, hipStream_t s);

}  // namespace csa
