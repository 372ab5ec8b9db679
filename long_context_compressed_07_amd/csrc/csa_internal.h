// Internal interface between the C-ABI layer (api.hip) and the kernel translation units.
// Not installed; the public interface is include/csa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csa.h"

namespace csa {

// A cache-row store as seen by kernels (plain values; device pointers).
struct Store {
  const void* c;
  const void* r;
  const float* scale;
  const int64_t* pos0;
  int dtype;        // csa_dtype of c; r is bf16 unless dtype == CSA_F32 (then fp32)
  int d_c, d_r;
  int64_t rows;     // rows per sequence
  int64_t ld_c, ld_r;
};

struct OutStore {
  void* c;
  void* r;
  float* scale;
  int dtype;
  int d_c, d_r;
  int64_t rows;
  int64_t ld_c, ld_r;
};

struct Queries {
  const int32_t* seq;
  const int64_t* pos;
  int nq;
};

// ---- compress ----------------------------------------------------------------------------
struct CompressArgs {
  const void* x;
  const void* g;
  int in_dtype;
  const float* bias;
  int m;
  int B;
  int64_t T;
  int d_c, d_r;
  const float* hidden;
  const float* w_x;
  const float* w_g;
  int d_model;
  OutStore out;
  float* raw_x_out;
};
hipError_t launch_compress(const CompressArgs& a, hipStream_t s);

// ---- index ---------------------------------------------------------------------------------
struct IndexArgs {
  Queries Q;
  const void* q_i;
  const float* q_i_scale;
  int dtype;            // of q_i and k_i
  const float* w;
  int H_I, d_I;
  const void* k_i;
  const float* k_i_scale;
  int B;
  int64_t N;
  int m;
  float* scores;
  int64_t ld_scores;
};
hipError_t launch_index(const IndexArgs& a, hipStream_t s);

// MXFP4 indexer with bf16 scores (index_fp4.hip): E2M1 codes, two per byte (low nibble first),
// with one E8M0 scale per 32 values; d_I = 64, H_I = 8.
struct IndexFp4Args {
  Queries Q;
  const uint8_t* q_i;        // [nq][8][32] packed codes
  const uint8_t* q_i_scale;  // [nq][8][2]
  const float* w;            // [nq][8]
  const uint8_t* k_i;        // [B][N][32]
  const uint8_t* k_i_scale;  // [B][N][2]
  int B;
  int64_t N;
  int m;
  uint16_t* scores;          // [nq][ld_scores] bf16
  int64_t ld_scores;
};
hipError_t launch_index_fp4(const IndexFp4Args& a, hipStream_t s);

// ---- top-k ---------------------------------------------------------------------------------
struct TopkArgs {
  Queries Q;
  const void* scores;   // fp32, or bf16 codes when bf16 != 0
  int bf16;
  int64_t ld_scores;
  int64_t N;
  int m;
  int k;
  int32_t* idx;
  void* ws;
  size_t ws_bytes;
};
size_t topk_workspace(int nq, int64_t N, int k);
bool topk_supported(int64_t N, int k);
// The no-allocation top-k's scratch: a device array of kTopkScratchBytes per GPU; *ptr receives
// the current device's address of it.
constexpr size_t kTopkScratchBytes = (size_t)16 << 20;
hipError_t topk_scratch(void** ptr);
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);

// Instrumentation: event timing of the main attention kernel (see csa.h).
constexpr int kTimingCap = 1024;
hipError_t kernel_timing_enable(int cap);
hipError_t kernel_timing_read(int slot, double* ms, int* n);
int timing_start(int slot, hipStream_t s);   // >= 0: index of the event pair opened for this launch
void timing_stop(int slot, int i, hipStream_t s);

// ---- attention -----------------------------------------------------------------------------
struct AttendArgs {
  Queries Q;
  const void* q;
  int q_dtype;
  int H;
  Store ent;
  int m;
  int dense;            // 1: HCA, every visible entry is a key; 0: CSA, the k slots of idx
  const int32_t* idx;   // [nq][k] selected entries (CSA); unused when dense or k == 0
  int k;
  int tok_m;            // > 0: token selection, each slot's block contributes its tok_m raw rows
  Store raw;            // raw.c == NULL or window == 0: no window
  int window;
  float sm_scale;
  float* out;
  float* lse;
  void* ws;
  size_t ws_bytes;
};
size_t attend_workspace(int nq, int H, int d_c, int64_t max_keys, bool dense);
hipError_t launch_attend(const AttendArgs& a, hipStream_t s);

}  // namespace csa
