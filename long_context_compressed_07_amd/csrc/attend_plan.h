// Work decomposition shared by the MFMA attention kernels, their split-K combine and the fp32
// fixup pass.
#pragma once

#include "csa_internal.h"

namespace csa {

struct AttnPlan {
  int ksw;            // fp16-staging kernel: key splits inside a workgroup (4 / ksw head groups)
  int rg;             // DMA kernels: 32-head row groups per workgroup (bf16: 2, fp8: 4)
  int head_groups;    // workgroups per query along heads
  int n_split;        // workgroups per query along keys
  int f8_dma;         // 1: fp8 rows staged by DMA and converted in LDS (attend_fp8.hip)
  int pp;             // 1: bf16, 64 heads per workgroup, QK and PV wave roles (attend_pp.hip)
  _Float16* ws_o;     // [nq][n_split][H][512] partial outputs normalised by their l, n_split > 1
  float* ws_ml;       // [nq][n_split][H][2] partial (max in log2 units, sum)
  int* flags;         // [nq][head_groups][n_split] 1 = some head left the range of P
};

// The work item of this workgroup. Workgroups go to the 8 XCDs in turn (workgroup b to XCD
// b mod 8); this mapping gives each XCD a contiguous range of items, so that the key splits and
// head groups of one query, and neighbouring queries, share that XCD's L2. The last
// gridDim.x mod 8 workgroups keep their own index.
__device__ __forceinline__ int xcd_item() {
  const int b = blockIdx.x, n = gridDim.x;
  const int n8 = n & ~7;
  if (b >= n8) return b;
  return (b & 7) * (n8 >> 3) + (b >> 3);
}

// Four values of a normalised partial output row (o / l in fp16; zeros when l == 0).
__device__ __forceinline__ void store_partial4(_Float16* dst, float a, float b, float c, float d,
                                               float inv) {
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  *reinterpret_cast<h4*>(dst) = h4{(_Float16)(a * inv), (_Float16)(b * inv), (_Float16)(c * inv),
                                   (_Float16)(d * inv)};
}

hipError_t launch_attend_fp8(const AttendArgs& a, const AttnPlan& p, hipStream_t s);
hipError_t launch_attend_pp(const AttendArgs& a, const AttnPlan& p, hipStream_t s);

}  // namespace csa
