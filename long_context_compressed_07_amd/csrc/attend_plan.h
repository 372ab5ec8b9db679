// Work decomposition shared by the MFMA attention kernels, their split-K combine and the fp32
// fixup pass.
#pragma once

#include "csa_internal.h"

namespace csa {

struct AttnPlan {
  int ksw;            // key splits inside a workgroup (4 waves = 4 / ksw head groups x ksw)
  int head_groups;    // workgroups per query along heads (each covers 128 / ksw heads)
  int n_split;        // workgroups per query along keys
  int bf16_dma;       // 1: bf16 rows staged by DMA (attend_bf16.hip); 0: fp16 staging
  float* ws_o;        // [nq][n_split][H][512] partial outputs (unnormalised), n_split > 1
  float* ws_ml;       // [nq][n_split][H][2] partial (max in log2 units, sum)
  int* flags;         // [nq][head_groups][n_split] 1 = some head left the range of P
};

hipError_t launch_attend_bf16(const AttendArgs& a, const AttnPlan& p, hipStream_t s);

}  // namespace csa
