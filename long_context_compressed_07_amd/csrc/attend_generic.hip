// Reference attention kernel for csa_attend / hca_attend: one workgroup per (query, head). It
// serves the fp32 workloads, shapes without a specialised MFMA path, and as the GPU-side
// cross-check of the MFMA kernel.
#include "attend_generic.h"

namespace csa {
namespace {

__global__ void __launch_bounds__(kGenThreads) attend_generic_kernel(AttendArgs a) {
  extern __shared__ float smem[];
  const int qi = blockIdx.x / a.H;
  const int h = blockIdx.x - qi * a.H;
  attend_generic_one(a, qi, h, smem);
}

}  // namespace

hipError_t launch_attend_generic(const AttendArgs& a, hipStream_t s) {
  const int d = a.ent.d_c + a.ent.d_r;
  attend_generic_kernel<<<(unsigned)((int64_t)a.Q.nq * a.H), kGenThreads, generic_smem_bytes(d), s>>>(a);
  return hipGetLastError();
}

}  // namespace csa
