// Reference attention kernel for csa_attend / hca_attend: one workgroup per (query, head), key rows
// staged through LDS chunk by chunk. It serves the fp32 workloads, shapes without a specialised
// MFMA path, and as the GPU-side cross-check of the MFMA kernel.
#include "attend_generic.h"

namespace csa {
namespace {

// Dynamic LDS per workgroup: the staged key chunk and the per-key arrays (64 KB, the default
// limit of dynamic shared memory; 117 keys of 128 dims, 27 of 576).
constexpr size_t kGenLdsBudget = 64 * 1024;

__global__ void __launch_bounds__(kGenThreads) attend_generic_kernel(AttendArgs a, int chunk) {
  extern __shared__ float smem[];
  const int qi = blockIdx.x / a.H;
  const int h = blockIdx.x - qi * a.H;
  attend_generic_staged(a, qi, h, smem, chunk);
}

}  // namespace

hipError_t launch_attend_generic(const AttendArgs& a, hipStream_t s) {
  const int d = a.ent.d_c + a.ent.d_r;
  const int chunk = staged_chunk(d, kGenLdsBudget);
  attend_generic_kernel<<<(unsigned)((int64_t)a.Q.nq * a.H), kGenThreads,
                          staged_smem_bytes(d, chunk), s>>>(a, chunk);
  return hipGetLastError();
}

}  // namespace csa
