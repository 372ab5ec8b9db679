// Dispatch of csa_attend / hca_attend to the attention kernels.
#include "csa_internal.h"

namespace csa {

hipError_t launch_attend_generic(const AttendArgs& a, hipStream_t s);

size_t attend_workspace(int /*nq*/, int /*H*/, int /*d_c*/, int64_t /*max_keys*/) { return 0; }

hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
  if (a.Q.nq == 0 || a.H == 0) return hipSuccess;
  return launch_attend_generic(a, s);
}

}  // namespace csa
