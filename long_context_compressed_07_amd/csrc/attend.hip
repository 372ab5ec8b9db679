// Dispatch of csa_attend / hca_attend to the attention kernels: the MFMA kernel for bf16 queries
// against bf16 or fp8 cache rows of 512 + 64 dims (heads in groups of 32), the fp32 reference
// kernel otherwise. CSA_ATTEND_KERNEL=generic forces the reference kernel (cross-checks).
#include <cstdlib>
#include <cstring>

#include "csa_internal.h"

namespace csa {

hipError_t launch_attend_generic(const AttendArgs& a, hipStream_t s);
bool attend_mfma_supported(const AttendArgs& a);
size_t attend_mfma_workspace(int nq, int H, int64_t max_keys, bool dense);
hipError_t launch_attend_mfma(const AttendArgs& a, int64_t max_keys, hipStream_t s);

size_t attend_workspace(int nq, int H, int d_c, int64_t max_keys, bool dense) {
  if (d_c != 512 || H % 32 != 0) return 0;
  return attend_mfma_workspace(nq, H, max_keys, dense);
}

static bool force_generic() {
  const char* e = std::getenv("CSA_ATTEND_KERNEL");
  return e != nullptr && std::strcmp(e, "generic") == 0;
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
  if (a.Q.nq == 0 || a.H == 0) return hipSuccess;
  const int64_t max_keys =
      a.dense ? a.ent.rows : (int64_t)a.k * (a.tok_m > 0 ? a.tok_m : 1) + a.window;
  if (!force_generic() && attend_mfma_supported(a)) return launch_attend_mfma(a, max_keys, s);
  const int slot = a.dense ? 1 : 0;
  const int timed = timing_start(slot, s);
  const hipError_t e = launch_attend_generic(a, s);
  if (timed >= 0) timing_stop(slot, timed, s);
  return e;
}

}  // namespace csa
