// bf16 forward: the instances for 192-wide q/k heads (d_v 128 or 64).  The
// kernel is in splash_fwd_bf16_kernel.h.

#include "splash_fwd_bf16_kernel.h"

namespace splash {

hipError_t launch_fwd_bf16_d192(const FwdParams& p, int d_v, int n_cu, hipStream_t s) {
  if (d_v == 128) return launch_default<192, 128>(p, n_cu, s);
  if (d_v == 64) return launch_default<192, 64>(p, n_cu, s);
  return hipErrorInvalidValue;
}

}  // namespace splash
