// bf16 forward: the instances for the 64-wide head dims (64/64, 64/128,
// 128/64).  The kernel is in splash_fwd_bf16_kernel.h.

#include "splash_fwd_bf16_kernel.h"

namespace splash {

hipError_t launch_fwd_bf16_d64(const FwdParams& p, int d_qk, int d_v, int n_cu, hipStream_t s) {
  if (d_qk == 64 && d_v == 64) return launch_default<64, 64>(p, n_cu, s);
  if (d_qk == 128 && d_v == 64) return launch_default<128, 64>(p, n_cu, s);
  if (d_qk == 64 && d_v == 128) return launch_default<64, 128>(p, n_cu, s);
  return hipErrorInvalidValue;
}

}  // namespace splash
