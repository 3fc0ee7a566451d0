// Forward-kernel instances for head dim 256 (f16/bf16 x causal/non-causal).
#include "fa_fwd_kernel.h"

namespace fa {
hipError_t launch_fwd_d256(const FwdArgs& a, bool bf16, bool band, hipStream_t stream) {
  return launch_fwd_d<256>(a, bf16, band, stream);
}
}  // namespace fa
