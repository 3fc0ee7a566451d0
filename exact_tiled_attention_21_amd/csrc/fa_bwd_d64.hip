// Backward-pass instances for head dim 64.
#include "fa_bwd_kernel.h"

namespace fa {
hipError_t launch_bwd_d64(const BwdArgs& a, bool bf16, bool causal, hipStream_t stream) {
  return launch_bwd_d<64>(a, bf16, causal, stream);
}
}  // namespace fa
