// Backward-pass instances for head dim 96.
#include "fa_bwd_kernel.h"

namespace fa {
hipError_t launch_bwd_d96(const BwdArgs& a, bool bf16, bool causal, hipStream_t stream) {
  return launch_bwd_d<96>(a, bf16, causal, stream);
}
}  // namespace fa
