// Backward-pass instances for head dim 128.
#include "fa_bwd_kernel.h"

namespace fa {
hipError_t launch_bwd_d128(const BwdArgs& a, bool bf16, bool causal, hipStream_t stream) {
  return launch_bwd_d<128>(a, bf16, causal, stream);
}
}  // namespace fa
