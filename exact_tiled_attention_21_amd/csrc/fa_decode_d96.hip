// Split-KV decode instances for head dim 96.
#include "fa_decode_kernel.h"

namespace fa {
hipError_t launch_decode_d96(const DecodeArgs& a, bool bf16, bool causal, hipStream_t stream) {
  return launch_decode_d<96>(a, bf16, causal, stream);
}
}  // namespace fa
