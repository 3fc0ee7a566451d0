// Split-KV decode instances for head dim 256.
#include "fa_decode_kernel.h"

namespace fa {
hipError_t launch_decode_d256(const DecodeArgs& a, bool bf16, bool causal, hipStream_t stream) {
  return launch_decode_d<256>(a, bf16, causal, stream);
}
}  // namespace fa
