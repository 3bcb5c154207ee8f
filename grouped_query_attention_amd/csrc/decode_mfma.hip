// decode_mfma.hip -- split-KV cached decode (placeholder until the kernel lands).
#include <hip/hip_runtime.h>

#include "launch.h"

namespace gqa {

DecodePlan plan_decode(int, int, int total_len, int, int, int, int) {
  return DecodePlan{1, total_len, 0, false};
}

hipError_t launch_attn_decode_mfma(const DecodeArgs&, const DecodePlan&, hipStream_t) {
  return hipErrorInvalidValue;
}

}  // namespace gqa
