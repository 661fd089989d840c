// Forward dispatch by head size.
#include "fa_launch.h"

namespace fa {

hipError_t launch_fwd_bf16(const void* Q, const void* K, const void* V, void* O, float* LSE,
                           const AttnShape& s, hipStream_t stream) {
  if (s.d == 64) return launch_fwd_bf16_d64(Q, K, V, O, LSE, s, stream);
  return launch_fwd_bf16_d128(Q, K, V, O, LSE, s, stream);
}

}  // namespace fa
