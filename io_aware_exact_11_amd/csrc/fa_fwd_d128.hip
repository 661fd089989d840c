// Forward kernel instantiated for head size 128.
#include "fa_fwd.h"

namespace fa {

hipError_t launch_fwd_bf16_d128(const void* Q, const void* K, const void* V, void* O, float* LSE,
                               const AttnShape& s, hipStream_t stream) {
  return launch_fwd_d<128, FwdCfg128>(Q, K, V, O, LSE, s, stream);
}

}  // namespace fa
