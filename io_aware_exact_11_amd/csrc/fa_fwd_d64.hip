// Forward kernel instantiated for head size 64.
#include "fa_fwd.h"

namespace fa {

hipError_t launch_fwd_bf16_d64(const void* Q, const void* K, const void* V, void* O, float* LSE,
                               const AttnShape& s, hipStream_t stream) {
  if (s.causal) return launch_fwd_d<64, FwdCfg64Causal>(Q, K, V, O, LSE, s, stream);
  return launch_fwd_d<64, FwdCfg64Full>(Q, K, V, O, LSE, s, stream);
}

}  // namespace fa
