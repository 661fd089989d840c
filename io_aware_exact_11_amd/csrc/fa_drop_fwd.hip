// Forward with fused dropout, both head sizes, in the forward's configurations.
#include "fa_fwd.h"

namespace fa {

hipError_t launch_fwd_drop_bf16(const void* Q, const void* K, const void* V, void* O, float* LSE,
                                const AttnShape& s, const DropParams& dp, hipStream_t stream) {
  if (s.d == 128) return launch_fwd_d<128, FwdCfg128, true>(Q, K, V, O, LSE, s, stream, dp);
  if (s.causal) return launch_fwd_d<64, FwdCfg64Causal, true>(Q, K, V, O, LSE, s, stream, dp);
  return launch_fwd_d<64, FwdCfg64Full, true>(Q, K, V, O, LSE, s, stream, dp);
}

}  // namespace fa
