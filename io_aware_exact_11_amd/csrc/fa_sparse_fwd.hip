// Block-sparse forward: the forward kernels with the key-tile list of the
// block mask, in the one-slab configurations whose 128 query rows per
// workgroup match the 128 x 128 blocks.
#include "fa_fwd.h"

namespace fa {

hipError_t launch_fwd_sparse_bf16(const void* Q, const void* K, const void* V, void* O, float* LSE,
                                  const AttnShape& s, const uint8_t* bmask, long long bmask_stride,
                                  hipStream_t stream) {
  if (s.d == 128)
    return launch_fwd_d<128, FwdCfg128, false, true>(Q, K, V, O, LSE, s, stream, DropParams{}, bmask, bmask_stride);
  return launch_fwd_d<64, FwdCfg64Causal, false, true>(Q, K, V, O, LSE, s, stream, DropParams{}, bmask,
                                                      bmask_stride);
}

}  // namespace fa
