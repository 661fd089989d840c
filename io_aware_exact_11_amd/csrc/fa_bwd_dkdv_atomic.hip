// Key-outer backward kernel with the atomic dQ phase (FA_BWD_DQ_ATOMIC),
// both head sizes; kept out of the per-head-size units so that it builds
// with the compiler's default scheduler.
#include "fa_bwd.h"

namespace fa {

hipError_t launch_dkdv_atomic_bf16_d64(const BwdArgs& a, const AttnShape& s, bool precise, hipStream_t stream) {
  return launch_dkdv_atomic<64>(a, s, precise, stream);
}

hipError_t launch_dkdv_atomic_bf16_d128(const BwdArgs& a, const AttnShape& s, bool precise, hipStream_t stream) {
  return launch_dkdv_atomic<128>(a, s, precise, stream);
}

}  // namespace fa
