// Key-outer backward kernel (dK, dV) instantiated for head size 64.
#include "fa_bwd.h"

namespace fa {

hipError_t launch_dkdv_bf16_d64(const BwdArgs& a, const AttnShape& s, bool precise, hipStream_t stream) {
  return launch_dkdv_default<64>(a, s, precise, stream);
}

}  // namespace fa
