// Key-outer backward kernel (dK, dV; dQ too in the atomic variant)
// instantiated for head size 64.
#include "fa_bwd.h"

namespace fa {

hipError_t launch_dkdv_bf16_d64(const BwdArgs& a, const AttnShape& s, bool precise, bool dq_atomic,
                               hipStream_t stream) {
  return launch_dkdv_any<64>(a, s, precise, dq_atomic, stream);
}

}  // namespace fa
