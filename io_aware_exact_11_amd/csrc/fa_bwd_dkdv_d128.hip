// Key-outer backward kernel (dK, dV; dQ too in the atomic variant)
// instantiated for head size 128.
#include "fa_bwd.h"

namespace fa {

hipError_t launch_dkdv_bf16_d128(const BwdArgs& a, const AttnShape& s, bool precise, bool dq_atomic,
                               hipStream_t stream) {
  return launch_dkdv_any<128>(a, s, precise, dq_atomic, stream);
}

}  // namespace fa
