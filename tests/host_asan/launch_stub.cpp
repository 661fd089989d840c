// Host-only stand-ins for the kernel launchers of libflashattn.so. They let
// the C entry points (csrc/flash_attn_api.cpp) be built with the address and
// undefined-behaviour sanitizers and exercised on a machine without a GPU:
// each stub counts that it was reached and launches nothing.
#include "fa_launch.h"

namespace fa {

int g_launches = 0;

static hipError_t reached() {
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_fwd_bf16(const void*, const void*, const void*, void*, float*, const AttnShape&, hipStream_t) {
  return reached();
}
hipError_t launch_bwd_bf16(const void*, const void*, const void*, const void*, const void*, const float*, float*,
                           float*, float*, float*, const AttnShape&, bool, bool, hipStream_t) {
  return reached();
}
hipError_t launch_fwd_f32(const float*, const float*, const float*, float*, float*, const AttnShape&, hipStream_t) {
  return reached();
}
hipError_t launch_bwd_f32(const float*, const float*, const float*, const float*, const float*, const float*, float*,
                          float*, float*, float*, const AttnShape&, hipStream_t) {
  return reached();
}
hipError_t launch_fwd_drop_bf16(const void*, const void*, const void*, void*, float*, const AttnShape&,
                                const DropParams&, hipStream_t) {
  return reached();
}
hipError_t launch_bwd_drop_bf16(const void*, const void*, const void*, const void*, const void*, const float*, float*,
                                float*, float*, float*, const AttnShape&, const DropParams&, bool, hipStream_t) {
  return reached();
}
hipError_t launch_dropout_mask(uint8_t*, int, int, int, int, const DropParams&, hipStream_t) { return reached(); }
hipError_t launch_fwd_sparse_bf16(const void*, const void*, const void*, void*, float*, const AttnShape&,
                                  const uint8_t*, long long, hipStream_t) {
  return reached();
}
hipError_t launch_fwd_fp8(const void*, const void*, const void*, void*, float*, const AttnShape&, float, float, float,
                          hipStream_t) {
  return reached();
}
hipError_t launch_decode_bf16(const void*, const void*, const void*, void*, float*, float*, const DecodeShape&,
                              hipStream_t) {
  return reached();
}
// The library's decoding kernels take 512 keys per chunk.
int decode_chunks(int nk) { return (nk + 511) / 512; }

hipError_t noalloc_scratch(float** ptr) {
  static float stand_in[64];
  *ptr = stand_in;
  return hipSuccess;
}

}  // namespace fa
