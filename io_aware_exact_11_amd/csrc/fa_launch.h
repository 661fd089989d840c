// Host-side launchers of the gfx950 kernels (internal to libflashattn.so).
// Every launcher assumes its arguments were validated by the C entry points
// and only enqueues work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

struct AttnShape {
  int B, H, N, d;
  float scale;
  int causal;
  const int32_t* kv_len;  // device [B] or nullptr
};

hipError_t launch_fwd_bf16(const void* Q, const void* K, const void* V, void* O, float* LSE,
                           const AttnShape& s, hipStream_t stream);

// Dws: fp32 [B,H,N] scratch for the per-row term D_i.
hipError_t launch_bwd_bf16(const void* Q, const void* K, const void* V, const void* O,
                           const void* dO, const float* LSE, float* dQ, float* dK, float* dV,
                           float* Dws, const AttnShape& s, bool precise, bool dq_atomic,
                           hipStream_t stream);

hipError_t launch_fwd_f32(const float* Q, const float* K, const float* V, float* O, float* LSE,
                          const AttnShape& s, hipStream_t stream);

hipError_t launch_bwd_f32(const float* Q, const float* K, const float* V, const float* O,
                          const float* dO, const float* LSE, float* dQ, float* dK, float* dV,
                          float* Dws, const AttnShape& s, hipStream_t stream);

}  // namespace fa
