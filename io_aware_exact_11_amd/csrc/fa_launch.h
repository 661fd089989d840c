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

// Device pointers of one backward call. Q, K, V, O, dO are bf16 (or fp32
// for the fp32 path); Dws is the fp32 [B,H,N] scratch for D_i.
struct BwdArgs {
  const void *Q, *K, *V, *O, *dO;
  const float* LSE;
  float *dQ, *dK, *dV, *Dws;
};

hipError_t launch_fwd_bf16(const void* Q, const void* K, const void* V, void* O, float* LSE,
                           const AttnShape& s, hipStream_t stream);

// Per-head-size pieces, each in a translation unit of its own so that each
// can be compiled with the instruction-scheduling options that suit it.
hipError_t launch_fwd_bf16_d64(const void* Q, const void* K, const void* V, void* O, float* LSE,
                               const AttnShape& s, hipStream_t stream);
hipError_t launch_fwd_bf16_d128(const void* Q, const void* K, const void* V, void* O, float* LSE,
                                const AttnShape& s, hipStream_t stream);
hipError_t launch_dkdv_bf16_d64(const BwdArgs& a, const AttnShape& s, bool precise, hipStream_t stream);
hipError_t launch_dkdv_bf16_d128(const BwdArgs& a, const AttnShape& s, bool precise, hipStream_t stream);
hipError_t launch_dkdv_atomic_bf16_d64(const BwdArgs& a, const AttnShape& s, bool precise, hipStream_t stream);
hipError_t launch_dkdv_atomic_bf16_d128(const BwdArgs& a, const AttnShape& s, bool precise, hipStream_t stream);
hipError_t launch_dq_bf16_d64(const BwdArgs& a, const AttnShape& s, bool precise, hipStream_t stream);
hipError_t launch_dq_bf16_d128(const BwdArgs& a, const AttnShape& s, bool precise, hipStream_t stream);

// Fused dropout: Philox4x32-10 key words, the fourth counter word, the byte
// threshold t = round(256 p) (kept iff byte >= t) and the keep factor
// 256 / (256 - t).
struct DropParams {
  unsigned k0, k1;
  unsigned offset;
  unsigned thresh;
  float keep_scale;
};

hipError_t launch_fwd_drop_bf16(const void* Q, const void* K, const void* V, void* O, float* LSE,
                                const AttnShape& s, const DropParams& dp, hipStream_t stream);
hipError_t launch_bwd_drop_bf16(const void* Q, const void* K, const void* V, const void* O,
                                const void* dO, const float* LSE, float* dQ, float* dK, float* dV,
                                float* Dws, const AttnShape& s, const DropParams& dp, bool precise,
                                hipStream_t stream);
// The keep mask itself, [B, H, Nq, Nk] bytes (1 = kept).
hipError_t launch_dropout_mask(uint8_t* mask, int B, int H, int Nq, int Nk, const DropParams& dp,
                               hipStream_t stream);

// Block-sparse forward: bmask bytes [nb][nb] per (b, h), nb = ceil(N / 128),
// bmask_stride bytes between consecutive (b, h) (0: one mask for all heads).
hipError_t launch_fwd_sparse_bf16(const void* Q, const void* K, const void* V, void* O, float* LSE,
                                  const AttnShape& s, const uint8_t* bmask, long long bmask_stride,
                                  hipStream_t stream);

// 8-bit forward: Q8, K8 E4M3 [B,H,N,d], Vt8 E4M3 [B,H,d,N], fp32 dequantisation
// factors; O bf16, LSE fp32.
hipError_t launch_fwd_fp8(const void* Q8, const void* K8, const void* Vt8, void* O, float* LSE, const AttnShape& s,
                          float dq, float dk, float dv, hipStream_t stream);

// Dws: fp32 [B,H,N] scratch for the per-row term D_i.
hipError_t launch_bwd_bf16(const void* Q, const void* K, const void* V, const void* O,
                           const void* dO, const float* LSE, float* dQ, float* dK, float* dV,
                           float* Dws, const AttnShape& s, bool precise, bool dq_atomic,
                           hipStream_t stream);

// Allocation-free backward: the per-row term D_i of at most kNoAllocRows
// rows lives in a fixed device array (16 MiB per GPU for the life of the
// process). noalloc_scratch returns its address on the current device,
// looked up once per device.
constexpr size_t kNoAllocRows = size_t(4) << 20;
hipError_t noalloc_scratch(float** ptr);

// Decoding: Nq new queries per (b, h) against Nk cache slots.
struct DecodeShape {
  int B, H, Nq, Nk, d;
  float scale;
  int causal;
  const int32_t* kv_len;  // device [B] or nullptr
};

// Key chunks per (b, h); the workspace holds, per chunk and query, d fp32
// output values and one log-sum-exp.
int decode_chunks(int nk);

hipError_t launch_decode_bf16(const void* Q, const void* K, const void* V, void* O, float* LSE, float* ws,
                              const DecodeShape& s, hipStream_t stream);

hipError_t launch_fwd_f32(const float* Q, const float* K, const float* V, float* O, float* LSE,
                          const AttnShape& s, hipStream_t stream);

hipError_t launch_bwd_f32(const float* Q, const float* K, const float* V, const float* O,
                          const float* dO, const float* LSE, float* dQ, float* dK, float* dV,
                          float* Dws, const AttnShape& s, hipStream_t stream);

}  // namespace fa
