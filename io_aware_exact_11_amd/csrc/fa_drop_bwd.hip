// Backward with fused dropout, every kernel regenerating the keep mask.
// Default: the query-outer dQ kernel (which also forms D_i = dO_i . O_i from
// the dropped output), then the key-outer dK/dV kernel. Precise: the exact
// D_i = sum_j P_ij dP_ij pass, then both kernels with split P and dS.
// Also the keep-mask writer.
#include "fa_bwd.h"

namespace fa {

template <int D>
static hipError_t bwd_drop_d(const BwdArgs& a, const AttnShape& s, const DropParams& dp, bool precise,
                             hipStream_t stream) {
  const float sl2 = s.scale * kLog2e;
  const u16* q = static_cast<const u16*>(a.Q);
  const u16* k = static_cast<const u16*>(a.K);
  const u16* v = static_cast<const u16*>(a.V);
  const u16* o = static_cast<const u16*>(a.O);
  const u16* g = static_cast<const u16*>(a.dO);
  if (precise) {
    const int nqb = (s.N + ExactDCfg<D>::BR - 1) / ExactDCfg<D>::BR;
    const int total = s.B * s.H * nqb;
    hipLaunchKernelGGL((bwd_exact_d_kernel<D, true>), dim3(total), dim3(256), 0, stream, q, k, v, g, a.LSE, a.Dws,
                       s.H, s.N, sl2, s.causal, s.kv_len, nqb, total, dp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_dkdv<D, true, false, true>(q, k, v, g, a.LSE, a.Dws, a.dQ, a.dK, a.dV, s, sl2, stream, dp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_dq<D, true, true>(q, k, v, o, g, a.LSE, a.Dws, a.dQ, s, sl2, stream, dp);
    return hipGetLastError();
  }
  launch_dq<D, false, true>(q, k, v, o, g, a.LSE, a.Dws, a.dQ, s, sl2, stream, dp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_dkdv<D, false, false, true>(q, k, v, g, a.LSE, a.Dws, a.dQ, a.dK, a.dV, s, sl2, stream, dp);
  return hipGetLastError();
}

hipError_t launch_bwd_drop_bf16(const void* Q, const void* K, const void* V, const void* O,
                                const void* dO, const float* LSE, float* dQ, float* dK, float* dV,
                                float* Dws, const AttnShape& s, const DropParams& dp, bool precise,
                                hipStream_t stream) {
  const BwdArgs a{Q, K, V, O, dO, LSE, dQ, dK, dV, Dws};
  return s.d == 64 ? bwd_drop_d<64>(a, s, dp, precise, stream) : bwd_drop_d<128>(a, s, dp, precise, stream);
}

// One generator call per 4 x 4 (query, key) block: element (i, j) is kept
// iff byte j % 4 of word i % 4 >= thresh. Grid-stride over the blocks.
__global__ void dropout_mask_kernel(uint8_t* __restrict__ mask, int BH, int Nq, int Nk, DropParams dp) {
  const int nbi = (Nq + 3) / 4, nbj = (Nk + 3) / 4;
  const size_t total = (size_t)BH * nbi * nbj;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int j4 = (int)(idx % nbj);
    const int i4 = (int)((idx / nbj) % nbi);
    const int bh = (int)(idx / ((size_t)nbj * nbi));
    const u32x4 x = philox4x32_10((unsigned)j4, (unsigned)i4, (unsigned)bh, dp.offset, dp.k0, dp.k1);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int i = 4 * i4 + m;
      if (i >= Nq) break;
      uint8_t* row = mask + ((size_t)bh * Nq + i) * Nk;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int j = 4 * j4 + k;
        if (j < Nk) row[j] = ((x[m] >> (8 * k)) & 0xFFu) >= dp.thresh ? 1 : 0;
      }
    }
  }
}

hipError_t launch_dropout_mask(uint8_t* mask, int B, int H, int Nq, int Nk, const DropParams& dp,
                               hipStream_t stream) {
  const size_t blocks4 = (size_t)B * H * ((Nq + 3) / 4) * ((Nk + 3) / 4);
  size_t grid = (blocks4 + 255) / 256;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(dropout_mask_kernel, dim3((unsigned)grid), dim3(256), 0, stream, mask, B * H, Nq, Nk, dp);
  return hipGetLastError();
}

}  // namespace fa
