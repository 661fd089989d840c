// Backward orchestration. Default: the query-outer dQ kernel (which also
// forms the per-row term D_i = dO_i . O_i), then the key-outer dK/dV kernel.
// Precise mode: an exact-D pre-pass, then both kernels. Atomic-dQ mode: the
// rowsum(dO o O) pre-pass, then the key-outer kernel alone, accumulating dQ
// with atomics.
#include "fa_bwd.h"

#include <mutex>

namespace fa {

// Fixed scratch of the allocation-free backward: D_i for up to kNoAllocRows
// rows. Each GPU holds its own copy at its own address; host code never
// passes the array's name to a kernel (in host code it is only a stand-in),
// only the device address that hipGetSymbolAddress reports for the current
// device.
static __device__ __align__(256) float scratch[kNoAllocRows];

hipError_t noalloc_scratch(float** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = static_cast<float*>(addr[dev]);
  return hipSuccess;
}

__global__ void fill_zero_kernel(float4* __restrict__ p, size_t n4) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

static hipError_t fill_zero(float* p, size_t n, hipStream_t stream) {
  const size_t n4 = n / 4;  // n is a multiple of 4 (d in {64, 128})
  size_t blocks = (n4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<float4*>(p), n4);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_row_term(const BwdArgs& a, const AttnShape& s, bool precise, hipStream_t stream) {
  const size_t rows = (size_t)s.B * s.H * s.N;
  const u16* q = static_cast<const u16*>(a.Q);
  const u16* k = static_cast<const u16*>(a.K);
  const u16* v = static_cast<const u16*>(a.V);
  const u16* o = static_cast<const u16*>(a.O);
  const u16* g = static_cast<const u16*>(a.dO);
  if (precise) {
    const int nqb = (s.N + ExactDCfg<D>::BR - 1) / ExactDCfg<D>::BR;
    const int total = s.B * s.H * nqb;
    hipLaunchKernelGGL(bwd_exact_d_kernel<D>, dim3(total), dim3(256), 0, stream, q, k, v, g, a.LSE,
                       a.Dws, s.H, s.N, s.scale * kLog2e, s.causal, s.kv_len, nqb, total, DropParams{});
  } else {
    hipLaunchKernelGGL(bwd_dot_kernel<D>, dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0,
                       stream, o, g, a.Dws, (int)rows);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_bf16(const void* Q, const void* K, const void* V, const void* O,
                           const void* dO, const float* LSE, float* dQ, float* dK, float* dV,
                           float* Dws, const AttnShape& s, bool precise, bool dq_atomic,
                           hipStream_t stream) {
  const BwdArgs a{Q, K, V, O, dO, LSE, dQ, dK, dV, Dws};
  const bool d64 = s.d == 64;
  hipError_t e;
  if (dq_atomic) {
    e = fill_zero(dQ, (size_t)s.B * s.H * s.N * s.d, stream);
    if (e != hipSuccess) return e;
  }
  if (!precise && !dq_atomic) {
    // The dQ kernel forms D_i = dO_i . O_i itself and stores it for the
    // dK/dV kernel, which therefore runs second.
    e = d64 ? launch_dq_bf16_d64(a, s, false, stream) : launch_dq_bf16_d128(a, s, false, stream);
    if (e != hipSuccess) return e;
    return d64 ? launch_dkdv_bf16_d64(a, s, false, stream) : launch_dkdv_bf16_d128(a, s, false, stream);
  }
  e = d64 ? launch_row_term<64>(a, s, precise, stream) : launch_row_term<128>(a, s, precise, stream);
  if (e != hipSuccess) return e;
  if (dq_atomic)
    return d64 ? launch_dkdv_atomic_bf16_d64(a, s, precise, stream)
               : launch_dkdv_atomic_bf16_d128(a, s, precise, stream);
  e = d64 ? launch_dkdv_bf16_d64(a, s, precise, stream) : launch_dkdv_bf16_d128(a, s, precise, stream);
  if (e != hipSuccess) return e;
  return d64 ? launch_dq_bf16_d64(a, s, precise, stream) : launch_dq_bf16_d128(a, s, precise, stream);
}

}  // namespace fa
