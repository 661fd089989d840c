// fp32 exact attention, forward and backward, on the vector ALUs.
//
// One wave per row; each lane holds d/64 elements of every row vector and
// dot products are wave reductions. The forward walks the visible keys one
// at a time with the running maximum and sum of "FlashAttention and GPU
// Memory", chapter 08 (a block of one key), keeping the output unnormalised
// until the end; the backward rebuilds each P_ij from the saved LSE
// (chapter 09) and applies dV = P^T dO, dS = P o (dP - D), dQ = s dS K,
// dK = s dS^T Q with D_i = dO_i . O_i, in fp32 throughout.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ __forceinline__ int clamp_len(const int32_t* kv_len, int b, int N) {
  if (!kv_len) return N;
  const int L = kv_len[b];
  return L < 0 ? 0 : (L > N ? N : L);
}

template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(const float* __restrict__ Q,
                                                      const float* __restrict__ K,
                                                      const float* __restrict__ V,
                                                      float* __restrict__ O, float* __restrict__ LSE,
                                                      int H, int N, float scale, int causal,
                                                      const int32_t* __restrict__ kv_len, int rows) {
  constexpr int E = D / 64;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;  // uniform per wave
  const int bh = row / N, i = row % N, b = bh / H;
  const size_t head = (size_t)bh * N * D;
  int jend = clamp_len(kv_len, b, N);
  if (causal) jend = min(jend, i + 1);
  float q[E], o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q[e] = Q[head + (size_t)i * D + lane + 64 * e];
    o[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int j = 0; j < jend; ++j) {
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) part += q[e] * K[head + (size_t)j * D + lane + 64 * e];
    const float sc = scale * wave_sum(part);
    const float m_new = fmaxf(m, sc);
    const float alpha = expf(m - m_new);
    const float p = expf(sc - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = o[e] * alpha + p * V[head + (size_t)j * D + lane + 64 * e];
    m = m_new;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) O[head + (size_t)i * D + lane + 64 * e] = o[e] * inv;
  if (lane == 0) LSE[row] = l > 0.f ? m + logf(l) : -INFINITY;
}

template <int D>
__global__ __launch_bounds__(256) void dot_f32_kernel(const float* __restrict__ O,
                                                      const float* __restrict__ dO,
                                                      float* __restrict__ Dout, int rows) {
  constexpr int E = D / 64;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float part = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) part += O[(size_t)row * D + lane + 64 * e] * dO[(size_t)row * D + lane + 64 * e];
  part = wave_sum(part);
  if (lane == 0) Dout[row] = part;
}

// dQ_i = s sum_j P_ij (dP_ij - D_i) k_j, one wave per query row.
template <int D>
__global__ __launch_bounds__(256) void dq_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                     const float* __restrict__ V, const float* __restrict__ dO,
                                                     const float* __restrict__ LSE, const float* __restrict__ Dr,
                                                     float* __restrict__ dQ, int H, int N, float scale,
                                                     int causal, const int32_t* __restrict__ kv_len, int rows) {
  constexpr int E = D / 64;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int bh = row / N, i = row % N, b = bh / H;
  const size_t head = (size_t)bh * N * D;
  int jend = clamp_len(kv_len, b, N);
  if (causal) jend = min(jend, i + 1);
  float q[E], g[E], acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q[e] = Q[head + (size_t)i * D + lane + 64 * e];
    g[e] = dO[head + (size_t)i * D + lane + 64 * e];
    acc[e] = 0.f;
  }
  const float lse = LSE[row], Di = Dr[row];
  for (int j = 0; j < jend; ++j) {
    float ps = 0.f, pd = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      ps += q[e] * K[head + (size_t)j * D + lane + 64 * e];
      pd += g[e] * V[head + (size_t)j * D + lane + 64 * e];
    }
    const float p = expf(scale * wave_sum(ps) - lse);
    const float ds = p * (wave_sum(pd) - Di);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += ds * K[head + (size_t)j * D + lane + 64 * e];
  }
#pragma unroll
  for (int e = 0; e < E; ++e) dQ[head + (size_t)i * D + lane + 64 * e] = scale * acc[e];
}

// dV_j = sum_i P_ij dO_i and dK_j = s sum_i dS_ij q_i, one wave per key row.
template <int D>
__global__ __launch_bounds__(256) void dkdv_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                       const float* __restrict__ V, const float* __restrict__ dO,
                                                       const float* __restrict__ LSE, const float* __restrict__ Dr,
                                                       float* __restrict__ dK, float* __restrict__ dV, int H,
                                                       int N, float scale, int causal,
                                                       const int32_t* __restrict__ kv_len, int rows) {
  constexpr int E = D / 64;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int bh = row / N, j = row % N, b = bh / H;
  const size_t head = (size_t)bh * N * D;
  const int lim = clamp_len(kv_len, b, N);
  float k[E], v[E], ak[E], av[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    k[e] = K[head + (size_t)j * D + lane + 64 * e];
    v[e] = V[head + (size_t)j * D + lane + 64 * e];
    ak[e] = 0.f;
    av[e] = 0.f;
  }
  if (j < lim) {
    for (int i = causal ? j : 0; i < N; ++i) {
      float ps = 0.f, pd = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        ps += Q[head + (size_t)i * D + lane + 64 * e] * k[e];
        pd += dO[head + (size_t)i * D + lane + 64 * e] * v[e];
      }
      const float p = expf(scale * wave_sum(ps) - LSE[(size_t)bh * N + i]);
      const float ds = p * (wave_sum(pd) - Dr[(size_t)bh * N + i]);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        av[e] += p * dO[head + (size_t)i * D + lane + 64 * e];
        ak[e] += ds * Q[head + (size_t)i * D + lane + 64 * e];
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    dK[head + (size_t)j * D + lane + 64 * e] = scale * ak[e];
    dV[head + (size_t)j * D + lane + 64 * e] = av[e];
  }
}

template <int D>
static hipError_t launch_fwd_f32_d(const float* Q, const float* K, const float* V, float* O, float* LSE,
                                   const AttnShape& s, hipStream_t stream) {
  const int rows = s.B * s.H * s.N;
  hipLaunchKernelGGL(fwd_f32_kernel<D>, dim3((rows + 3) / 4), dim3(256), 0, stream, Q, K, V, O, LSE,
                     s.H, s.N, s.scale, s.causal, s.kv_len, rows);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd_f32_d(const float* Q, const float* K, const float* V, const float* O,
                                   const float* dO, const float* LSE, float* dQ, float* dK, float* dV,
                                   float* Dws, const AttnShape& s, hipStream_t stream) {
  const int rows = s.B * s.H * s.N;
  const dim3 grid((rows + 3) / 4);
  hipLaunchKernelGGL(dot_f32_kernel<D>, grid, dim3(256), 0, stream, O, dO, Dws, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dq_f32_kernel<D>, grid, dim3(256), 0, stream, Q, K, V, dO, LSE, Dws, dQ, s.H, s.N,
                     s.scale, s.causal, s.kv_len, rows);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dkdv_f32_kernel<D>, grid, dim3(256), 0, stream, Q, K, V, dO, LSE, Dws, dK, dV, s.H,
                     s.N, s.scale, s.causal, s.kv_len, rows);
  return hipGetLastError();
}

hipError_t launch_fwd_f32(const float* Q, const float* K, const float* V, float* O, float* LSE,
                          const AttnShape& s, hipStream_t stream) {
  if (s.d == 64) return launch_fwd_f32_d<64>(Q, K, V, O, LSE, s, stream);
  return launch_fwd_f32_d<128>(Q, K, V, O, LSE, s, stream);
}

hipError_t launch_bwd_f32(const float* Q, const float* K, const float* V, const float* O,
                          const float* dO, const float* LSE, float* dQ, float* dK, float* dV,
                          float* Dws, const AttnShape& s, hipStream_t stream) {
  if (s.d == 64) return launch_bwd_f32_d<64>(Q, K, V, O, dO, LSE, dQ, dK, dV, Dws, s, stream);
  return launch_bwd_f32_d<128>(Q, K, V, O, dO, LSE, dQ, dK, dV, Dws, s, stream);
}

}  // namespace fa
