// Decoding forward: n_q (1..8) new queries per (b, h) against a cache of
// n_k key/value slots, the first kv_len[b] of which hold keys. One new
// query against a long cache reads every cached key and value once and does
// little arithmetic per byte, so the pass is bound by memory bandwidth
// (decoding is the bandwidth-bound regime: "FlashAttention — why it
// mattered", closing note), and it runs on the vector ALUs rather than the
// matrix cores.
//
// The keys are split into chunks of 512 processed by separate workgroups
// (so that a short batch still fills the GPU); each chunk keeps a running
// maximum, sum and unnormalised output per query ("FlashAttention and GPU
// Memory", chapter 08), and a second kernel merges the chunks with the same
// rule: LSE = log sum_c e^(LSE_c), O = sum_c e^(LSE_c - LSE) O_c.
//
// Inside a chunk each wave streams 128 keys. A key row of d bf16 values is
// spread over d/8 lanes (16 bytes each), so one 16-byte load per lane
// fetches 64/(d/8) whole rows; the score of a query with a row is a
// dot2 product per lane and a sum over those lanes by data-parallel
// primitive moves within the row. Each group of d/8 lanes keeps its own
// running tally; the groups, then the waves, are merged at the end.
#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

constexpr int kDecChunk = 512;  // keys per workgroup

template <int D, int NQ>
struct DecCfg {
  static constexpr int NW = 4;
  static constexpr int LPK = D / 8;             // lanes per key row
  static constexpr int KPI = 64 / LPK;          // rows per wave load
  static constexpr int KPW = kDecChunk / NW;    // keys per wave
  // Loads per tensor in flight: fewer for more queries, whose per-query
  // state would otherwise push the kernel below two waves per SIMD.
  static constexpr int UNROLL = NQ >= 8 ? 1 : (NQ >= 4 ? 2 : 4);
  static constexpr int ITER = KPW / (KPI * UNROLL);
  static_assert(ITER * KPI * UNROLL == KPW, "chunk split");
};

// Sum over the lanes of one key row: 8 lanes (d=64) or 16 (d=128), all of
// which receive the sum. Butterfly over quads, half rows and rows.
template <int LPK>
__device__ __forceinline__ float row_sum(float x) {
  auto mv = [](float v, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value, 0xF, 0xF, false));
  };
  x += mv(x, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
  x += mv(x, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
  x += mv(x, std::integral_constant<int, 0x141>{});  // row_half_mirror
  if constexpr (LPK == 16) x += mv(x, std::integral_constant<int, 0x140>{});  // row_mirror
  return x;
}

// One chunk of keys for every query of one (b, h): writes the chunk's
// normalised output and its log-sum-exp (natural log) to the workspace.
template <int D, int NQ>
__global__ __launch_bounds__(256) void decode_chunk_kernel(
    const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ V,
    float* __restrict__ Opart, float* __restrict__ Lpart, int H, int nq, int nk, int nchunk,
    float sl2, int causal, const int32_t* __restrict__ kv_len) {
  using C = DecCfg<D, NQ>;
  constexpr int LPK = C::LPK, KPI = C::KPI;
  __shared__ float red_o[C::NW][NQ][D];
  __shared__ float red_ml[C::NW][NQ][2];

  const int chunk = blockIdx.x % nchunk;
  const int bh = blockIdx.x / nchunk;
  const int b = bh / H;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int grp = lane / LPK, sub = lane % LPK;

  int L = nk;
  if (kv_len) {
    const int x = kv_len[b];
    L = x < 0 ? 0 : (x > nk ? nk : x);
  }
  const unsigned kv_bytes = (unsigned)nk * D * 2;
  const auto rK = make_rsrc(K + (size_t)bh * nk * D, kv_bytes);
  const auto rV = make_rsrc(V + (size_t)bh * nk * D, kv_bytes);
  const auto rQ = make_rsrc(Q + (size_t)bh * nq * D, (unsigned)nq * D * 2);

  // This lane's 8 elements of every query (rows past nq read zeros).
  u32x4 qv[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) qv[q] = ld_buf16(rQ, (unsigned)(q * D + 8 * sub) * 2);
  // Last key each query may see: L - 1, or L - nq + q with causal masking;
  // queries past nq see none.
  int last[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) last[q] = q < nq ? (causal ? L - nq + q : L - 1) : -1;

  float m[NQ], l[NQ], o[NQ][8];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    m[q] = -INFINITY;
    l[q] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[q][e] = 0.f;
  }

  const int key0 = chunk * kDecChunk + w * C::KPW;
  const int kend = min(L, key0 + C::KPW);  // no query sees keys at or past L
  for (int it = 0; it < C::ITER && key0 + it * KPI * C::UNROLL < kend; ++it) {
    u32x4 kr[C::UNROLL], vr[C::UNROLL];
    const int base = key0 + it * KPI * C::UNROLL;
#pragma unroll
    for (int u = 0; u < C::UNROLL; ++u) {
      const unsigned off = (unsigned)((base + u * KPI + grp) * D + 8 * sub) * 2;
      kr[u] = ld_buf16(rK, off);
      vr[u] = ld_buf16(rV, off);
    }
#pragma unroll
    for (int u = 0; u < C::UNROLL; ++u) {
      const int key = base + u * KPI + grp;
      float s[NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        float acc = 0.f;
#pragma unroll
        for (int h = 0; h < 4; ++h)
          acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qv[q][h]), as_bf16x2(kr[u][h]), acc, false);
        acc = row_sum<LPK>(acc);
        s[q] = key <= last[q] ? acc * sl2 : -INFINITY;
      }
      // Lazy running maximum (base-2 units): moved only when a score exceeds
      // it by more than 8, for every lane at once.
      bool grow = false;
#pragma unroll
      for (int q = 0; q < NQ; ++q) grow |= s[q] > m[q] + 8.f;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          if (s[q] > m[q] + 8.f) {
            const float alpha = m[q] == -INFINITY ? 0.f : fast_exp2(m[q] - s[q]);
            l[q] *= alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[q][e] *= alpha;
            m[q] = s[q];
          }
        }
      }
      float vf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) vf[e] = __uint_as_float(bf16_bits(vr[u], e) << 16);
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const float p = fast_exp2(s[q] - (m[q] == -INFINITY ? 0.f : m[q]));
        l[q] += p;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[q][e] = fmaf(p, vf[e], o[q][e]);
      }
    }
  }

  // Merge the key groups of the wave (lanes sub, sub + LPK, ...).
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    float mt = m[q];
#pragma unroll
    for (int x = LPK; x < 64; x <<= 1) mt = fmaxf(mt, __shfl_xor(mt, x));
    const float f = m[q] == -INFINITY ? 0.f : fast_exp2(m[q] - mt);
    float lt = l[q] * f;
#pragma unroll
    for (int x = LPK; x < 64; x <<= 1) lt += __shfl_xor(lt, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = o[q][e] * f;
#pragma unroll
      for (int x = LPK; x < 64; x <<= 1) v += __shfl_xor(v, x);
      o[q][e] = v;
    }
    m[q] = mt;
    l[q] = lt;
  }
  if (grp == 0) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
#pragma unroll
      for (int e = 0; e < 8; ++e) red_o[w][q][8 * sub + e] = o[q][e];
      if (sub == 0) {
        red_ml[w][q][0] = m[q];
        red_ml[w][q][1] = l[q];
      }
    }
  }
  __syncthreads();
  // Merge the waves: thread t takes (query, element) pairs t, t + 256, ...
  const size_t slot = (size_t)bh * nchunk + chunk;
  for (int i = tid; i < NQ * D; i += 256) {
    const int q = i / D, e = i % D;
    float mt = -INFINITY;
#pragma unroll
    for (int v = 0; v < C::NW; ++v) mt = fmaxf(mt, red_ml[v][q][0]);
    float lt = 0.f, ot = 0.f;
#pragma unroll
    for (int v = 0; v < C::NW; ++v) {
      const float mv = red_ml[v][q][0];
      const float f = mv == -INFINITY ? 0.f : fast_exp2(mv - mt);
      lt += red_ml[v][q][1] * f;
      ot += red_o[v][q][e] * f;
    }
    if (q < nq) {
      Opart[(slot * nq + q) * D + e] = lt > 0.f ? ot / lt : 0.f;
      if (e == 0) Lpart[slot * nq + q] = lt > 0.f ? (mt + __log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

// Merge the chunks of one (b, h, query): one wave, d/64 elements per lane.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(const float* __restrict__ Opart,
                                                          const float* __restrict__ Lpart,
                                                          u16* __restrict__ O, float* __restrict__ LSE,
                                                          int nq, int nchunk) {
  constexpr int EPL = D / 64;
  const int row = blockIdx.x;  // (bh, q)
  const int bh = row / nq, q = row % nq;
  const int lane = threadIdx.x;
  float mx = -INFINITY;
  for (int c = 0; c < nchunk; ++c) mx = fmaxf(mx, Lpart[((size_t)bh * nchunk + c) * nq + q]);
  float sum = 0.f, acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  if (mx != -INFINITY) {
    for (int c = 0; c < nchunk; ++c) {
      const size_t slot = (size_t)bh * nchunk + c;
      const float lc = Lpart[slot * nq + q];
      const float f = lc == -INFINITY ? 0.f : __expf(lc - mx);
      sum += f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] += f * Opart[(slot * nq + q) * D + EPL * lane + e];
    }
  }
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  u16* orow = O + (size_t)row * D;
#pragma unroll
  for (int e = 0; e < EPL; ++e) orow[EPL * lane + e] = __builtin_bit_cast(u16, (__bf16)(acc[e] * inv));
  if (lane == 0) LSE[row] = sum > 0.f ? mx + __logf(sum) : -INFINITY;
}

template <int D, int NQ>
static void launch_decode_nq(const void* Q, const void* K, const void* V, void* O, float* LSE, float* ws,
                             const DecodeShape& s, hipStream_t stream) {
  const int nchunk = decode_chunks(s.Nk);
  float* Opart = ws;
  float* Lpart = ws + (size_t)s.B * s.H * nchunk * s.Nq * D;
  hipLaunchKernelGGL((decode_chunk_kernel<D, NQ>), dim3(s.B * s.H * nchunk), dim3(256), 0, stream,
                     static_cast<const u16*>(Q), static_cast<const u16*>(K), static_cast<const u16*>(V), Opart,
                     Lpart, s.H, s.Nq, s.Nk, nchunk, s.scale * kLog2e, s.causal, s.kv_len);
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(s.B * s.H * s.Nq), dim3(64), 0, stream, Opart, Lpart,
                     static_cast<u16*>(O), LSE, s.Nq, nchunk);
}

template <int D>
static void launch_decode_d(const void* Q, const void* K, const void* V, void* O, float* LSE, float* ws,
                            const DecodeShape& s, hipStream_t stream) {
  if (s.Nq <= 1)
    launch_decode_nq<D, 1>(Q, K, V, O, LSE, ws, s, stream);
  else if (s.Nq <= 2)
    launch_decode_nq<D, 2>(Q, K, V, O, LSE, ws, s, stream);
  else if (s.Nq <= 4)
    launch_decode_nq<D, 4>(Q, K, V, O, LSE, ws, s, stream);
  else
    launch_decode_nq<D, 8>(Q, K, V, O, LSE, ws, s, stream);
}

int decode_chunks(int nk) { return (nk + kDecChunk - 1) / kDecChunk; }

hipError_t launch_decode_bf16(const void* Q, const void* K, const void* V, void* O, float* LSE, float* ws,
                              const DecodeShape& s, hipStream_t stream) {
  if (s.d == 64)
    launch_decode_d<64>(Q, K, V, O, LSE, ws, s, stream);
  else
    launch_decode_d<128>(Q, K, V, O, LSE, ws, s, stream);
  return hipGetLastError();
}

}  // namespace fa
