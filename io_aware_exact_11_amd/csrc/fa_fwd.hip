// Forward pass of exact attention for gfx950, bf16 in, fp32 accumulation.
//
// One workgroup owns BR = 128 query rows of one (b, h) and streams the keys
// and values through LDS in tiles of BC = 64 rows, double-buffered: the
// global loads of tile j+1 are in flight while tile j is computed
// ("FlashAttention and GPU Memory", chapter 07 Blocks: one block of Q stays
// on chip while blocks of K and V come in; only O and the row statistics
// are written back).
//
// Each of the 4 waves owns 32 query rows. Scores are produced transposed,
// S^T = K Q^T, with the 32x32x16 bf16 matrix-core product: A = a K tile
// from LDS, B = the wave's Q fragment held in registers for the whole loop.
// In that layout each lane holds one query's scores for 32 of the tile's
// keys and its partner lane (lane ^ 32) the other 32, so the running
// maximum needs one cross-lane exchange per tile and the running sum none
// (each lane keeps a partial sum; the halves are added once at the end).
//
// Running softmax ("FlashAttention and GPU Memory", chapter 08): m is kept
// in base-2 units of the scaled score, m' = max(m, max_j s_j * scale*log2e),
// P~ = 2^(s*scale*log2e - m'), l' = 2^(m-m') l + sum P~, and the unnormalised
// output is rescaled by the same 2^(m-m'). O is divided by l once, after
// the last tile, and LSE = (m + log2 l) ln 2 is stored for the backward.
//
// The P~ V product reuses the score registers directly as its B operand
// (O^T = V^T P^T): the 8 k-slots a lane feeds are 8 of its own score
// elements. Its A operand needs V transposed, so V tiles are written to LDS
// as V^T with their key columns permuted by swap23 to match those slots.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

template <int D>
struct FwdCfg {
  static constexpr int NW = 4;                  // waves per workgroup
  static constexpr int BR = 32 * NW;            // query rows per workgroup
  static constexpr int BC = 64;                 // keys per tile
  static constexpr int KSTR = D + 8;            // K tile row stride (elements)
  static constexpr int VSTR = BC + 8;           // V^T tile row stride (elements)
  static constexpr int KCH = BC * D / 8 / 256;  // 16-byte K chunks per thread
  static constexpr int VKR = BC * D / 8 / 256;  // keys per thread in the V^T store
  static constexpr int NKG = BC / VKR;          // key groups in the V^T store
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(NKG * (D / 8) == 256, "V^T store covers the tile once");
};

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(
    const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ V,
    u16* __restrict__ O, float* __restrict__ LSE, int H, int N, float sl2, int causal,
    const int32_t* __restrict__ kv_len, int nqb, int total) {
  using C = FwdCfg<D>;
  constexpr int BC = C::BC;
  __shared__ __attribute__((aligned(16))) u16 Ks[2][BC * C::KSTR];
  __shared__ __attribute__((aligned(16))) u16 Vt[2][D * C::VSTR];

  const int tile = xcd_tile(blockIdx.x, total);
  int qb = tile % nqb;
  const int bh = tile / nqb;
  if (causal) qb = nqb - 1 - qb;  // longest rows first
  const int b = bh / H;
  const int q0 = qb * C::BR;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, r = lane & 31, g = lane >> 5;
  const size_t head = (size_t)bh * N * D;
  const u16* Kh = K + head;
  const u16* Vh = V + head;

  int kv_lim = N;
  if (kv_len) {
    const int L = kv_len[b];
    kv_lim = L < 0 ? 0 : (L > N ? N : L);
  }
  int kv_end = kv_lim;
  if (causal) kv_end = min(kv_end, q0 + C::BR);
  const int nt = (kv_end + BC - 1) / BC;

  const int q = q0 + 32 * w + r;  // this lane's query row
  const int wave_q_first = q0 + 32 * w;
  const int wave_q_last = wave_q_first + 31;

  bf16x8 qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (q < N) v = ld_global16(Q + head + (size_t)q * D + 16 * kk + 8 * g);
    qf[kk] = as_bf16x8(v);
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[t][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  u32x4 kreg[C::KCH], vreg[C::VKR];
  const int vkg = tid % C::NKG, vdc = tid / C::NKG;

  auto load_tile = [&](int kb) {
#pragma unroll
    for (int rr = 0; rr < C::KCH; ++rr) {
      const int c = tid + 256 * rr;
      const int key = kb + c / (D / 8);
      u32x4 v = {0u, 0u, 0u, 0u};
      if (key < N) v = ld_global16(Kh + (size_t)key * D + (c % (D / 8)) * 8);
      kreg[rr] = v;
    }
#pragma unroll
    for (int rr = 0; rr < C::VKR; ++rr) {
      const int key = kb + vkg * C::VKR + rr;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (key < N) v = ld_global16(Vh + (size_t)key * D + vdc * 8);
      vreg[rr] = v;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int rr = 0; rr < C::KCH; ++rr) {
      const int c = tid + 256 * rr;
      *reinterpret_cast<u32x4*>(&Ks[buf][(c / (D / 8)) * C::KSTR + (c % (D / 8)) * 8]) = kreg[rr];
    }
    const int col = swap23(vkg * C::VKR);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      u16* dst = &Vt[buf][(vdc * 8 + e) * C::VSTR + col];
      if constexpr (C::VKR == 4) {
        u32x2 p;
        p[0] = bf16_bits(vreg[0], e) | (bf16_bits(vreg[1], e) << 16);
        p[1] = bf16_bits(vreg[2], e) | (bf16_bits(vreg[3], e) << 16);
        *reinterpret_cast<u32x2*>(dst) = p;
      } else {
        *reinterpret_cast<unsigned*>(dst) = bf16_bits(vreg[0], e) | (bf16_bits(vreg[1], e) << 16);
      }
    }
  };

  if (nt > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int it = 0; it < nt; ++it) {
    const int buf = it & 1;
    const int kb = it * BC;
    if (it + 1 < nt) load_tile(kb + BC);

    if (!causal || kb <= wave_q_last) {
      // S^T tile: rows = keys kb + 32*mt + (8i + 4g + j), column = query q.
      f32x16 s[BC / 32];
#pragma unroll
      for (int mt = 0; mt < BC / 32; ++mt) {
#pragma unroll
        for (int e = 0; e < 16; ++e) s[mt][e] = 0.f;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
          s[mt] = mfma32(ld_lds16(&Ks[buf][(32 * mt + r) * C::KSTR + 16 * kk + 8 * g]), qf[kk], s[mt]);
      }

      const bool need_mask = (kb + BC > kv_lim) || (causal && kb + BC - 1 > wave_q_first);
      if (need_mask) {
#pragma unroll
        for (int mt = 0; mt < BC / 32; ++mt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kb + 32 * mt + 8 * (e >> 2) + 4 * g + (e & 3);
            if (key >= kv_lim || (causal && key > q)) s[mt][e] = -INFINITY;
          }
      }

      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < BC / 32; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[mt][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx * sl2);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float rs = 0.f;
#pragma unroll
      for (int mt = 0; mt < BC / 32; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = fast_exp2(s[mt][e] * sl2 - m_use);
          s[mt][e] = p;
          rs += p;
        }
      l_run = l_run * alpha + rs;
      m_run = m_new;
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[t][e] *= alpha;

      bf16x8 pb[BC / 16];
#pragma unroll
      for (int c = 0; c < BC / 16; ++c) pb[c] = pack_bf16x8(s[c >> 1], 8 * (c & 1));
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int c = 0; c < BC / 16; ++c)
          o[t] = mfma32(ld_lds16(&Vt[buf][(32 * t + r) * C::VSTR + 16 * c + 8 * g]), pb[c], o[t]);
    }

    if (it + 1 < nt) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q < N) {
    u16* orow = O + head + (size_t)q * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 p;
        __bf16 h0 = (__bf16)(o[t][4 * i + 0] * inv), h1 = (__bf16)(o[t][4 * i + 1] * inv);
        __bf16 h2 = (__bf16)(o[t][4 * i + 2] * inv), h3 = (__bf16)(o[t][4 * i + 3] * inv);
        p[0] = (unsigned)__builtin_bit_cast(u16, h0) | ((unsigned)__builtin_bit_cast(u16, h1) << 16);
        p[1] = (unsigned)__builtin_bit_cast(u16, h2) | ((unsigned)__builtin_bit_cast(u16, h3) << 16);
        *reinterpret_cast<u32x2*>(orow + 32 * t + 8 * i + 4 * g) = p;
      }
    if (g == 0) LSE[(size_t)bh * N + q] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D>
static hipError_t launch_fwd_d(const void* Q, const void* K, const void* V, void* O, float* LSE,
                               const AttnShape& s, hipStream_t stream) {
  const int nqb = (s.N + FwdCfg<D>::BR - 1) / FwdCfg<D>::BR;
  const int total = s.B * s.H * nqb;
  hipLaunchKernelGGL(fwd_bf16_kernel<D>, dim3(total), dim3(256), 0, stream,
                     static_cast<const u16*>(Q), static_cast<const u16*>(K),
                     static_cast<const u16*>(V), static_cast<u16*>(O), LSE, s.H, s.N,
                     s.scale * kLog2e, s.causal, s.kv_len, nqb, total);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(const void* Q, const void* K, const void* V, void* O, float* LSE,
                           const AttnShape& s, hipStream_t stream) {
  if (s.d == 64) return launch_fwd_d<64>(Q, K, V, O, LSE, s, stream);
  return launch_fwd_d<128>(Q, K, V, O, LSE, s, stream);
}

}  // namespace fa
