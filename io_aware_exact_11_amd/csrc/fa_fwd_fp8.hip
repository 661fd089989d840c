// 8-bit floating-point forward ("FlashAttention — why it mattered" and
// "FlashAttention and GPU Memory", chapter 11: FlashAttention-3 adds an
// 8-bit forward mode, the one place the method rounds away precision).
//
// Q, K and V arrive as OCP FP8 E4M3 codes with one fp32 dequantisation
// factor each; V is given transposed, [B, H, d, N], so that both operands of
// every matrix-core product are read along their contraction index. The
// scores and the running softmax are fp32 as in the bf16 forward; the
// unnormalised weights (at most 2^8 with the lazy rescale) are rounded to
// E4M3 only as the operand of the P V product. Products are the gfx950
// 32x32x64 E4M3 matrix-core instruction with unit block scales.
//
// One workgroup owns 128 query rows (4 waves of 32) and streams 64-key
// tiles: K as [64 keys][d] and V^T as [d][64 keys], byte tiles padded so the
// 32-byte operand reads of 16 consecutive rows fall in distinct banks, moved
// by direct buffer-to-LDS loads and double-buffered. V^T rows are N bytes,
// so a tile row's 16-byte loads run into the next row (keys >= N get zero
// weight) and, for the last row, past the head's range, which reads zeros
// dword by dword; N is a multiple of 4 (checked on the host) so that no
// dword straddles that end.
//
// Operand bytes: the instruction pairs byte b of lane group g in A with
// byte b of lane group g in B (both map it to the same k index), so
//   * S^T = K Q^T: lane (g, r) holds 32 bytes d = 64kk + 32g + 0..31 of key
//     row r (A) and of query row r (B);
//   * O^T += V^T P^T: lane (g, r) holds 32 bytes keys 32g + 0..31 of V^T row
//     d = 32t + r (A) and the weights of the same 32 keys for query r (B).
// The score layout leaves lane group g with the keys whose bit 2 equals g;
// one permlane32 swap per word hands each group the 32 consecutive keys it
// needs.
#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;

__device__ __forceinline__ f32x16 mfma_e4m3(i32x8 a, i32x8 b, f32x16 c) {
  // Block-scale exponents 127: scale factor 1 for both operands.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 ld_lds32(const uint8_t* p) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(p);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(p + 16);
  const i32x8 v = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  return v;
}

// Direct-to-LDS copy of ROWS rows of ROWB bytes (source rows src_stride
// bytes apart, starting at byte src0) into a tile whose rows are STRB bytes
// apart. Each wave instruction fills 1 KB of LDS, 16 bytes per lane; lanes
// that land in a row's padding re-read the row's first chunk. Reads past the
// end of the buffer resource give zeros.
template <int ROWB, int STRB, int ROWS, int NW>
__device__ __forceinline__ void bytes_to_lds(__amdgpu_buffer_rsrc_t rs, int src0, int src_stride, uint8_t* tile,
                                             int w, int lane) {
  constexpr int NBLK = ROWS * STRB / 1024;
  static_assert(ROWS * STRB % 1024 == 0, "whole 1 KB blocks");
#pragma unroll
  for (int i = 0; i < (NBLK + NW - 1) / NW; ++i) {
    const int blk = w + NW * i;
    if (NBLK % NW == 0 || blk < NBLK) {
      const int off = blk * 1024 + lane * 16;
      const int row = off / STRB, cb = off % STRB;
      const int src = src0 + row * src_stride + (cb < ROWB ? cb : 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(tile + blk * 1024), 16, src, 0, 0, 0);
    }
  }
}

template <int D>
struct Fp8Cfg {
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  static constexpr int BR = 32 * NW;
  static constexpr int BC = 64;
  static constexpr int KSTRB = D + 16;   // K tile row stride, bytes (36 or 20 banks: conflict-free)
  static constexpr int VSTRB = BC + 16;  // V^T tile row stride, bytes (20 banks)
};

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ Vt,
    u16* __restrict__ O, float* __restrict__ LSE, int H, int N, float sl2, float ov, int causal,
    const int32_t* __restrict__ kv_len, int nqb, int total) {
  using C = Fp8Cfg<D>;
  constexpr int BC = C::BC, KK = D / 64, TT = D / 32, NW = C::NW;
  __shared__ __attribute__((aligned(16))) uint8_t Kb0[BC * C::KSTRB];
  __shared__ __attribute__((aligned(16))) uint8_t Kb1[BC * C::KSTRB];
  __shared__ __attribute__((aligned(16))) uint8_t Vb0[D * C::VSTRB];
  __shared__ __attribute__((aligned(16))) uint8_t Vb1[D * C::VSTRB];

  const int tile = xcd_tile(blockIdx.x, total);
  int qb = tile % nqb;
  const int bh = tile / nqb;
  if (causal) qb = nqb - 1 - qb;  // longest rows first
  const int b = bh / H;
  const int q0 = qb * C::BR;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, r = lane & 31, g = lane >> 5;
  const size_t head = (size_t)bh * N * D;
  const unsigned head_bytes = (unsigned)N * D;
  const auto rQ = make_rsrc(Q + head, head_bytes);
  const auto rK = make_rsrc(K + head, head_bytes);
  const auto rV = make_rsrc(Vt + head, head_bytes);

  int kv_lim = N;
  if (kv_len) {
    const int L = kv_len[b];
    kv_lim = L < 0 ? 0 : (L > N ? N : L);
  }
  int kv_end = kv_lim;
  if (causal) kv_end = min(kv_end, q0 + C::BR);
  const int nt = (kv_end + BC - 1) / BC;
  const int wave_q_first = q0 + 32 * w, wave_q_last = wave_q_first + 31;
  const int q = wave_q_first + r;
  const int nt_w = causal ? min(nt, wave_q_last / BC + 1) : nt;

  i32x8 qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const unsigned off = (unsigned)(q * D + 64 * kk + 32 * g);
    const u32x4 lo = ld_buf16(rQ, off), hi = ld_buf16(rQ, off + 16);
    const i32x8 v = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    qf[kk] = v;
  }
  f32x16 o[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[t][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  auto load = [&](int kb, uint8_t* Kt, uint8_t* Vtt) __attribute__((always_inline)) {
    bytes_to_lds<D, C::KSTRB, BC, NW>(rK, kb * D, D, Kt, w, lane);
    bytes_to_lds<BC, C::VSTRB, D, NW>(rV, kb, N, Vtt, w, lane);
  };
  // One 64-key tile: scores, mask, running maximum, E4M3 weights, P V.
  auto compute = [&](int kb, const uint8_t* Kt, const uint8_t* Vtt) __attribute__((always_inline)) {
    f32x16 sv[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sv[mt][e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        sv[mt] = mfma_e4m3(ld_lds32(Kt + (32 * mt + r) * C::KSTRB + 64 * kk + 32 * g), qf[kk], sv[mt]);
    }
    if ((kb + BC > kv_lim) || (causal && kb + BC - 1 > wave_q_first)) {
      // Element e of score tile mt is key kb + 4g + c, c = 32mt + 8(e/4) + e%4: hidden iff c > lim.
      const int lim = min(kv_lim - 1, causal ? q : kv_lim - 1) - (kb + 4 * g);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int c = 32 * mt + 8 * (e >> 2) + (e & 3);
          sv[mt][e] = c > lim ? -INFINITY : sv[mt][e];
        }
    }
    float mx = sv[0][0];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = (mt == 0 ? 1 : 0); e < 16; ++e) mx = fmaxf(mx, sv[mt][e]);
    const float tmax = pair_max(mx) * sl2;
    if (__builtin_amdgcn_ballot_w64(tmax > m_run + 8.f) != 0) {
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[t][e] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float rs = 0.f;
    unsigned pw[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          p[j] = fast_exp2(sv[mt][4 * i + j] * sl2 - m_use);
          rs += p[j];
        }
        // Keys 32mt + 8i + 4g + 0..3, one byte each, lowest key first.
        int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
        wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], wd, true);
        pw[mt][i] = (unsigned)wd;
      }
    l_run += rs;
    // Lane group 0 takes keys 0..31 of the tile, group 1 keys 32..63.
    i32x8 pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto sw = __builtin_amdgcn_permlane32_swap(pw[0][i], pw[1][i], false, false);
      pb[2 * i] = (int)sw[0];
      pb[2 * i + 1] = (int)sw[1];
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) o[t] = mfma_e4m3(ld_lds32(Vtt + (32 * t + r) * C::VSTRB + 32 * g), pb, o[t]);
  };

  if (nt > 0) load(0, Kb0, Vb0);
  wait_vmem_all();
  __syncthreads();
  // Tile it sits in buffer it % 2; tile it+1 is loaded into the other one.
  auto step = [&](auto odd, int it) __attribute__((always_inline)) {
    constexpr bool P = decltype(odd)::value;
    if (it + 1 < nt) load((it + 1) * BC, P ? Kb0 : Kb1, P ? Vb0 : Vb1);
    if (it < nt_w) compute(it * BC, P ? Kb1 : Kb0, P ? Vb1 : Vb0);
    // Each wave waits for its own loads before the barrier publishes them.
    wait_vmem_all();
    __syncthreads();
  };
  for (int it = 0; it < nt; it += 2) {
    step(std::integral_constant<bool, false>{}, it);
    if (it + 1 < nt) step(std::integral_constant<bool, true>{}, it + 1);
  }

  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? ov / l_tot : 0.f;
  if (q < N) {
    u16* orow = O + head + (size_t)q * D;
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 pk;
        __bf16 h0 = (__bf16)(o[t][4 * i + 0] * inv), h1 = (__bf16)(o[t][4 * i + 1] * inv);
        __bf16 h2 = (__bf16)(o[t][4 * i + 2] * inv), h3 = (__bf16)(o[t][4 * i + 3] * inv);
        pk[0] = (unsigned)__builtin_bit_cast(u16, h0) | ((unsigned)__builtin_bit_cast(u16, h1) << 16);
        pk[1] = (unsigned)__builtin_bit_cast(u16, h2) | ((unsigned)__builtin_bit_cast(u16, h3) << 16);
        *reinterpret_cast<u32x2*>(orow + 32 * t + 8 * i + 4 * g) = pk;
      }
    if (g == 0) LSE[(size_t)bh * N + q] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D>
static hipError_t launch_fp8_d(const void* Q8, const void* K8, const void* Vt8, void* O, float* LSE,
                               const AttnShape& s, float dq, float dk, float dv, hipStream_t stream) {
  using C = Fp8Cfg<D>;
  const int nqb = (s.N + C::BR - 1) / C::BR;
  const int total = s.B * s.H * nqb;
  hipLaunchKernelGGL((fwd_fp8_kernel<D>), dim3(total), dim3(C::NT), 0, stream, static_cast<const uint8_t*>(Q8),
                     static_cast<const uint8_t*>(K8), static_cast<const uint8_t*>(Vt8), static_cast<u16*>(O), LSE,
                     s.H, s.N, s.scale * dq * dk * kLog2e, dv, s.causal, s.kv_len, nqb, total);
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const void* Q8, const void* K8, const void* Vt8, void* O, float* LSE, const AttnShape& s,
                          float dq, float dk, float dv, hipStream_t stream) {
  if (s.d == 64) return launch_fp8_d<64>(Q8, K8, Vt8, O, LSE, s, dq, dk, dv, stream);
  return launch_fp8_d<128>(Q8, K8, Vt8, O, LSE, s, dq, dk, dv, stream);
}

}  // namespace fa
