// Backward pass of exact attention for gfx950: bf16 inputs, fp32 gradients.
//
// The forward kept only O and one log-sum-exp per row; here the score and
// probability tiles are rebuilt block by block from Q, K, V
// ("FlashAttention and GPU Memory", chapter 09 Backward: recomputing beats
// reading; "FlashAttention does more arithmetic to move less data", move 4).
// With P_ij = exp(s q_i.k_j - LSE_i) the gradients are, by the chain rule,
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  dK = s dS^T Q,  dQ = s dS K,
// where D_i = sum_j P_ij dP_ij. Since O = P V, D_i equals dO_i . O_i, which a
// bandwidth-bound pre-pass computes from O and dO (default), or, with
// FA_BWD_PRECISE, a separate recompute pass sums P o dP exactly.
//
// Key-outer kernel (one workgroup per 128 keys of one (b, h), two such key
// blocks in causal grids, 4 waves of 32 keys; the d=128 instances without
// the precise or atomic-dQ modes run 8 waves on 256 keys and keep V in LDS,
// see below):
//   * the wave's K and V rows sit in registers as the B operands of
//     S = Q K^T and dP = dO V^T (32x32x16 bf16 products, fp32 accumulate);
//   * query blocks (64 rows at d=128, 32 at d=64) stream through LDS, stored both row-major
//     (A operand of S and dP) and transposed (A operand of dV^T = dO^T P and
//     dK^T = Q^T dS, whose B operands are the P and dS registers themselves);
//   * dV^T and dK^T for the wave's keys accumulate in registers across all
//     query blocks and are written once;
//   * dS goes to LDS, and the workgroup adds dQ_i += s dS K for its 128 keys
//     into the fp32 dQ output with hardware float atomics.
// Causal workgroups start at the first query block that can see their keys;
// waves whose keys are all invisible to a block skip its products.
#pragma once

#include <climits>
#include <type_traits>

#include "fa_common.h"
#include "fa_dropout.h"
#include "fa_launch.h"

namespace fa {

// D_i = sum_c dO[i,c] * O[i,c] in fp32 from the bf16 tensors; 16 lanes per row.
template <int D>
__global__ __launch_bounds__(256) void bwd_dot_kernel(const u16* __restrict__ O,
                                                      const u16* __restrict__ dO,
                                                      float* __restrict__ Dout, int rows) {
  constexpr int EPL = D / 16;  // elements per lane: 8 or 4
  const int gid = blockIdx.x * 256 + threadIdx.x;
  const int row = gid >> 4, sub = gid & 15;
  float acc = 0.f;
  if (row < rows) {
    const size_t off = (size_t)row * D + sub * EPL;
    if constexpr (EPL == 8) {
      const u32x4 a = ld_global16(O + off), c = ld_global16(dO + off);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        acc += __uint_as_float(bf16_bits(a, e) << 16) * __uint_as_float(bf16_bits(c, e) << 16);
    } else {
      const u32x2 a = *reinterpret_cast<const u32x2*>(O + off);
      const u32x2 c = *reinterpret_cast<const u32x2*>(dO + off);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const unsigned ab = (a[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
        const unsigned cb = (c[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
        acc += __uint_as_float(ab << 16) * __uint_as_float(cb << 16);
      }
    }
  }
  acc += __shfl_xor(acc, 8);
  acc += __shfl_xor(acc, 4);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 1);
  if (row < rows && sub == 0) Dout[row] = acc;
}

// D_i = sum_j P_ij dP_ij taken literally, for FA_BWD_PRECISE: a query-outer
// pass (one workgroup per 128 query rows, 32 per wave) that recomputes the
// score tile S^T = K Q^T and dP^T = V dO^T on the matrix cores, with both K
// and V tiles streamed row-major through double-buffered LDS and the wave's
// Q and dO rows held as B operands; P_ij = 2^(s_ij*scale*log2e - LSE_i*log2e)
// uses the saved LSE. Independent of O, so the bf16 rounding of O does not
// enter D.
template <int D>
struct ExactDCfg {
  static constexpr int BR = 128;
  static constexpr int BC = 64;
  static constexpr int KSTR = D + 8;
  static constexpr int KCH = BC * D / 8 / 256;
};

// DROP: dP of kept elements is scaled by the keep factor, dropped ones are 0
// (the mask regenerated as in the dQ kernel).
template <int D, bool DROP = false>
__global__ __launch_bounds__(256, 2) void bwd_exact_d_kernel(
    const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ V,
    const u16* __restrict__ dO, const float* __restrict__ LSE, float* __restrict__ Dout, int H,
    int N, float sl2, int causal, const int32_t* __restrict__ kv_len, int nqb, int total,
    DropParams dpar) {
  using C = ExactDCfg<D>;
  constexpr int BC = C::BC;
  __shared__ __attribute__((aligned(16))) u16 Ks[2][BC * C::KSTR];
  __shared__ __attribute__((aligned(16))) u16 Vs[2][BC * C::KSTR];

  const int tile = xcd_tile(blockIdx.x, total);
  int qb = tile % nqb;
  const int bh = tile / nqb;
  if (causal) qb = nqb - 1 - qb;
  const int b = bh / H;
  const int q0 = qb * C::BR;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, r = lane & 31, g = lane >> 5;
  const size_t head = (size_t)bh * N * D;

  int kv_lim = N;
  if (kv_len) {
    const int L = kv_len[b];
    kv_lim = L < 0 ? 0 : (L > N ? N : L);
  }
  int kv_end = kv_lim;
  if (causal) kv_end = min(kv_end, q0 + C::BR);
  const int nt = (kv_end + BC - 1) / BC;

  const int q = q0 + 32 * w + r;
  const int wave_q_first = q0 + 32 * w, wave_q_last = wave_q_first + 31;
  bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 a = {0u, 0u, 0u, 0u}, c = {0u, 0u, 0u, 0u};
    if (q < N) {
      a = ld_global16(Q + head + (size_t)q * D + 16 * kk + 8 * g);
      c = ld_global16(dO + head + (size_t)q * D + 16 * kk + 8 * g);
    }
    qf[kk] = as_bf16x8(a);
    df[kk] = as_bf16x8(c);
  }
  const float lse2 = q < N ? LSE[(size_t)bh * N + q] * kLog2e : INFINITY;
  float part = 0.f;

  u32x4 kreg[C::KCH], vreg[C::KCH];
  auto load_tile = [&](int kb) {
#pragma unroll
    for (int rr = 0; rr < C::KCH; ++rr) {
      const int c = tid + 256 * rr;
      const int key = kb + c / (D / 8);
      u32x4 a = {0u, 0u, 0u, 0u}, v = {0u, 0u, 0u, 0u};
      if (key < N) {
        a = ld_global16(K + head + (size_t)key * D + (c % (D / 8)) * 8);
        v = ld_global16(V + head + (size_t)key * D + (c % (D / 8)) * 8);
      }
      kreg[rr] = a;
      vreg[rr] = v;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int rr = 0; rr < C::KCH; ++rr) {
      const int c = tid + 256 * rr;
      const int off = (c / (D / 8)) * C::KSTR + (c % (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(&Ks[buf][off]) = kreg[rr];
      *reinterpret_cast<u32x4*>(&Vs[buf][off]) = vreg[rr];
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
      f32x16 s[BC / 32], dp[BC / 32];
#pragma unroll
      for (int mt = 0; mt < BC / 32; ++mt) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          s[mt][e] = 0.f;
          dp[mt][e] = 0.f;
        }
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          const int off = (32 * mt + r) * C::KSTR + 16 * kk + 8 * g;
          s[mt] = mfma32(ld_lds16(&Ks[buf][off]), qf[kk], s[mt]);
          dp[mt] = mfma32(ld_lds16(&Vs[buf][off]), df[kk], dp[mt]);
        }
      }
      const bool need_mask = (kb + BC > kv_lim) || (causal && kb + BC - 1 > wave_q_first);
      // Key kb + 4g + c, c = 32mt + 8(e/4) + e%4, is hidden iff c > lim.
      const int lim = need_mask ? min(kv_lim - 1, causal ? q : kv_lim - 1) - (kb + 4 * g) : INT_MAX;
#pragma unroll
      for (int mt = 0; mt < BC / 32; ++mt) {
        unsigned W[4];
        if constexpr (DROP) drop_words_query_lane(dpar, bh, q, kb + 32 * mt, g, lane, W);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int c = 32 * mt + 8 * (e >> 2) + (e & 3);
          float p = fast_exp2(s[mt][e] * sl2 - lse2);
          if (c > lim) p = 0.f;
          if constexpr (DROP)
            part += drop_keep(W, e, dpar.thresh) ? p * dp[mt][e] * dpar.keep_scale : 0.f;
          else
            part += p * dp[mt][e];
        }
      }
    }
    if (it + 1 < nt) store_tile(buf ^ 1);
    __syncthreads();
  }
  part += __shfl_xor(part, 32);
  if (q < N && g == 0) Dout[(size_t)bh * N + q] = part;
}

// ---------------------------------------------------------------- key-outer kernel
//
// Default backward: two kernels that each write their outputs once, no
// atomics. dK, dV come from the key-outer kernel below; dQ from a query-outer
// kernel shaped like the forward. Both recompute S and dP, so together they
// do 7 of the 5 algorithmic matrix products' worth of work, in exchange for
// no dQ accumulation traffic and no cross-workgroup dependency.
// FA_BWD_DQ_ATOMIC instead runs the key-outer kernel with DQ_ATOMIC set: it
// also forms dQ_i += dS K for its keys and adds it into dQ with fp32 atomics.

template <int D>
struct DkdvCfg {
  static constexpr int NW = 4;
  static constexpr int BKV = 32 * NW;          // keys per workgroup (32 per wave)
  // Query rows per block. At d=64 blocks of 32 rows keep the plain kernel
  // within 168 VGPRs, i.e. three waves per SIMD (backward +3% at N=1024 and
  // N=8192); the d=128 instances that hold K and V in registers run one wave
  // per SIMD, where 32-row blocks measured 4% slower. (The d=128 instances
  // with V in LDS override NW and BQ: dkdv_waves below.)
  static constexpr int BQ = D == 64 ? 32 : 64;
  // Q and dO tile row stride (elements) of the xpad layout (xpad_off): both
  // tiles are read row-wise and transposed, conflict-free in that layout.
  static constexpr int QSTR = D + 32;
  static constexpr int KCH = BKV * D / 8 / 256;
  static constexpr int DSTR = BKV + 8;         // dS tile row stride (row reads only)
};

// dK, dV for 32 keys per wave of one (b, h) (128 or 256 keys per workgroup).
// The wave's K and V rows are B operands held in registers (V in LDS in the
// d=128 instances without precise or atomic-dQ mode); query blocks of Q and
// dO stream through swizzled, double-buffered LDS tiles that serve as A
// operands both row-wise (S = Q K^T, dP = dO V^T) and transposed
// (dV^T = dO^T P, dK^T = Q^T dS, through ds_read_b64_tr_b16), with P and dS
// taken from registers.
//
// DROP: fused dropout regenerated from the generator state (fa_dropout.h):
// dV takes the kept weights, dP of kept elements is scaled by the keep
// factor and dropped ones contribute only the -P D term of dS.
// The d=128 instance (plain or with dropout) keeps V in LDS instead of
// registers and computes 32 query rows at a time: its registers then fit
// two waves per SIMD (the dropout one with a few spilled registers). It
// runs eight waves (256 keys) per workgroup, one workgroup per CU, on blocks
// of 64 query rows, so that each block brought into LDS (and each barrier)
// serves twice the products of a four-wave workgroup.
template <int D, bool PRECISE, bool DQ_ATOMIC, bool DROP>
constexpr bool dkdv_v_in_lds() { return D == 128 && !PRECISE && !DQ_ATOMIC; }
template <int D, bool PRECISE, bool DQ_ATOMIC, bool DROP>
constexpr int dkdv_waves() { return dkdv_v_in_lds<D, PRECISE, DQ_ATOMIC, DROP>() ? 8 : DkdvCfg<D>::NW; }

template <int D, bool PRECISE, bool DQ_ATOMIC, bool DROP = false>
__global__ __launch_bounds__((64 * dkdv_waves<D, PRECISE, DQ_ATOMIC, DROP>()), D == 64 && !PRECISE && !DQ_ATOMIC && !DROP
                                      ? 3
                                      : (dkdv_v_in_lds<D, PRECISE, DQ_ATOMIC, DROP>() ? 2 : 1)) void bwd_dkdv_kernel(
    const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ V,
    const u16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dg,
    float* __restrict__ dQ, float* __restrict__ dK, float* __restrict__ dV, int H, int N, float scale,
    float sl2, int causal, const int32_t* __restrict__ kv_len, int nkb, int total, DropParams dpar) {
  using C = DkdvCfg<D>;
  constexpr bool VLDS = dkdv_v_in_lds<D, PRECISE, DQ_ATOMIC, DROP>();
  constexpr int NW = dkdv_waves<D, PRECISE, DQ_ATOMIC, DROP>();
  constexpr int BKV = 32 * NW;
  constexpr int BQ = VLDS ? 64 : C::BQ;
  constexpr int NSPLIT = PRECISE ? 2 : 1;
  constexpr int QSTR = C::QSTR;
  // Q and dO blocks arrive by direct-to-LDS loads into padded tiles. The two
  // buffers of each tensor are separate arrays named at compile time (loop
  // unrolled by two), so the compiler does not make the reads of one buffer
  // wait for the loads in flight into the other.
  __shared__ __attribute__((aligned(16))) u16 Q0[BQ * QSTR];
  __shared__ __attribute__((aligned(16))) u16 Q1[BQ * QSTR];
  __shared__ __attribute__((aligned(16))) u16 G0[BQ * QSTR];
  __shared__ __attribute__((aligned(16))) u16 G1[BQ * QSTR];
  __shared__ __attribute__((aligned(16))) float lse2s[2][BQ];
  __shared__ __attribute__((aligned(16))) float Ds[2][BQ];  // -D_i
  // dQ path only: the workgroup's K rows (swizzled) and the dS tile(s).
  __shared__ __attribute__((aligned(16))) u16 Kt[DQ_ATOMIC ? C::BKV * D : 8];
  __shared__ __attribute__((aligned(16))) u16 dSs[DQ_ATOMIC ? NSPLIT * BQ * C::DSTR : 8];
  // V rows of the workgroup's keys (swizzled, read by rows as the B operand
  // of dP = dO V^T) when they are not held in registers.
  constexpr int VLSTR = D + 8;
  __shared__ __attribute__((aligned(16))) u16 Vl[VLDS ? BKV * VLSTR : 8];

  // Causal grids pair key block i with block nkb - 1 - i in one workgroup,
  // the one with more query rows (the lower) first, so that every workgroup
  // does the same work.
  const int per_head = causal ? (nkb + 1) / 2 : nkb;
  const int tile = xcd_tile(blockIdx.x, total);
  const int pi = tile % per_head;
  const int bh = tile / per_head;
  const int b = bh / H;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, r = lane & 31, g = lane >> 5;
  auto block = [&](const int kbi) {
    const int kb0 = kbi * BKV;
    const int kw0 = kb0 + 32 * w;
    const int key = kw0 + r;
    const size_t head = (size_t)bh * N * D;
    const unsigned head_bytes = (unsigned)N * D * 2;

    int kv_lim = N;
    if (kv_len) {
      const int L = kv_len[b];
      kv_lim = L < 0 ? 0 : (L > N ? N : L);
    }

    f32x16 dv[D / 32], dk[D / 32];
  #pragma unroll
    for (int t = 0; t < D / 32; ++t)
  #pragma unroll
      for (int e = 0; e < 16; ++e) {
        dv[t][e] = 0.f;
        dk[t][e] = 0.f;
      }

    if (kb0 < kv_lim) {
      const auto rQ = make_rsrc(Q + head, head_bytes);
      const auto rK = make_rsrc(K + head, head_bytes);
      const auto rV = make_rsrc(V + head, head_bytes);
      const auto rO = make_rsrc(dO + head, head_bytes);
      bf16x8 kf[D / 16], vf[VLDS ? 1 : D / 16];
  #pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const unsigned off = (unsigned)(key * D + 16 * kk + 8 * g) * 2;
        kf[kk] = as_bf16x8(ld_buf16(rK, off));
        if constexpr (!VLDS) vf[kk] = as_bf16x8(ld_buf16(rV, off));
      }
      if constexpr (VLDS) tile_to_lds_padded<D, VLSTR, BKV, NW>(rV, kb0, Vl, w, lane);
      // B operand of dP for d-chunk kk: this wave's key row 32w + r of Vl.
      const u16* vrow = Vl + (32 * w + r) * VLSTR + 8 * g;
      auto vop = [&](int kk) {
        if constexpr (VLDS)
          return ld_lds16(vrow + 16 * kk);
        else
          return vf[kk];
      };
      if constexpr (DQ_ATOMIC) {
  #pragma unroll
        for (int rr = 0; rr < C::KCH; ++rr) {
          const int c = tid + 256 * rr;
          const int row = c / (D / 8), col = (c % (D / 8)) * 8;
          *reinterpret_cast<u32x4*>(&Kt[swz_off<D>(row, col)]) =
              ld_buf16(rK, (unsigned)((kb0 + row) * D + col) * 2);
        }
      }

      const int nqb = (N + BQ - 1) / BQ;
      const int qb_start = causal ? kb0 / BQ : 0;
      // Row statistics of the head through buffer resources: raw loads only
      // here, arithmetic at store time, so that nothing waits on the prefetch
      // (memory counters retire in order) until the block is written to LDS.
      const auto rL = make_rsrc(LSE + (size_t)bh * N, (unsigned)N * 4);
      const auto rD = make_rsrc(Dg + (size_t)bh * N, (unsigned)N * 4);
      float lraw = 0.f, draw = 0.f;
      int qrow = 0;
      // Block q0: Q and dO rows straight into LDS; this thread's row
      // statistics raw into registers (scaled when stored).
      auto load = [&](int q0, u16* Qt, u16* Gt) {
        if constexpr (VLDS) {
          // 64-row tiles are twenty 1 KB blocks each: waves 0-3 fill the Q
          // tile and waves 4-7 the dO tile, five blocks per wave.
          const int ws = __builtin_amdgcn_readfirstlane(w);
          if (ws < NW / 2)
            tile_to_lds_xpad<D, QSTR, BQ, NW / 2>(rQ, q0, Qt, ws, lane);
          else
            tile_to_lds_xpad<D, QSTR, BQ, NW / 2>(rO, q0, Gt, ws - NW / 2, lane);
        } else {
          tile_to_lds_xpad<D, QSTR, BQ, C::NW>(rQ, q0, Qt, w, lane);
          tile_to_lds_xpad<D, QSTR, BQ, C::NW>(rO, q0, Gt, w, lane);
        }
        qrow = q0 + (tid & (BQ - 1));
        lraw = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rL, (unsigned)qrow * 4, 0, 0));
        draw = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rD, (unsigned)qrow * 4, 0, 0));
      };
      auto store = [&](int buf) {
        if (tid < BQ) {
          // rows past N: weight 0 (LSE = +inf) and no D term. Stored as -D
          // (dropout: -D / keep_scale), the start value of the dP product.
          lse2s[buf][tid] = qrow < N ? lraw * kLog2e : INFINITY;
          Ds[buf][tid] = qrow < N ? (DROP ? -draw / dpar.keep_scale : -draw) : 0.f;
        }
      };
      // Transposing-read coordinates of this lane (see ld_lds_tr): row part
      // 4g + (lane % 16) / 4 inside a 16-row chunk, column part
      // 16 * ((lane / 16) % 2) + 4 * (lane % 4) inside a 32-column tile.
      const int tr_row = 4 * g + ((lane & 15) >> 2);
      const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      // This lane's offsets in the xpad tiles. Row-wise: chunk 2kk + g of row
      // 32qt + r is at rw[kk % 2] + 32qt*QSTR + 32(kk / 2) (bits 2..3 of the row
      // are those of r). Transposed: columns 32t + tr_col of rows
      // 16c + tr_row + 8j are at tw[j] + 16c*QSTR + 32t (bits 2..3 of those
      // rows are g + 2j).
      const int xr = (r >> 2) & 3;
      const int rw0 = r * QSTR + 8 * (g ^ xr), rw1 = r * QSTR + 8 * ((2 + g) ^ xr);
      const int tw0 = tr_row * QSTR + 8 * ((tr_col >> 3) ^ g) + (tr_col & 7);
      const int tw1 = (tr_row + 8) * QSTR + 8 * ((tr_col >> 3) ^ g ^ 2) + (tr_col & 7);

      load(qb_start * BQ, Q0, G0);
      wait_vmem_all();
      store(0);
      __syncthreads();
      // Block qb: its tiles in buffer (qb - qb_start) % 2, the next block's
      // loaded into the other meanwhile.
      auto step = [&](auto odd, int qb) {
        constexpr int buf = decltype(odd)::value ? 1 : 0;
        const u16* Qt = buf ? Q1 : Q0;
        const u16* Gt = buf ? G1 : G0;
        const int q0 = qb * BQ;
        if (qb + 1 < nqb) load(q0 + BQ, buf ? Q0 : Q1, buf ? G0 : G1);

        if constexpr (VLDS) {
          // 32 query rows at a time (sub-block sb: rows q0 + 32sb ..).
  #pragma unroll
          for (int sb = 0; sb < BQ / 32; ++sb) {
            const int qs = q0 + 32 * sb;
            if (!((kw0 < kv_lim) && (!causal || qs + 31 >= kw0))) continue;
            const int rb = 32 * sb * QSTR;
            // S = Q K^T, dP = dO V^T: rows = queries qs + 8i + 4g + j, column
            // = key; dP accumulates onto -D_i of its row.
            f32x16 sa = mfma32_first(ld_lds16(Qt + rb + rw0), kf[0]);
            f32x16 pa;
            {
              f32x16 nd;
  #pragma unroll
              for (int i = 0; i < 4; ++i) {
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(&Ds[buf][32 * sb + 8 * i + 4 * g]);
  #pragma unroll
                for (int j = 0; j < 4; ++j) nd[4 * i + j] = d4[j];
              }
              pa = mfma32(ld_lds16(Gt + rb + rw0), vop(0), nd);
            }
  #pragma unroll
            for (int kk = 1; kk < D / 16; ++kk) {
              const int o = rb + 32 * (kk >> 1) + ((kk & 1) ? rw1 : rw0);
              sa = mfma32(ld_lds16(Qt + o), kf[kk], sa);
              pa = mfma32(ld_lds16(Gt + o), vop(kk), pa);
            }
            // Operand reads one d-chunk ahead of the products.
            __builtin_amdgcn_sched_group_barrier(0x100, 7, 0);
  #pragma unroll
            for (int kk = 1; kk < D / 16; ++kk) {
              __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
              __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            if ((kw0 + 31 >= kv_lim) || (causal && qs < kw0 + 31)) {
              // Element e is query qs + 4g + c, c = 8(e/4) + e%4; hidden iff c < lim.
              const int lim = key >= kv_lim ? INT_MAX : (causal ? key - qs - 4 * g : INT_MIN);
  #pragma unroll
              for (int e = 0; e < 16; ++e) {
                const int c = 8 * (e >> 2) + (e & 3);
                sa[e] = c < lim ? -INFINITY : sa[e];
              }
            }
            unsigned W[4];
            if constexpr (DROP) drop_words_key_lane(dpar, bh, key, qs, g, lane, W);
  #pragma unroll
            for (int i = 0; i < 4; ++i) {
              const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse2s[buf][32 * sb + 8 * i + 4 * g]);
              f32x4 d4 = {};
              if constexpr (DROP) d4 = *reinterpret_cast<const f32x4*>(&Ds[buf][32 * sb + 8 * i + 4 * g]);
  #pragma unroll
              for (int j = 0; j < 4; ++j) {
                const int e = 4 * i + j;
                const float p = fast_exp2(sa[e] * sl2 - l4[j]);
                if constexpr (DROP) {
                  // kept: p (ks dP - D); dropped: -p D (d4 holds -D / ks)
                  const bool keep = drop_keep(W, e, dpar.thresh);
                  sa[e] = keep ? p : 0.f;
                  pa[e] = (p * dpar.keep_scale) * (keep ? pa[e] : d4[j]);
                } else {
                  sa[e] = p;
                  pa[e] = p * pa[e];
                }
              }
            }
            bf16x8 pb[2], db[2];
  #pragma unroll
            for (int h = 0; h < 2; ++h) {
              pb[h] = pack_bf16x8(sa, 8 * h);
              db[h] = pack_bf16x8(pa, 8 * h);
            }
            // dV^T += dO^T P, dK^T += Q^T dS over the sub-block's query
            // chunks c = 2sb + h.
  #pragma unroll
            for (int t = 0; t < D / 32; ++t)
  #pragma unroll
              for (int h = 0; h < 2; ++h) {
                const int o = 16 * (2 * sb + h) * QSTR + 32 * t;
                const bf16x8 aO = join_tr(ld_lds_tr(Gt + o + tw0), ld_lds_tr(Gt + o + tw1));
                const bf16x8 aQ = join_tr(ld_lds_tr(Qt + o + tw0), ld_lds_tr(Qt + o + tw1));
                dv[t] = mfma32(aO, pb[h], dv[t]);
                dk[t] = mfma32(aQ, db[h], dk[t]);
              }
            // Transposing reads two (t, h) steps ahead of the products.
            __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
  #pragma unroll
            for (int i = 2; i < (D / 32) * 2; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
          }
        } else if ((kw0 < kv_lim) && (!causal || q0 + BQ - 1 >= kw0)) {
          // S = Q K^T, dP = dO V^T: rows = queries 32*qt + 8i + 4g + j, column = key.
          f32x16 sa[BQ / 32], pa[BQ / 32];
  #pragma unroll
          for (int qt = 0; qt < BQ / 32; ++qt) {
            const int rb = 32 * qt * QSTR;
            sa[qt] = mfma32_first(ld_lds16(Qt + rb + rw0), kf[0]);
            {
              // dP - D_i in one pass: the product accumulates onto -D_i of its
              // row (element 4i + j is query 32qt + 8i + 4g + j); with dropout
              // onto -D_i / keep_scale.
              f32x16 nd;
  #pragma unroll
              for (int i = 0; i < 4; ++i) {
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(&Ds[buf][32 * qt + 8 * i + 4 * g]);
  #pragma unroll
                for (int j = 0; j < 4; ++j) nd[4 * i + j] = d4[j];
              }
              pa[qt] = mfma32(ld_lds16(Gt + rb + rw0), vop(0), nd);
            }
  #pragma unroll
            for (int kk = 1; kk < D / 16; ++kk) {
              const int o = rb + 32 * (kk >> 1) + ((kk & 1) ? rw1 : rw0);
              sa[qt] = mfma32(ld_lds16(Qt + o), kf[kk], sa[qt]);
              pa[qt] = mfma32(ld_lds16(Gt + o), vop(kk), pa[qt]);
            }
          }
          // Masked scores become -inf, so their weights come out exactly 0.
          if ((kw0 + 31 >= kv_lim) || (causal && q0 < kw0 + 31)) {
            // Element e of tile qt is query q0 + 4g + c with the constant
            // c = 32qt + 8(e/4) + e%4; this lane's key is hidden from it iff the
            // key is >= kv_lim (every c) or, causal, key > query (c < lim).
            const int lim = key >= kv_lim ? INT_MAX : (causal ? key - q0 - 4 * g : INT_MIN);
  #pragma unroll
            for (int qt = 0; qt < BQ / 32; ++qt)
  #pragma unroll
              for (int e = 0; e < 16; ++e) {
                const int c = 32 * qt + 8 * (e >> 2) + (e & 3);
                sa[qt][e] = c < lim ? -INFINITY : sa[qt][e];
              }
          }
  #pragma unroll
          for (int qt = 0; qt < BQ / 32; ++qt) {
            unsigned W[4];
            if constexpr (DROP) drop_words_key_lane(dpar, bh, key, q0 + 32 * qt, g, lane, W);
  #pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int ql = 32 * qt + 8 * i + 4 * g;
              const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse2s[buf][ql]);
              f32x4 d4 = {};
              if constexpr (DROP) d4 = *reinterpret_cast<const f32x4*>(&Ds[buf][ql]);
  #pragma unroll
              for (int j = 0; j < 4; ++j) {
                const int e = 4 * i + j;
                const float p = fast_exp2(sa[qt][e] * sl2 - l4[j]);
                if constexpr (DROP) {
                  const bool keep = drop_keep(W, e, dpar.thresh);
                  sa[qt][e] = keep ? p : 0.f;
                  // kept: p (ks dP - D); dropped: -p D (d4 holds -D / ks)
                  pa[qt][e] = (p * dpar.keep_scale) * (keep ? pa[qt][e] : d4[j]);
                } else {
                  sa[qt][e] = p;
                  pa[qt][e] = p * pa[qt][e];
                }
              }
            }
          }
          bf16x8 pb[BQ / 16], db[BQ / 16], pl[PRECISE ? BQ / 16 : 1], dl[PRECISE ? BQ / 16 : 1];
  #pragma unroll
          for (int c = 0; c < BQ / 16; ++c) {
            if constexpr (PRECISE) {
              pack_split_bf16x8(sa[c >> 1], 8 * (c & 1), pb[c], pl[c]);
              pack_split_bf16x8(pa[c >> 1], 8 * (c & 1), db[c], dl[c]);
            } else {
              pb[c] = pack_bf16x8(sa[c >> 1], 8 * (c & 1));
              db[c] = pack_bf16x8(pa[c >> 1], 8 * (c & 1));
            }
          }
          // dV^T += dO^T P and dK^T += Q^T dS: A = the transposed tile (rows d =
          // 32t + r, k-slots = queries 16c + 8h + 4g + 0..3 for slots 4h..4h+3),
          // B = P / dS registers in the same slot order.
  #pragma unroll
          for (int t = 0; t < D / 32; ++t)
  #pragma unroll
            for (int c = 0; c < BQ / 16; ++c) {
              const int o = 16 * c * QSTR + 32 * t;
              const bf16x8 aO = join_tr(ld_lds_tr(Gt + o + tw0), ld_lds_tr(Gt + o + tw1));
              const bf16x8 aQ = join_tr(ld_lds_tr(Qt + o + tw0), ld_lds_tr(Qt + o + tw1));
              dv[t] = mfma32(aO, pb[c], dv[t]);
              dk[t] = mfma32(aQ, db[c], dk[t]);
              if constexpr (PRECISE) {
                dv[t] = mfma32(aO, pl[c], dv[t]);
                dk[t] = mfma32(aQ, dl[c], dk[t]);
              }
            }
          if constexpr (DQ_ATOMIC) {
            // dS (bf16, and its low half in precise mode) into the [query][key]
            // tile: slot s of chunk c is query 16c + 8(s/4) + 4g + s%4.
  #pragma unroll
            for (int part = 0; part < NSPLIT; ++part) {
              u16* dst = dSs + part * BQ * C::DSTR;
  #pragma unroll
              for (int c = 0; c < BQ / 16; ++c) {
                const u32x4 words = __builtin_bit_cast(u32x4, part == 0 ? db[c] : dl[PRECISE ? c : 0]);
  #pragma unroll
                for (int s8 = 0; s8 < 8; ++s8) {
                  const int ql = 16 * c + 8 * (s8 >> 2) + 4 * g + (s8 & 3);
                  dst[ql * C::DSTR + 32 * w + r] = (u16)(words[s8 >> 1] >> ((s8 & 1) * 16));
                }
              }
            }
          }
        } else if constexpr (DQ_ATOMIC) {
          for (int idx = lane; idx < NSPLIT * BQ * 4; idx += 64) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(&dSs[(idx >> 2) * C::DSTR + 32 * w + 8 * (idx & 3)]) = z;
          }
        }

        if constexpr (DQ_ATOMIC) {
          __syncthreads();
          // dQ_i += s dS K over the workgroup's keys: 32x32 tiles (qt, dt) split
          // over the waves; A = dS rows, B = K^T read transposed from Kt with
          // the natural key order (k-slots 16c + 8g + 0..7).
          constexpr int NT = (BQ / 32) * (D / 32);
          const int kt_row = 8 * g + ((lane & 15) >> 2);
          for (int tt = w; tt < NT; tt += C::NW) {
            const int qt = tt / (D / 32), dt = tt % (D / 32);
            f32x16 acc;
  #pragma unroll
            for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  #pragma unroll
            for (int c = 0; c < C::BKV / 16; ++c) {
              const int r0 = 16 * c + kt_row, col = 32 * dt + tr_col;
              const bf16x8 bK = join_tr(ld_lds_tr(&Kt[swz_off<D>(r0, col)]),
                                        ld_lds_tr(&Kt[swz_off<D>(r0 + 4, col)]));
  #pragma unroll
              for (int part = 0; part < NSPLIT; ++part)
                acc = mfma32(ld_lds16(&dSs[(part * BQ + 32 * qt + r) * C::DSTR + 16 * c + 8 * g]), bK, acc);
            }
  #pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int qq = q0 + 32 * qt + 8 * (e >> 2) + 4 * g + (e & 3);
              if (qq < N) unsafeAtomicAdd(dQ + head + (size_t)qq * D + 32 * dt + r, acc[e] * scale);
            }
          }
        }
        // Each wave waits for its own loads before the barrier publishes them.
        wait_vmem_all();
        if (qb + 1 < nqb) store(buf ^ 1);
        __syncthreads();
      };
      for (int qb = qb_start; qb < nqb; qb += 2) {
        step(std::integral_constant<bool, false>{}, qb);
        if (qb + 1 < nqb) step(std::integral_constant<bool, true>{}, qb + 1);
      }
    }

    if (key < N) {
      float* dkrow = dK + head + (size_t)key * D;
      float* dvrow = dV + head + (size_t)key * D;
  #pragma unroll
      for (int t = 0; t < D / 32; ++t)
  #pragma unroll
        for (int i = 0; i < 4; ++i) {
          f32x4 a, c;
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            a[j] = dk[t][4 * i + j] * scale;
            c[j] = DROP ? dv[t][4 * i + j] * dpar.keep_scale : dv[t][4 * i + j];
          }
          *reinterpret_cast<f32x4*>(dkrow + 32 * t + 8 * i + 4 * g) = a;
          *reinterpret_cast<f32x4*>(dvrow + 32 * t + 8 * i + 4 * g) = c;
        }
    }
  };
  block(pi);
  if (causal && nkb - 1 - pi != pi) {
    // The first block's waves are past their last barrier: no LDS reads of
    // it remain.
    __syncthreads();
    block(nkb - 1 - pi);
  }
}

template <int D>
struct DqCfg {
  static constexpr int NW = 4;
  static constexpr int BR = 32 * NW;           // query rows per workgroup
  static constexpr int BC = 64;                // keys per tile
  // LDS row strides (elements). K is read row-wise and transposed, from an
  // xpad tile (xpad_off), conflict-free for both. V is read row-wise only:
  // a padded step of 4 banks.
  static constexpr int KSTR = D + 32;
  static constexpr int VSTR = D + 8;
};

// dQ for 128 query rows of one (b, h), written once. Shaped like the
// forward: S^T = K Q^T and dP^T = V dO^T with the wave's Q and dO rows as B
// operands, so each lane holds one query's P and dS for 32 keys of a tile;
// dQ^T += K^T dS^T takes dS from those registers and K^T from the same
// (padded) K tile through transposing reads. K and V tiles arrive by
// direct buffer-to-LDS loads, double-buffered, which keeps the kernel's
// registers within two waves per SIMD without spilling.
//
// Outside precise mode the kernel also forms the per-row term itself,
// D_i = dO_i . O_i, from the dO rows it already holds and one read of O, and
// stores it to Dg for the dK/dV kernel that runs after it (no separate
// pre-pass). In precise mode it reads the exact D_i from Dg.
//
// DROP: fused dropout regenerated from the generator state (fa_dropout.h);
// dP of kept elements is scaled by the keep factor, dropped ones give
// dS = -P D.
template <int D, bool PRECISE, bool DROP = false>
__global__ __launch_bounds__(256, PRECISE ? 1 : (D == 64 && !DROP ? 3 : 2)) void bwd_dq_kernel(
    const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ V,
    const u16* __restrict__ O, const u16* __restrict__ dO, const float* __restrict__ LSE,
    float* __restrict__ Dg, float* __restrict__ dQ, int H, int N, float scale, float sl2, int causal,
    const int32_t* __restrict__ kv_len, int nqb, int total, DropParams dpar) {
  using C = DqCfg<D>;
  constexpr int BC = C::BC, KSTR = C::KSTR, VSTR = C::VSTR;
  // Tiles arrive by direct-to-LDS loads. The two buffers of each tensor are
  // separate arrays named at compile time (loop unrolled by two), so the
  // compiler does not make the reads of one buffer wait for the loads in
  // flight into the other.
  __shared__ __attribute__((aligned(16))) u16 K0[BC * KSTR];
  __shared__ __attribute__((aligned(16))) u16 K1[BC * KSTR];
  __shared__ __attribute__((aligned(16))) u16 V0[BC * VSTR];
  __shared__ __attribute__((aligned(16))) u16 V1[BC * VSTR];

  // Causal grids pair query block i with block nqb - 1 - i in one
  // workgroup, the longer first, so that every workgroup does the same work.
  const int per_head = causal ? (nqb + 1) / 2 : nqb;
  const int tile = xcd_tile(blockIdx.x, total);
  const int pi = tile % per_head;
  const int bh = tile / per_head;
  const int b = bh / H;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, r = lane & 31, g = lane >> 5;
  const size_t head = (size_t)bh * N * D;
  const unsigned head_bytes = (unsigned)N * D * 2;
  const auto rQ = make_rsrc(Q + head, head_bytes);
  const auto rK = make_rsrc(K + head, head_bytes);
  const auto rV = make_rsrc(V + head, head_bytes);
  const auto rO = make_rsrc(dO + head, head_bytes);

  int kv_lim = N;
  if (kv_len) {
    const int L = kv_len[b];
    kv_lim = L < 0 ? 0 : (L > N ? N : L);
  }
  auto block = [&](const int qb) {
    const int q0 = qb * C::BR;
    int kv_end = kv_lim;
    if (causal) kv_end = min(kv_end, q0 + C::BR);
    const int nt = (kv_end + BC - 1) / BC;
    const int q = q0 + 32 * w + r;
    const int wave_q_first = q0 + 32 * w, wave_q_last = wave_q_first + 31;
    const int nt_w = causal ? min(nt, wave_q_last / BC + 1) : nt;

    bf16x8 qf[D / 16], df[D / 16];
  #pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const unsigned off = (unsigned)(q * D + 16 * kk + 8 * g) * 2;
      qf[kk] = as_bf16x8(ld_buf16(rQ, off));
      df[kk] = as_bf16x8(ld_buf16(rO, off));
    }
    const float lse2 = q < N ? LSE[(size_t)bh * N + q] * kLog2e : INFINITY;
    float Dq;
    if constexpr (PRECISE) {
      Dq = q < N ? Dg[(size_t)bh * N + q] : 0.f;
    } else {
      // This lane holds d-chunks 16kk + 8g .. +7 of the row's dO; its partner
      // lane (lane ^ 32) holds the other half. Rows past N read zeros.
      const auto rOut = make_rsrc(O + head, head_bytes);
      float part = 0.f;
  #pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const u32x4 ov = ld_buf16(rOut, (unsigned)(q * D + 16 * kk + 8 * g) * 2);
        const u32x4 gv = __builtin_bit_cast(u32x4, df[kk]);
  #pragma unroll
        for (int e = 0; e < 8; ++e)
          part += __uint_as_float(bf16_bits(ov, e) << 16) * __uint_as_float(bf16_bits(gv, e) << 16);
      }
      Dq = pair_sum(part);
      if (q < N && g == 0) Dg[(size_t)bh * N + q] = Dq;
    }

    f32x16 acc[D / 32];
  #pragma unroll
    for (int t = 0; t < D / 32; ++t)
  #pragma unroll
      for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;
    f32x16 ndq;
  #pragma unroll
    for (int e = 0; e < 16; ++e) ndq[e] = -Dq;

    auto load = [&](int kb, u16* Kt, u16* Vt) {
      tile_to_lds_xpad<D, KSTR, BC, C::NW>(rK, kb, Kt, w, lane);
      tile_to_lds_padded<D, VSTR, BC, C::NW>(rV, kb, Vt, w, lane);
    };
    const int tr_row = 4 * g + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    // This lane's offsets in the xpad K tile, as in the dK/dV kernel: row-wise
    // chunk 2kk + g of row 32mt + r at rw[kk % 2] + 32mt*KSTR + 32(kk / 2);
    // transposed columns 32t + tr_col of rows 16c + tr_row + 8j at
    // tw[j] + 16c*KSTR + 32t.
    const int xr = (r >> 2) & 3;
    const int rw0 = r * KSTR + 8 * (g ^ xr), rw1 = r * KSTR + 8 * ((2 + g) ^ xr);
    const int tw0 = tr_row * KSTR + 8 * ((tr_col >> 3) ^ g) + (tr_col & 7);
    const int tw1 = (tr_row + 8) * KSTR + 8 * ((tr_col >> 3) ^ g ^ 2) + (tr_col & 7);

    if (nt > 0) load(0, K0, V0);
    wait_vmem_all();
    __syncthreads();
    // Tile it: K_it, V_it in buffer it % 2; tile it+1 is loaded into the other.
    auto step = [&](auto odd, int it) {
      constexpr bool P = decltype(odd)::value;
      const u16* Kc = P ? K1 : K0;
      const u16* Vc = P ? V1 : V0;
      const int kb = it * BC;
      if (it + 1 < nt) load(kb + BC, P ? K0 : K1, P ? V0 : V1);
      if (it < nt_w) {
        // One 32-key half of the tile at a time: its score and dP products,
        // mask, dS and dQ products, which keeps the live score registers to
        // one half.
        const bool need_mask = (kb + BC > kv_lim) || (causal && kb + BC - 1 > wave_q_first);
        // Key kb + 4g + c, c = 32mt + 8(e/4) + e%4, is hidden iff c > lim.
        const int lim = min(kv_lim - 1, causal ? q : kv_lim - 1) - (kb + 4 * g);
  #pragma unroll
        for (int mt = 0; mt < BC / 32; ++mt) {
          const int row = 32 * mt + r;
          f32x16 s = mfma32_first(ld_lds16(Kc + 32 * mt * KSTR + rw0), qf[0]);
          // Plain mode: the dP product accumulates onto -D_i, so that
          // dS = P (dP - D_i) is one multiply.
          f32x16 dp = (PRECISE || DROP) ? mfma32_first(ld_lds16(Vc + row * VSTR + 8 * g), df[0])
                                        : mfma32(ld_lds16(Vc + row * VSTR + 8 * g), df[0], ndq);
  #pragma unroll
          for (int kk = 1; kk < D / 16; ++kk) {
            s = mfma32(ld_lds16(Kc + 32 * mt * KSTR + 32 * (kk >> 1) + ((kk & 1) ? rw1 : rw0)), qf[kk], s);
            dp = mfma32(ld_lds16(Vc + row * VSTR + 16 * kk + 8 * g), df[kk], dp);
          }
          if constexpr (!PRECISE && !DROP) {
            // Operand reads two d-chunks ahead of the products.
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
  #pragma unroll
            for (int i = 2; i < D / 16; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
          }
          if (need_mask) {
  #pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int c = 32 * mt + 8 * (e >> 2) + (e & 3);
              s[e] = c > lim ? -INFINITY : s[e];
            }
          }
          unsigned W[4];
          if constexpr (DROP) drop_words_query_lane(dpar, bh, q, kb + 32 * mt, g, lane, W);
  #pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float p = fast_exp2(s[e] * sl2 - lse2);
            if constexpr (DROP)
              dp[e] = p * ((drop_keep(W, e, dpar.thresh) ? dp[e] * dpar.keep_scale : 0.f) - Dq);
            else if constexpr (PRECISE)
              dp[e] = p * (dp[e] - Dq);
            else
              dp[e] = p * dp[e];
          }
          bf16x8 db[2], dl[PRECISE ? 2 : 1];
  #pragma unroll
          for (int h = 0; h < 2; ++h) {
            if constexpr (PRECISE)
              pack_split_bf16x8(dp, 8 * h, db[h], dl[h]);
            else
              db[h] = pack_bf16x8(dp, 8 * h);
          }
          // dQ^T += K^T dS^T: A = K^T rows d = 32t + r, k-slots = keys of
          // chunk c = 2mt + h.
  #pragma unroll
          for (int t = 0; t < D / 32; ++t)
  #pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int o = 16 * (2 * mt + h) * KSTR + 32 * t;
              const bf16x8 aK = join_tr(ld_lds_tr(Kc + o + tw0), ld_lds_tr(Kc + o + tw1));
              acc[t] = mfma32(aK, db[h], acc[t]);
              if constexpr (PRECISE) acc[t] = mfma32(aK, dl[h], acc[t]);
            }
          if constexpr (!PRECISE && !DROP) {
            // Transposing reads two products ahead.
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
  #pragma unroll
            for (int i = 2; i < D / 32 * 2; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          }
        }
      }
      // Each wave waits for its own loads before the barrier publishes them.
      wait_vmem_all();
      __syncthreads();
    };
    for (int it = 0; it < nt; it += 2) {
      step(std::integral_constant<bool, false>{}, it);
      if (it + 1 < nt) step(std::integral_constant<bool, true>{}, it + 1);
    }

    if (q < N) {
      float* row = dQ + head + (size_t)q * D;
  #pragma unroll
      for (int t = 0; t < D / 32; ++t)
  #pragma unroll
        for (int i = 0; i < 4; ++i) {
          f32x4 a;
  #pragma unroll
          for (int j = 0; j < 4; ++j) a[j] = acc[t][4 * i + j] * scale;
          *reinterpret_cast<f32x4*>(row + 32 * t + 8 * i + 4 * g) = a;
        }
    }
  };
  block(causal ? nqb - 1 - pi : pi);
  if (causal && nqb - 1 - pi != pi) {
    // The first block's waves are past their last barrier: no LDS reads of
    // it remain.
    __syncthreads();
    block(pi);
  }
}

template <int D, bool PRECISE, bool DQ_ATOMIC, bool DROP = false>
static void launch_dkdv(const u16* q, const u16* k, const u16* v, const u16* g, const float* LSE,
                        const float* Dws, float* dQ, float* dK, float* dV, const AttnShape& s, float sl2,
                        hipStream_t stream, DropParams dp = {}) {
  constexpr int NW = dkdv_waves<D, PRECISE, DQ_ATOMIC, DROP>();
  const int nkb = (s.N + 32 * NW - 1) / (32 * NW);
  const int total = s.B * s.H * (s.causal ? (nkb + 1) / 2 : nkb);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, PRECISE, DQ_ATOMIC, DROP>), dim3(total), dim3(64 * NW), 0, stream, q, k, v,
                     g, LSE, Dws, dQ, dK, dV, s.H, s.N, s.scale, sl2, s.causal, s.kv_len, nkb, total, dp);
}

template <int D, bool PRECISE, bool DROP = false>
static void launch_dq(const u16* q, const u16* k, const u16* v, const u16* o, const u16* g,
                      const float* LSE, float* Dws, float* dQ, const AttnShape& s, float sl2,
                      hipStream_t stream, DropParams dp = {}) {
  const int nqb = (s.N + DqCfg<D>::BR - 1) / DqCfg<D>::BR;
  const int total = s.B * s.H * (s.causal ? (nqb + 1) / 2 : nqb);
  hipLaunchKernelGGL((bwd_dq_kernel<D, PRECISE, DROP>), dim3(total), dim3(256), 0, stream, q, k, v, o, g, LSE,
                     Dws, dQ, s.H, s.N, s.scale, sl2, s.causal, s.kv_len, nqb, total, dp);
}

// Entry points of the translation units: the key-outer kernel per head
// size, and (in a unit of its own, compiled with the default scheduler) its
// variants that also accumulate dQ with atomics.
template <int D>
static hipError_t launch_dkdv_default(const BwdArgs& a, const AttnShape& s, bool precise, hipStream_t stream) {
  const float sl2 = s.scale * kLog2e;
  const u16* q = static_cast<const u16*>(a.Q);
  const u16* k = static_cast<const u16*>(a.K);
  const u16* v = static_cast<const u16*>(a.V);
  const u16* g = static_cast<const u16*>(a.dO);
  if (precise)
    launch_dkdv<D, true, false>(q, k, v, g, a.LSE, a.Dws, a.dQ, a.dK, a.dV, s, sl2, stream);
  else
    launch_dkdv<D, false, false>(q, k, v, g, a.LSE, a.Dws, a.dQ, a.dK, a.dV, s, sl2, stream);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_dkdv_atomic(const BwdArgs& a, const AttnShape& s, bool precise, hipStream_t stream) {
  const float sl2 = s.scale * kLog2e;
  const u16* q = static_cast<const u16*>(a.Q);
  const u16* k = static_cast<const u16*>(a.K);
  const u16* v = static_cast<const u16*>(a.V);
  const u16* g = static_cast<const u16*>(a.dO);
  if (precise)
    launch_dkdv<D, true, true>(q, k, v, g, a.LSE, a.Dws, a.dQ, a.dK, a.dV, s, sl2, stream);
  else
    launch_dkdv<D, false, true>(q, k, v, g, a.LSE, a.Dws, a.dQ, a.dK, a.dV, s, sl2, stream);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_dq_any(const BwdArgs& a, const AttnShape& s, bool precise, hipStream_t stream) {
  const float sl2 = s.scale * kLog2e;
  const u16* q = static_cast<const u16*>(a.Q);
  const u16* k = static_cast<const u16*>(a.K);
  const u16* v = static_cast<const u16*>(a.V);
  const u16* o = static_cast<const u16*>(a.O);
  const u16* g = static_cast<const u16*>(a.dO);
  if (precise)
    launch_dq<D, true>(q, k, v, o, g, a.LSE, a.Dws, a.dQ, s, sl2, stream);
  else
    launch_dq<D, false>(q, k, v, o, g, a.LSE, a.Dws, a.dQ, s, sl2, stream);
  return hipGetLastError();
}

}  // namespace fa
