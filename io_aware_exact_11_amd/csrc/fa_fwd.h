// Forward pass of exact attention for gfx950, bf16 in, fp32 accumulation.
//
// One workgroup owns a block of BR query rows of one (b, h) (128, or 256
// with two slabs per wave; in causal grids two blocks, one after the other)
// and streams the keys and values through LDS in tiles of BC = 64 rows,
// double-buffered: the global loads of the next tile are in flight while
// the current one is computed ("FlashAttention and GPU Memory", chapter 07
// Blocks: one block of Q stays on chip while blocks of K and V come in;
// only O and the row statistics are written back).
//
// Each of the 4 waves owns one or two 32-row query slabs. Scores are produced transposed,
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
// elements. Its A operand is V transposed; V tiles stay row-major in LDS and
// are read transposed with ds_read_b64_tr_b16, two reads per operand, with
// the key order chosen to match those slots.
//
// The running maximum moves lazily: only when a tile's maximum exceeds it by
// more than 8 (base 2), which keeps every weight below 2^8 and skips the O
// rescale on almost every tile. Loads go through buffer resources, whose
// hardware bounds check returns zeros past the end of a head.
#pragma once

#include <type_traits>

#include "fa_common.h"
#include "fa_dropout.h"
#include "fa_launch.h"

namespace fa {

// Tile configuration. NW waves per workgroup, each owning QS slabs of 32
// query rows; every K and V operand read from LDS feeds QS matrix-core
// products, so LDS read traffic per flop falls as 1/QS. PIPE runs the
// score products of tile j+1 ahead of the softmax of tile j; OCC is the
// number of waves per SIMD the register budget is cut for. DL (with PIPE)
// moves K and V tiles from global memory straight into LDS with buffer
// loads that bypass the registers, instead of staging them in registers.
template <int D, int NW_, int QS_, bool PIPE_, int OCC_, bool DL_ = false>
struct FwdCfg {
  static constexpr int NW = NW_;
  static constexpr int QS = QS_;
  static constexpr bool PIPE = PIPE_;
  static constexpr int OCC = OCC_;
  static constexpr bool DL = DL_;
  static_assert(!DL || PIPE, "direct loads are implemented for the pipelined loop");
  static constexpr int NT = 64 * NW;            // threads per workgroup
  static constexpr int BR = 32 * NW * QS;       // query rows per workgroup
  static constexpr int BC = 64;                 // keys per tile
  // K tile row stride (elements). The tile is read by rows only (16-byte
  // reads, 16 rows per LDS cycle): a 4-bank step keeps those conflict-free.
  // The d=128 direct-to-LDS tile is unpadded and chunk-swizzled instead
  // (tile_to_lds, swz), so each tile loads 16 KB, four blocks per wave.
  static constexpr bool KSWZ = D == 128 && DL_;
  static constexpr int KSTR = KSWZ ? D : D + 8;
  // V tile row stride: the 4 rows of a transposing read must land in
  // disjoint banks. At d=64 a stride of D+8 places them 36 banks apart (and
  // the smaller tile lets four workgroups share a CU). At d=128 the direct-
  // to-LDS tile is unpadded and XOR-permuted instead (tile_to_lds_trxor):
  // no padding to load; the register-staged d=128 tile keeps a 16-bank step.
  static constexpr bool VXOR = D == 128 && DL_;
  static constexpr int VSTR = D == 64 ? D + 8 : (VXOR ? D : D + 32);
  static constexpr int CH = BC * D / 8 / NT;    // 16-byte chunks per thread per tile
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(CH * NT * 8 == BC * D, "tile split");
};

// Measured choices. d=128: one slab per wave, pipelined, direct-to-LDS
// tile loads, two waves per SIMD (two slabs need more than the 256
// registers of two waves per SIMD, and one wave per SIMD measured slower;
// register-staged loads measured 9% slower). d=64 causal: one slab, unpipelined, four
// waves per SIMD: causal workgroups are short, and more of them in flight
// hide their start-up latency better than the pipeline does. d=64
// non-causal: two slabs per wave, unpipelined, two waves per SIMD, which
// halves the LDS operand reads per product.
using FwdCfg128 = FwdCfg<128, 4, 1, true, 2, true>;
using FwdCfg64Causal = FwdCfg<64, 4, 1, false, 4>;
using FwdCfg64Full = FwdCfg<64, 4, 2, false, 2>;


// Block-sparse attention: blocks of kSparseBlock queries by kSparseBlock keys,
// at most kSparseMaxTiles key tiles (N <= 65536) per row of blocks.
constexpr int kSparseBlock = 128;
constexpr int kSparseMaxTiles = 1024;

// DROP: fused dropout on the normalised weights (see fa_dropout.h); the row
// sums and the saved LSE are those of the undropped scores.
// SPARSE: block-sparse attention ("FlashAttention and GPU Memory", chapters
// 10 and 12 name the approximate block-sparse variant). bmask holds one byte
// per (query block, key block) of 128 x 128, row-major, bmask_stride bytes
// apart for consecutive (b, h); only key tiles whose block is on are loaded
// and computed, on top of the causal and padding masks.
// Whether causal query blocks run in pairs (see fwd_bf16_kernel); not for
// the dropout kernel at four waves per SIMD, whose 128 registers do not
// hold the pairing's bookkeeping without spilling.
template <class C, bool DROP>
constexpr bool fwd_pairs() { return !(DROP && C::OCC >= 4); }

template <int D, class C, bool DROP = false, bool SPARSE = false>
__global__ __launch_bounds__(C::NT, C::OCC * 4 / C::NW) void fwd_bf16_kernel(
    const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ V,
    u16* __restrict__ O, float* __restrict__ LSE, int H, int N, float sl2, int causal,
    const int32_t* __restrict__ kv_len, int nqb, int total, DropParams dpar,
    const uint8_t* __restrict__ bmask, long long bmask_stride) {
  constexpr int BC = C::BC, NT = C::NT, QS = C::QS;
  constexpr bool DL = C::DL;
  // Register-staged tiles: two buffers per tensor, indexed at run time.
  __shared__ __attribute__((aligned(16))) u16 Ks[2][DL ? 8 : BC * C::KSTR];
  __shared__ __attribute__((aligned(16))) u16 Vs[2][DL ? 8 : BC * C::VSTR];
  // Direct-to-LDS tiles: the two buffers of each tensor are separate arrays
  // and the loop names them at compile time, so the compiler can tell that
  // the loads in flight into one buffer do not overlap the reads of the
  // other and does not make those reads wait for them.
  __shared__ __attribute__((aligned(16))) u16 Kd0[DL ? BC * C::KSTR : 8];
  __shared__ __attribute__((aligned(16))) u16 Kd1[DL ? BC * C::KSTR : 8];
  __shared__ __attribute__((aligned(16))) u16 Vd0[DL ? BC * C::VSTR : 8];
  __shared__ __attribute__((aligned(16))) u16 Vd1[DL ? BC * C::VSTR : 8];

  // Causal grids pair query block i with block nqb - 1 - i in one
  // workgroup, run one after the other (the longer first): every workgroup
  // then does the same amount of work, so no long block is left to start
  // near the end of the grid, and both blocks read the same head's K and V.
  // Unpaired causal grids run the longest blocks of each head first.
  constexpr bool PAIR = fwd_pairs<C, DROP>();
  const int per_head = (PAIR && causal) ? (nqb + 1) / 2 : nqb;
  const int tile = xcd_tile(blockIdx.x, total);
  const int pi = tile % per_head;
  const int bh = tile / per_head;
  const int npass = (PAIR && causal && nqb - 1 - pi != pi) ? 2 : 1;
  const int b = bh / H;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, r = lane & 31, g = lane >> 5;
  const size_t head = (size_t)bh * N * D;
  const unsigned head_bytes = (unsigned)N * D * 2;
  const auto rQ = make_rsrc(Q + head, head_bytes);
  const auto rK = make_rsrc(K + head, head_bytes);
  const auto rV = make_rsrc(V + head, head_bytes);

  int kv_lim = N;
  if (kv_len) {
    const int L = kv_len[b];
    kv_lim = L < 0 ? 0 : (L > N ? N : L);
  }

  auto block = [&](const int qb) {
    const int q0 = qb * C::BR;
    int kv_end = kv_lim;
    if (causal) kv_end = min(kv_end, q0 + C::BR);
    // Block-sparse: the ascending list of key tiles (64 keys, half a block)
    // whose block is on for this workgroup's 128 query rows, built by wave 0
    // with a ballot prefix count; the loop runs over the list and its tile t
    // starts at key tkb(t).
    static_assert(!SPARSE || (C::BR == kSparseBlock && BC * 2 == kSparseBlock), "sparse tiles");
    __shared__ unsigned short tlist[SPARSE ? kSparseMaxTiles : 1];
    __shared__ int tlist_n;
    auto sparse_list = [&](int nt_all) {
      if (tid < 64) {
        const uint8_t* brow = bmask + (size_t)bh * bmask_stride + (size_t)qb * ((N + kSparseBlock - 1) / kSparseBlock);
        // Every mask byte the list needs is requested before the first is
        // used, so the row costs one memory latency rather than one per 64
        // tiles. Indices are clamped into the row (a row has at least one
        // block); tiles past nt_all are off.
        constexpr int MAXIT = kSparseMaxTiles / 64;
        const int tlast = nt_all > 0 ? nt_all - 1 : 0;
        unsigned char mb[MAXIT];
  #pragma unroll
        for (int i = 0; i < MAXIT; ++i) mb[i] = brow[min(64 * i + tid, tlast) >> 1];
        int cnt = 0;
  #pragma unroll
        for (int i = 0; i < MAXIT; ++i) {
          const int t = 64 * i + tid;
          const bool on = t < nt_all && mb[i] != 0;
          const unsigned long long bal = __builtin_amdgcn_ballot_w64(on);
          const int pos = cnt + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32),
                                                               __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u));
          if (on) tlist[pos] = (unsigned short)t;
          cnt += __popcll(bal);
        }
        if (tid == 0) tlist_n = cnt;
      }
      __syncthreads();
      return tlist_n;
    };
    const int nt = SPARSE ? sparse_list((kv_end + BC - 1) / BC) : (kv_end + BC - 1) / BC;
    // Start of loop tile t + k given the start kb of tile t (the dense loop
    // keeps its own arithmetic).
    auto tnext = [&](int t, int kb, int k) { return SPARSE ? (int)tlist[t + k] * BC : kb + k * BC; };

    // Slab s of wave w holds query rows q0 + 32*(QS*w + s) + 0..31; this lane
    // owns row r of each slab.
    const int wave_q_first = q0 + 32 * QS * w;
    const int wave_q_last = wave_q_first + 32 * QS - 1;

    // Q fragments: B operands of S^T = K Q^T (column = query, k = d).
    bf16x8 qf[QS][D / 16];
  #pragma unroll
    for (int s = 0; s < QS; ++s)
  #pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
        qf[s][kk] = as_bf16x8(ld_buf16(rQ, (unsigned)((wave_q_first + 32 * s + r) * D + 16 * kk + 8 * g) * 2));

    f32x16 o[QS][D / 32];
    float m_run[QS], l_run[QS];
  #pragma unroll
    for (int s = 0; s < QS; ++s) {
  #pragma unroll
      for (int t = 0; t < D / 32; ++t)
  #pragma unroll
        for (int e = 0; e < 16; ++e) o[s][t][e] = 0.f;
      m_run[s] = -INFINITY;
      l_run[s] = 0.f;
    }

    // Tile loads: chunk c = tid + NT*rr is row c / (D/8), 16-byte column c % (D/8).
    u32x4 kreg[C::CH], vreg[C::CH];
    auto tile_off = [&](int kb, int rr) {
      const int c = tid + NT * rr;
      return (unsigned)((kb + c / (D / 8)) * D + (c % (D / 8)) * 8) * 2;
    };
    auto load_k = [&](int kb) {
  #pragma unroll
      for (int rr = 0; rr < C::CH; ++rr) kreg[rr] = ld_buf16(rK, tile_off(kb, rr));
    };
    auto load_v = [&](int kb) {
  #pragma unroll
      for (int rr = 0; rr < C::CH; ++rr) vreg[rr] = ld_buf16(rV, tile_off(kb, rr));
    };
    auto store_k = [&](int buf) {
  #pragma unroll
      for (int rr = 0; rr < C::CH; ++rr) {
        const int c = tid + NT * rr;
        *reinterpret_cast<u32x4*>(&Ks[buf][(c / (D / 8)) * C::KSTR + (c % (D / 8)) * 8]) = kreg[rr];
      }
    };
    auto store_v = [&](int buf) {
  #pragma unroll
      for (int rr = 0; rr < C::CH; ++rr) {
        const int c = tid + NT * rr;
        *reinterpret_cast<u32x4*>(&Vs[buf][(c / (D / 8)) * C::VSTR + (c % (D / 8)) * 8]) = vreg[rr];
      }
    };
    // S^T tiles from K tile Kt for every slab: rows = keys
    // 32*mt + (8i + 4g + j), column = the slab's query. Each K read serves
    // all QS slabs.
    // This lane's K read offsets: chunk 2kk + g of row 32mt + r (the swizzle
    // depends on r only, since 32mt leaves bits 0..3 of the row unchanged).
    int k_off[D / 16];
  #pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      k_off[kk] = C::KSWZ ? swz_off<D>(r, 16 * kk + 8 * g) : r * C::KSTR + 16 * kk + 8 * g;
    auto qk = [&](const u16* Kt, f32x16 (*sv)[BC / 32]) {
  #pragma unroll
      for (int mt = 0; mt < BC / 32; ++mt) {
        const u16* kp = Kt + 32 * mt * C::KSTR;
        const bf16x8 a0 = ld_lds16(kp + k_off[0]);
  #pragma unroll
        for (int s = 0; s < QS; ++s) sv[s][mt] = mfma32_first(a0, qf[s][0]);
  #pragma unroll
        for (int kk = 1; kk < D / 16; ++kk) {
          const bf16x8 a = ld_lds16(kp + k_off[kk]);
  #pragma unroll
          for (int s = 0; s < QS; ++s) sv[s][mt] = mfma32(a, qf[s][kk], sv[s][mt]);
        }
      }
    };
    // Per-lane offsets of the transposing V reads (see ld_lds_tr): row part
    // 4g + (lane % 16) / 4, column part 16 * ((lane / 16) % 2) + 4 * (lane % 4).
    // In the XOR-permuted tile the 32-column group t of this lane's rows sits
    // at group t ^ q, q = row % 4 = (lane / 4) % 4, the same for all its rows.
    const int v_tr_off = (4 * g + ((lane & 15) >> 2)) * C::VSTR + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    int v_grp[D / 32];
  #pragma unroll
    for (int t = 0; t < D / 32; ++t) v_grp[t] = C::VXOR ? 32 * (t ^ ((lane >> 2) & 3)) : 32 * t;
    // Causal waves compute only the tiles that reach their rows (a prefix).
    // Causal block-sparse: the listed tiles that reach this wave's rows (a
    // prefix of the ascending list).
    auto sparse_prefix = [&]() {
      int c = 0;
      for (int i0 = 0; i0 < nt; i0 += 64) {
        const bool in = i0 + lane < nt && (int)tlist[i0 + lane] <= wave_q_last / BC;
        c += __popcll(__builtin_amdgcn_ballot_w64(in));
      }
      return c;
    };
    const int nt_w = causal ? (SPARSE ? sparse_prefix() : min(nt, wave_q_last / BC + 1)) : nt;

    // Mask, running maximum and lazy rescale of one tile's scores.
    auto mask_max = [&](int kb, f32x16 (*sv)[BC / 32]) {
  #pragma unroll
      for (int s = 0; s < QS; ++s) {
        const int slab_first = wave_q_first + 32 * s;
        const int q = slab_first + r;
        const bool need_mask = (kb + BC > kv_lim) || (causal && kb + BC - 1 > slab_first);
        if (need_mask) {
          // Element e of score tile mt is key kb + 4g + c with the constant
          // c = 32mt + 8(e/4) + e%4; the key is hidden iff it is >= kv_lim or
          // (causal) > q, i.e. iff c > lim: one compare and select per score.
          const int lim = min(kv_lim - 1, causal ? q : kv_lim - 1) - (kb + 4 * g);
  #pragma unroll
          for (int mt = 0; mt < BC / 32; ++mt)
  #pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int c = 32 * mt + 8 * (e >> 2) + (e & 3);
              sv[s][mt][e] = c > lim ? -INFINITY : sv[s][mt][e];
            }
        }
        float mx = sv[s][0][0];
  #pragma unroll
        for (int mt = 0; mt < BC / 32; ++mt)
  #pragma unroll
          for (int e = (mt == 0 ? 1 : 0); e < 16; ++e) mx = fmaxf(mx, sv[s][mt][e]);
        const float tmax = pair_max(mx) * sl2;
        // Move the reference maximum only when some row of the slab outgrows it.
        if (__builtin_amdgcn_ballot_w64(tmax > m_run[s] + kRescaleSlack) != 0) {
          const float m_new = fmaxf(m_run[s], tmax);
          const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run[s] - m_new);
          l_run[s] *= alpha;
  #pragma unroll
          for (int t = 0; t < D / 32; ++t)
  #pragma unroll
            for (int e = 0; e < 16; ++e) o[s][t][e] *= alpha;
          m_run[s] = m_new;
        }
      }
    };
    // P~ = 2^(s*scale*log2e - m), row sums, then O^T += V^T P^T from V buffer
    // `buf`: A = V^T rows d = 32t + r, k-slots = keys of chunk c in the order
    // of the score registers (16c + 8h + 4g + 0..3 for slots 4h..4h+3); each
    // V read serves all QS slabs.
    auto exp_pv = [&](const u16* Vt, f32x16 (*sv)[BC / 32], int kb) {
      bf16x8 pb[QS][BC / 16];
  #pragma unroll
      for (int s = 0; s < QS; ++s) {
        const float m_use = (m_run[s] == -INFINITY) ? 0.f : m_run[s];
        float rs = 0.f;
  #pragma unroll
        for (int mt = 0; mt < BC / 32; ++mt)
  #pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float p = fast_exp2(sv[s][mt][e] * sl2 - m_use);
            sv[s][mt][e] = p;
            rs += p;
          }
        l_run[s] += rs;
        if constexpr (DROP) {
          // Dropped weights leave the P V product; l keeps them.
  #pragma unroll
          for (int mt = 0; mt < BC / 32; ++mt) {
            unsigned W[4];
            drop_words_query_lane(dpar, bh, wave_q_first + 32 * s + r, kb + 32 * mt, g, lane, W);
  #pragma unroll
            for (int e = 0; e < 16; ++e)
              if (!drop_keep(W, e, dpar.thresh)) sv[s][mt][e] = 0.f;
          }
        }
  #pragma unroll
        for (int c = 0; c < BC / 16; ++c) pb[s][c] = pack_bf16x8(sv[s][c >> 1], 8 * (c & 1));
      }
      const u16* vb = Vt + v_tr_off;
  #pragma unroll
      for (int t = 0; t < D / 32; ++t)
  #pragma unroll
        for (int c = 0; c < BC / 16; ++c) {
          const u16* vp = vb + (16 * c) * C::VSTR + v_grp[t];
          const bf16x8 a = join_tr(ld_lds_tr(vp), ld_lds_tr(vp + 8 * C::VSTR));
  #pragma unroll
          for (int s = 0; s < QS; ++s) o[s][t] = mfma32(a, pb[s][c], o[s][t]);
        }
    };

    f32x16 s_cur[QS][BC / 32];
    // Direct-to-LDS K and V tile loads in the layouts the reads above expect.
    auto load_k_dl = [&](int kb, u16* Kt) {
      if constexpr (C::KSWZ)
        tile_to_lds<D, BC, C::NW>(rK, kb, Kt, w, lane);
      else
        tile_to_lds_padded<D, C::KSTR, BC, C::NW>(rK, kb, Kt, w, lane);
    };
    auto load_v_dl = [&](int kb, u16* Vt) {
      if constexpr (C::VXOR)
        tile_to_lds_trxor<BC, C::NW>(rV, kb, Vt, w, lane);
      else
        tile_to_lds_padded<D, C::VSTR, BC, C::NW>(rV, kb, Vt, w, lane);
    };
    if constexpr (DL) {
      // K_j sits in Kd{j%2}, V_j in Vd{j%2}; K runs one tile ahead of V as
      // below. Each tile's loads go straight to LDS: K_{j+2} into the buffer
      // K_j left, V_{j+1} into the one V_{j-1} left. Two tiles per trip so
      // that the buffer names are compile-time constants.
      if (nt > 0) {
        load_k_dl(tnext(0, 0, 0), Kd0);
        load_v_dl(tnext(0, 0, 0), Vd0);
      }
      if (nt > 1) load_k_dl(tnext(0, 0, 1), Kd1);
      wait_vmem_all();
      __syncthreads();
      if (nt_w > 0) qk(Kd0, s_cur);
      __syncthreads();
      f32x16 s_alt[QS][BC / 32];
      auto tile = [&](auto odd, int it, f32x16 (*cur)[BC / 32], f32x16 (*nxt)[BC / 32]) {
        constexpr bool P = decltype(odd)::value;
        const int kb = tnext(it, it * BC, 0);
        if (it + 2 < nt) load_k_dl(tnext(it, kb, 2), P ? Kd1 : Kd0);
        if (it + 1 < nt) load_v_dl(tnext(it, kb, 1), P ? Vd0 : Vd1);
        if (it < nt_w) {
          mask_max(kb, cur);
          qk(P ? Kd0 : Kd1, nxt);
          exp_pv(P ? Vd1 : Vd0, cur, kb);
        }
        // Each wave waits for its own loads before the barrier publishes them.
        wait_vmem_all();
        __syncthreads();
      };
      for (int it = 0; it < nt; it += 2) {
        tile(std::integral_constant<bool, false>{}, it, s_cur, s_alt);
        if (it + 1 < nt) tile(std::integral_constant<bool, true>{}, it + 1, s_alt, s_cur);
      }
    } else if constexpr (C::PIPE) {
      // K runs one tile ahead of V: while tile j's softmax is on the vector
      // ALUs the wave already issues tile j+1's S^T products. K_j sits in
      // Ks[j % 2], V_j in Vs[j % 2]; one barrier per tile.
      if (nt > 0) {
        load_k(tnext(0, 0, 0));
        load_v(tnext(0, 0, 0));
        store_k(0);
        store_v(0);
      }
      if (nt > 1) {
        load_k(tnext(0, 0, 1));
        store_k(1);
      }
      __syncthreads();
      if (nt_w > 0) qk(Ks[0], s_cur);
      // K_0's buffer is refilled with K_2 during the first tile: every wave
      // must have taken its scores from it first.
      __syncthreads();
      wait_vmem_all();

      for (int it = 0; it < nt; ++it) {
        const int kb = tnext(it, it * BC, 0);
        const bool more_k = it + 2 < nt, more_v = it + 1 < nt;
        if (more_k) load_k(tnext(it, kb, 2));
        if (more_v) load_v(tnext(it, kb, 1));
        if (it < nt_w) {
          mask_max(kb, s_cur);
          // Next tile's scores (on the last tile this reads a stale buffer and
          // the result is dropped), independent of the softmax below.
          f32x16 s_next[QS][BC / 32];
          qk(Ks[(it + 1) & 1], s_next);
          exp_pv(Vs[it & 1], s_cur, kb);
  #pragma unroll
          for (int s = 0; s < QS; ++s)
  #pragma unroll
            for (int mt = 0; mt < BC / 32; ++mt) s_cur[s][mt] = s_next[s][mt];
        }
        if (more_k) store_k(it & 1);
        if (more_v) store_v((it + 1) & 1);
        __syncthreads();
      }
    } else {
      // K_j and V_j both sit in buffer j % 2; tile j+1 is loaded into
      // registers while tile j is computed and stored after it.
      if (nt > 0) {
        load_k(tnext(0, 0, 0));
        load_v(tnext(0, 0, 0));
        store_k(0);
        store_v(0);
      }
      __syncthreads();
      wait_vmem_all();
      for (int it = 0; it < nt; ++it) {
        const int kb = tnext(it, it * BC, 0);
        const bool more = it + 1 < nt;
        if (more) {
          load_k(tnext(it, kb, 1));
          load_v(tnext(it, kb, 1));
        }
        if (it < nt_w) {
          qk(Ks[it & 1], s_cur);
          mask_max(kb, s_cur);
          exp_pv(Vs[it & 1], s_cur, kb);
        }
        if (more) {
          store_k((it + 1) & 1);
          store_v((it + 1) & 1);
        }
        __syncthreads();
      }
    }

  #pragma unroll
    for (int s = 0; s < QS; ++s) {
      const int q = wave_q_first + 32 * s + r;
      const float l_tot = pair_sum(l_run[s]);
      const float inv = l_tot > 0.f ? (DROP ? dpar.keep_scale : 1.f) / l_tot : 0.f;
      if (q < N) {
        u16* orow = O + head + (size_t)q * D;
  #pragma unroll
        for (int t = 0; t < D / 32; ++t)
  #pragma unroll
          for (int i = 0; i < 4; ++i) {
            u32x2 p;
            __bf16 h0 = (__bf16)(o[s][t][4 * i + 0] * inv), h1 = (__bf16)(o[s][t][4 * i + 1] * inv);
            __bf16 h2 = (__bf16)(o[s][t][4 * i + 2] * inv), h3 = (__bf16)(o[s][t][4 * i + 3] * inv);
            p[0] = (unsigned)__builtin_bit_cast(u16, h0) | ((unsigned)__builtin_bit_cast(u16, h1) << 16);
            p[1] = (unsigned)__builtin_bit_cast(u16, h2) | ((unsigned)__builtin_bit_cast(u16, h3) << 16);
            *reinterpret_cast<u32x2*>(orow + 32 * t + 8 * i + 4 * g) = p;
          }
        if (g == 0) LSE[(size_t)bh * N + q] = l_tot > 0.f ? (m_run[s] + __log2f(l_tot)) * kLn2 : -INFINITY;
      }
    }
  };
  block(causal ? nqb - 1 - pi : pi);
  if (npass == 2) {
    // The first block's waves are past their last barrier (no LDS reads of
    // it remain); the block-sparse tile list is rebuilt.
    __syncthreads();
    block(pi);
  }
}

template <int D, class C, bool DROP = false, bool SPARSE = false>
static hipError_t launch_fwd_d(const void* Q, const void* K, const void* V, void* O, float* LSE,
                               const AttnShape& s, hipStream_t stream, DropParams dp = {},
                               const uint8_t* bmask = nullptr, long long bmask_stride = 0) {
  const int nqb = (s.N + C::BR - 1) / C::BR;
  const int total = s.B * s.H * ((fwd_pairs<C, DROP>() && s.causal) ? (nqb + 1) / 2 : nqb);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, C, DROP, SPARSE>), dim3(total), dim3(C::NT), 0, stream,
                     static_cast<const u16*>(Q), static_cast<const u16*>(K),
                     static_cast<const u16*>(V), static_cast<u16*>(O), LSE, s.H, s.N,
                     s.scale * kLog2e, s.causal, s.kv_len, nqb, total, dp, bmask, bmask_stride);
  return hipGetLastError();
}

}  // namespace fa
