// Dropout keep-mask generation inside the attention kernels.
//
// The mask is never stored: every kernel that needs it (the forward, the
// query-outer dQ kernel and the key-outer dK/dV kernel) regenerates it from
// the generator state ("FlashAttention and GPU Memory", chapter 07 Blocks
// lists dropout among the fused steps; chapter 09 has the backward
// regenerate it instead of saving it).
//
// Generator: Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC 2011). Key = the 64-bit
// seed split into two words; counter = (key index / 4, query index / 4,
// b * H + h, offset). One call covers a 4 x 4 block of (query, key) pairs:
// element (i, j) takes byte j % 4 of output word i % 4 and is kept iff that
// byte >= thresh = round(256 p). Kept weights are scaled by
// 256 / (256 - thresh), the inverse of the exact keep probability.
//
// In the 32x32 matrix-core layouts a lane holds 16 elements of a 32 x 32
// slab: four groups of four consecutive indices along one axis, at a fixed
// index along the other. The four lanes of a quad (lanes 4a .. 4a+3) need
// the same four generator calls, so each lane computes one and a 4 x 4
// transpose across the quad (DPP moves) hands every lane its words.
#pragma once

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

__device__ __forceinline__ u32x4 philox4x32_10(unsigned c0, unsigned c1, unsigned c2, unsigned c3, unsigned k0,
                                               unsigned k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const unsigned long long p0 = (unsigned long long)c0 * 0xD2511F53u;
    const unsigned long long p1 = (unsigned long long)c2 * 0xCD9E8D57u;
    // Three-input XORs, one v_bitop3_b32 each (truth table 0x96).
    const unsigned n0 = __builtin_amdgcn_bitop3_b32((unsigned)(p1 >> 32), c1, k0, 0x96);
    const unsigned n2 = __builtin_amdgcn_bitop3_b32((unsigned)(p0 >> 32), c3, k1, 0x96);
    c1 = (unsigned)p1;
    c3 = (unsigned)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  const u32x4 out = {c0, c1, c2, c3};
  return out;
}

// Value of lane l ^ 1 / l ^ 2 within each quad (quad_perm DPP).
__device__ __forceinline__ unsigned quad_xor1(unsigned v) {
  return (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ unsigned quad_xor2(unsigned v) {
  return (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
}

// Lane m of a quad holds row m of a 4 x 4 word matrix; afterwards it holds
// column m (x[i] = row i's word m). Two exchange stages, across lanes m ^ 2
// and then m ^ 1, each swapping one half of the words.
__device__ __forceinline__ void quad_transpose(unsigned (&x)[4], int m) {
  const bool b1 = (m & 2) != 0, b0 = (m & 1) != 0;
  unsigned r0 = quad_xor2(b1 ? x[0] : x[2]);
  unsigned r1 = quad_xor2(b1 ? x[1] : x[3]);
  const unsigned y0 = b1 ? r0 : x[0], y1 = b1 ? r1 : x[1];
  const unsigned y2 = b1 ? x[2] : r0, y3 = b1 ? x[3] : r1;
  r0 = quad_xor1(b0 ? y0 : y1);
  r1 = quad_xor1(b0 ? y2 : y3);
  x[0] = b0 ? r0 : y0;
  x[1] = b0 ? y1 : r0;
  x[2] = b0 ? r1 : y2;
  x[3] = b0 ? y3 : r1;
}

// Transpose the 4 x 4 byte matrix held in four words (word j, byte k) so
// that word k packs byte k of words 0..3.
__device__ __forceinline__ void byte_transpose4(unsigned (&w)[4]) {
  const unsigned t0 = __builtin_amdgcn_perm(w[1], w[0], 0x06020400u);
  const unsigned t1 = __builtin_amdgcn_perm(w[1], w[0], 0x07030501u);
  const unsigned t2 = __builtin_amdgcn_perm(w[3], w[2], 0x06020400u);
  const unsigned t3 = __builtin_amdgcn_perm(w[3], w[2], 0x07030501u);
  w[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  w[1] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  w[2] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  w[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// Query-per-lane layout (S^T tiles: forward and dQ kernels). The lane's
// query is q (its quad holds queries 4(q/4) .. +3 in lane order); kb is the
// first key of a 32-key slab. On return, byte k of W[i] decides key
// kb + 8i + 4g + k for query q.
__device__ __forceinline__ void drop_words_query_lane(const DropParams& dp, int bh, int q, int kb, int g, int lane,
                                                      unsigned (&W)[4]) {
  const int m = lane & 3;
  const u32x4 x = philox4x32_10((unsigned)((kb >> 2) + 2 * m + g), (unsigned)(q >> 2), (unsigned)bh, dp.offset,
                                dp.k0, dp.k1);
  W[0] = x[0];
  W[1] = x[1];
  W[2] = x[2];
  W[3] = x[3];
  quad_transpose(W, m);
}

// Key-per-lane layout (S tiles: dK/dV kernel). The lane's key is key (its
// quad holds keys 4(key/4) .. +3 in lane order); qs is the first query of a
// 32-query slab. On return, byte j of W[i] decides query qs + 8i + 4g + j
// for this key.
__device__ __forceinline__ void drop_words_key_lane(const DropParams& dp, int bh, int key, int qs, int g, int lane,
                                                    unsigned (&W)[4]) {
  const int k = lane & 3;
  const u32x4 x = philox4x32_10((unsigned)(key >> 2), (unsigned)((qs >> 2) + 2 * k + g), (unsigned)bh, dp.offset,
                                dp.k0, dp.k1);
  W[0] = x[0];
  W[1] = x[1];
  W[2] = x[2];
  W[3] = x[3];
  byte_transpose4(W);
  quad_transpose(W, k);
}

__device__ __forceinline__ bool drop_keep(const unsigned (&W)[4], int e, unsigned thresh) {
  return ((W[e >> 2] >> (8 * (e & 3))) & 0xFFu) >= thresh;
}

}  // namespace fa
