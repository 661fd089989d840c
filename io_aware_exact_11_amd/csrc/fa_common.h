// Device-side types and helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef unsigned short u16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 32x32x16 bf16 matrix-core product with fp32 accumulation (wave64).
// Operand layout, lane l = 32*g + r (g in {0,1}, r in 0..31):
//   A (32 x 16): lane holds row r, k = 8g .. 8g+7
//   B (16 x 32): lane holds column r, k = 8g .. 8g+7
//   C (32 x 32): element e = 4*i + j (i, j in 0..3) of the lane's 16 is
//                row 8i + 4g + j, column r.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 ld_global16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ bf16x8 ld_lds16(const u16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Round 8 fp32 values to bf16 (round to nearest even) as one MFMA operand.
__device__ __forceinline__ bf16x8 pack_bf16x8(const f32x16& v, int base) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)v[base + e];
  return r;
}

// Split 8 fp32 values into bf16 pairs with x ~ hi + lo: hi = bf16(x),
// lo = bf16(x - hi). Two products over (hi, lo) carry about 16 significant
// bits of x instead of 8.
__device__ __forceinline__ void pack_split_bf16x8(const f32x16& v, int base, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 h = (__bf16)v[base + e];
    hi[e] = h;
    lo[e] = (__bf16)(v[base + e] - (float)h);
  }
}

// Element e (0..7) of a 16-byte chunk of bf16 values, as raw bits.
__device__ __forceinline__ unsigned bf16_bits(const u32x4& v, int e) {
  return (v[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
}

// Swap bits 2 and 3 of an index inside a 16-aligned group. Tiles that are
// stored transposed in LDS use it for their column order, so that the 8
// k-slots one lane feeds to a 32x32x16 product (the C-layout rows
// 8i+4g+j of an earlier product, i in {2h, 2h+1}) are 8 adjacent columns.
__device__ __forceinline__ int swap23(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// Map a linear workgroup id to a tile id so that the tiles of one (b, h)
// run on one XCD, in order: workgroups are dispatched round-robin over the
// 8 XCDs, each with its own L2, and neighbouring tiles of a head share K, V.
__device__ __forceinline__ int xcd_tile(int wg, int total) {
  if ((total & 7) != 0) return wg;
  return (wg & 7) * (total >> 3) + (wg >> 3);
}

}  // namespace fa
