// Device-side types and helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef unsigned short u16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __bf16 __attribute__((ext_vector_type(2))) bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Rescale threshold of the forward kernels, in base-2 units of the scaled
// score: the running maximum only moves (and O, l are only rescaled) when a
// tile's maximum exceeds it by more than this, so unnormalised weights stay
// below 2^8.
constexpr float kRescaleSlack = 8.f;

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

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;

// Raw buffer resource over `bytes` bytes at `base`: loads at offsets past
// the end return 0, so tails need no branches. Word 3 = 0x00020000 selects
// 32-bit raw (untyped) access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 ld_buf16(__amdgpu_buffer_rsrc_t r, unsigned byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16). Within each group of 16
// lanes, lane i receives in slot t the (i % 4)-th 16-bit element of the 8
// bytes addressed by lane 4t + i/4 of its group. When lane j of a group
// addresses row (r0 + j/4), columns (c0 + 4(j%4)) .. +3 of a row-major
// bf16 tile, lane i receives column c0 + i of rows r0 .. r0+3.
__device__ __forceinline__ s16x4 ld_lds_tr(const u16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

__device__ __forceinline__ bf16x8 join_tr(s16x4 lo, s16x4 hi) {
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Maximum of x over the lane pair (l, l ^ 32), returned on both lanes.
__device__ __forceinline__ float pair_max(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

__device__ __forceinline__ f32x16 mfma32_first(bf16x8 a, bf16x8 b) {
  const f32x16 z = {};
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, z, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld_global16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ bf16x8 ld_lds16(const u16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// A 32-bit word as two bf16 values (low half first). Written with memcpy:
// __builtin_bit_cast applied to an element of a vector value was compiled
// as a cast of the vector's first element.
__device__ __forceinline__ bf16x2 as_bf16x2(unsigned x) {
  bf16x2 r;
  __builtin_memcpy(&r, &x, sizeof(r));
  return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt vmcnt(0): wait for every outstanding vector-memory load of the
// wave. Used at the end of a prologue whose loads complete on some control
// paths only: the compiler's wait bookkeeping merges paths, so a load left
// pending on one path would otherwise be waited for inside the main loop,
// behind the loop's own prefetches. (Encoding: vmcnt 0, expcnt 7, lgkmcnt 15.)
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

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

// 16-byte chunk swizzle for unpadded row-major bf16 tiles of width D that
// are read both by rows (one 16-byte chunk per lane, 16 consecutive rows per
// LDS cycle) and transposed (ds_read_b64_tr_b16: 4 consecutive rows x 4
// chunks per 32 lanes). Chunk c of row r is stored at chunk c ^ swz(r); with
// 64 four-byte banks both access patterns then touch distinct banks.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Element offset of (row r, column col) in a swizzled tile; col % 8 is kept.
template <int D>
__device__ __forceinline__ int swz_off(int r, int col) {
  return r * D + ((((col >> 3) ^ swz<D>(r)) << 3) | (col & 7));
}

// Load a ROWS x D bf16 tile (global rows row0.., row stride D) into a
// swizzled LDS tile with direct buffer-to-LDS loads: no registers are
// staged. Each wave instruction moves 1 KB, lane l landing at byte 16 l of
// it; the lane therefore fetches the global chunk that the swizzle places
// there. Rows past the end of the buffer read as zeros (out-of-range lanes
// of a buffer-to-LDS load write zeros). The data is visible to the other
// waves after the next barrier, which waits for these loads.
template <int D, int ROWS, int NW>
__device__ __forceinline__ void tile_to_lds(__amdgpu_buffer_rsrc_t rs, int row0, u16* tile, int w,
                                            int lane) {
  constexpr int INST = ROWS * D * 2 / 1024;
  static_assert(INST % NW == 0, "whole 1 KB blocks per wave");
#pragma unroll
  for (int i = 0; i < INST / NW; ++i) {
    const int blk = w * (INST / NW) + i;
    const int e0 = blk * 512 + lane * 8;
    const int row = e0 / D, pc = (e0 % D) >> 3;
    const unsigned goff = (unsigned)((row0 + row) * D + ((pc ^ swz<D>(row)) << 3)) * 2;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(tile + blk * 512), 16, (int)goff, 0, 0, 0);
  }
}

// Direct-to-LDS copy of ROWS rows of D bf16 into a tile whose rows are
// STRIDE elements apart (padding keeps the row-wise and transposing reads
// free of bank conflicts). Each wave instruction fills 1 KB of LDS, 16
// bytes per lane at consecutive addresses; lane l of block blk covers tile
// byte 1024*blk + 16*l, i.e. row (that offset) / (2*STRIDE) and byte
// (that offset) % (2*STRIDE) of the row, which it fetches from the global
// row. Lanes that land in a row's padding re-read the row's first chunk.
// Rows past the end of the buffer resource read zeros.
template <int D, int STRIDE, int ROWS, int NW>
__device__ __forceinline__ void tile_to_lds_padded(__amdgpu_buffer_rsrc_t rs, int row0, u16* tile, int w,
                                                   int lane) {
  constexpr int BYTES = ROWS * STRIDE * 2;
  static_assert(BYTES % 1024 == 0, "whole 1 KB blocks");
  constexpr int NBLK = BYTES / 1024;
#pragma unroll
  for (int i = 0; i < (NBLK + NW - 1) / NW; ++i) {
    const int blk = w + NW * i;
    if (NBLK % NW == 0 || blk < NBLK) {
      const int off = blk * 1024 + lane * 16;
      const int row = off / (STRIDE * 2), cb = off % (STRIDE * 2);
      const int src = (row0 + row) * D * 2 + (cb < D * 2 ? cb : 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(tile + blk * 512), 16, src, 0, 0, 0);
    }
  }
}

// Tiles read both by rows and transposed. With 64 four-byte banks, a 16-byte
// row read serves 16 consecutive rows per LDS cycle, so those rows must
// start in 16 distinct 4-bank groups; a transposing read (ds_read_b64_tr_b16)
// serves 4 consecutive rows x 4 adjacent chunks per 32 lanes, so those rows
// must start 16 banks apart. No row padding satisfies both. The "xpad"
// layout pads each row to a 16-bank step (S*2 bytes = 64 or 192 mod 256)
// and stores chunk c of row r at chunk c ^ ((r >> 2) & 3): the XOR only
// permutes the four chunks of each 64-byte group, so the transposing read
// keeps its four rows in distinct 16-bank quarters and the row read spreads
// 16 consecutive rows over all 16 groups.
template <int S>
__device__ __forceinline__ constexpr int xpad_off(int row, int chunk) {
  return row * S + 8 * (chunk ^ ((row >> 2) & 3));
}

// Direct-to-LDS copy of ROWS rows of D bf16 into an xpad tile of row stride
// S elements (see xpad_off). Lane l of block blk fills tile byte
// 1024*blk + 16*l: it fetches the global chunk that the XOR places there
// (the map is its own inverse); lanes that land in the padding re-read the
// row's first chunk. Rows past the end of the buffer resource read zeros.
template <int D, int S, int ROWS, int NW>
__device__ __forceinline__ void tile_to_lds_xpad(__amdgpu_buffer_rsrc_t rs, int row0, u16* tile, int w, int lane) {
  static_assert((S * 2) % 256 == 64 || (S * 2) % 256 == 192, "16-bank row step");
  static_assert(S >= D, "row fits");
  constexpr int BYTES = ROWS * S * 2;
  static_assert(BYTES % 1024 == 0, "whole 1 KB blocks");
  constexpr int NBLK = BYTES / 1024;
#pragma unroll
  for (int i = 0; i < (NBLK + NW - 1) / NW; ++i) {
    const int blk = w + NW * i;
    if (NBLK % NW == 0 || blk < NBLK) {
      const int off = blk * 1024 + lane * 16;
      const int row = off / (S * 2), pc = (off % (S * 2)) >> 4;
      const int src = (row0 + row) * D * 2 + (pc < D / 8 ? (pc ^ ((row >> 2) & 3)) * 16 : 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(tile + blk * 512), 16, src, 0, 0, 0);
    }
  }
}

// Direct-to-LDS copy of ROWS rows of 128 bf16 into an unpadded tile that
// is only read transposed (ds_read_b64_tr_b16: 4 consecutive rows x 4
// adjacent chunks per 32 lanes). Chunk c of row r is stored at chunk
// c ^ 4(r & 3), which puts those four rows in distinct 16-bank quarters of
// the 64 four-byte banks. Lane l of block blk fills tile byte 1024*blk +
// 16*l and fetches the global chunk placed there (the map is its own
// inverse). Rows past the end of the buffer resource read zeros.
template <int ROWS, int NW>
__device__ __forceinline__ void tile_to_lds_trxor(__amdgpu_buffer_rsrc_t rs, int row0, u16* tile, int w, int lane) {
  constexpr int D = 128;
  constexpr int INST = ROWS * D * 2 / 1024;
  static_assert(INST % NW == 0, "whole 1 KB blocks per wave");
#pragma unroll
  for (int i = 0; i < INST / NW; ++i) {
    const int blk = w * (INST / NW) + i;
    const int row = blk * 4 + (lane >> 4), pc = lane & 15;
    const int src = (row0 + row) * D * 2 + ((pc ^ (4 * (row & 3))) << 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(tile + blk * 512), 16, src, 0, 0, 0);
  }
}

// Map a linear workgroup id to a tile id so that the tiles of one (b, h)
// run on one XCD, in order: workgroups are dispatched round-robin over the
// 8 XCDs, each with its own L2, and neighbouring tiles of a head share K, V.
__device__ __forceinline__ int xcd_tile(int wg, int total) {
  if ((total & 7) != 0) return wg;
  return (wg & 7) * (total >> 3) + (wg >> 3);
}

}  // namespace fa
