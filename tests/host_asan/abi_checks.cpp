// Host-side checks of the C entry points, built with the address and
// undefined-behaviour sanitizers against the launcher stand-ins of
// launch_stub.cpp: every argument check in flash_attn_api.cpp runs (sizes
// near the int32 element limit, the int64 span arithmetic of block-sparse
// masks, pointer ranges at the top of the address space, overlaps), and a
// call with valid arguments reaches its launcher stand-in. No GPU is used;
// the pointers are fake device addresses that are never dereferenced.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "flash_attn.h"

namespace fa {
extern int g_launches;
}

static int failures = 0;
static int checks = 0;

#define EXPECT(call, want)                                                                 \
  do {                                                                                     \
    ++checks;                                                                              \
    const int got_ = (call);                                                               \
    if (got_ != (want)) {                                                                  \
      std::printf("FAIL line %d: %s -> %d, want %d\n", __LINE__, #call, got_, (int)(want)); \
      ++failures;                                                                          \
    }                                                                                      \
  } while (0)

// Fake 16-byte-aligned device addresses, 64 GiB apart (no valid tensor here spans more).
static void* at(int i) { return reinterpret_cast<void*>(uintptr_t(1) << 40 | uintptr_t(i) << 36); }
static float* fat(int i) { return static_cast<float*>(at(i)); }
static void* top(size_t below) { return reinterpret_cast<void*>(std::numeric_limits<uintptr_t>::max() - below + 1); }

static int fwd(int B, int H, int N, int d, float scale = 0.125f, int causal = 0, void* q = at(0), void* o = at(3)) {
  return flash_attn_fwd(q, at(1), at(2), o, fat(4), B, H, N, d, scale, causal, nullptr, nullptr);
}

static int bwd(int B, int H, int N, int d, unsigned flags = 0, size_t ws = size_t(-1), void* dq = at(6)) {
  const size_t need = flash_attn_bwd_workspace_bytes(B, H, N, d, flags);
  return flash_attn_bwd(at(0), at(1), at(2), at(3), at(4), fat(5), static_cast<float*>(dq), fat(7), fat(8), at(9),
                        ws == size_t(-1) ? need : ws, B, H, N, d, 0.125f, 0, nullptr, flags, nullptr);
}

int main() {
  const float nan = std::numeric_limits<float>::quiet_NaN();
  const float inf = std::numeric_limits<float>::infinity();

  // forward: valid calls reach the launcher
  int before = fa::g_launches;
  EXPECT(fwd(1, 2, 300, 64), FA_OK);
  EXPECT(fwd(2, 3, 1, 128, 0.5f, 1), FA_OK);
  EXPECT(fa::g_launches - before, 2);
  // shape, scale and flag checks
  EXPECT(fwd(0, 1, 16, 64), FA_ERR_INVALID_ARG);
  EXPECT(fwd(1, -1, 16, 64), FA_ERR_INVALID_ARG);
  EXPECT(fwd(1, 1, 0, 64), FA_ERR_INVALID_ARG);
  EXPECT(fwd(1, 1, 16, 96), FA_ERR_UNSUPPORTED);
  EXPECT(fwd(1, 1, 16, 64, nan), FA_ERR_INVALID_ARG);
  EXPECT(fwd(1, 1, 16, 64, inf), FA_ERR_INVALID_ARG);
  EXPECT(fwd(1, 1, 16, 64, -0.0f), FA_ERR_INVALID_ARG);
  EXPECT(fwd(1, 1, 16, 64, 0.125f, 2), FA_ERR_INVALID_ARG);
  // B*H*N*d one element past the int32 index range, and products that overflow int
  EXPECT(fwd(1, 1, 16777216, 128), FA_ERR_UNSUPPORTED);
  EXPECT(fwd(1, 1, 16777215, 128), FA_OK);
  EXPECT(fwd(65536, 65536, 65536, 128), FA_ERR_UNSUPPORTED);
  EXPECT(fwd(std::numeric_limits<int>::max(), std::numeric_limits<int>::max(), std::numeric_limits<int>::max(), 64),
         FA_ERR_UNSUPPORTED);
  // pointers: NULL, misaligned, aliasing, and a range that runs past the top of the address space
  EXPECT(fwd(1, 1, 16, 64, 0.125f, 0, nullptr), FA_ERR_INVALID_ARG);
  EXPECT(fwd(1, 1, 16, 64, 0.125f, 0, static_cast<char*>(at(0)) + 8), FA_ERR_INVALID_ARG);
  EXPECT(fwd(1, 1, 16, 64, 0.125f, 0, at(0), at(0)), FA_ERR_INVALID_ARG);
  EXPECT(fwd(1, 1, 16, 64, 0.125f, 0, at(0), static_cast<char*>(at(0)) + 1024), FA_ERR_INVALID_ARG);
  EXPECT(fwd(1, 1, 16, 64, 0.125f, 0, at(0), static_cast<char*>(at(0)) + 2048), FA_OK);  // O right after Q
  EXPECT(fwd(1, 1, 16, 64, 0.125f, 0, top(256)), FA_ERR_INVALID_ARG);
  EXPECT(fwd(1, 1, 16, 64, 0.125f, 0, at(0), top(1024)), FA_ERR_INVALID_ARG);
  EXPECT(flash_attn_fwd_f32(fat(0), fat(1), fat(2), fat(3), fat(4), 1, 1, 128, 64, 0.125f, 0, nullptr, nullptr),
         FA_OK);

  // backward and its workspace
  EXPECT(bwd(2, 4, 1000, 128), FA_OK);
  EXPECT(bwd(2, 4, 1000, 128, 1u | 2u), FA_OK);
  EXPECT(bwd(2, 4, 1000, 128, 1u << 3), FA_ERR_INVALID_ARG);
  EXPECT(bwd(2, 4, 1000, 128, 0, 16), FA_ERR_INVALID_ARG);
  EXPECT(bwd(1, 1, 16, 64, 0, size_t(-1), at(0)), FA_ERR_INVALID_ARG);
  EXPECT((int)flash_attn_bwd_workspace_bytes(0, 1, 1, 64, 0), 0);
  EXPECT((int)(flash_attn_bwd_workspace_bytes(1, 1, 1, 128, 0) % 256), 0);
  EXPECT(flash_attn_bwd_f32(fat(0), fat(1), fat(2), fat(3), fat(4), fat(5), fat(6), fat(7), fat(8), at(9), 1 << 20,
                            1, 1, 128, 64, 0.125f, 0, nullptr, 1u, nullptr),
         FA_ERR_INVALID_ARG);
  // allocation-free backward: the scratch limit and the usual checks
  EXPECT(flash_attn_bwd_noalloc(at(0), at(1), at(2), at(3), at(4), fat(5), fat(6), fat(7), fat(8), 8, 32, 8192, 64,
                                0.125f, 0, nullptr, 0, nullptr),
         FA_OK);
  EXPECT(flash_attn_bwd_noalloc(at(0), at(1), at(2), at(3), at(4), fat(5), fat(6), fat(7), fat(8), 1, 1, 4194305, 64,
                                0.125f, 0, nullptr, 0, nullptr),
         FA_ERR_SCRATCH_LIMIT);
  EXPECT(flash_attn_bwd_noalloc(at(0), at(1), at(2), at(3), at(4), fat(5), fat(0), fat(7), fat(8), 1, 1, 16, 64,
                                0.125f, 0, nullptr, 0, nullptr),
         FA_ERR_INVALID_ARG);

  // decoding
  const size_t dws = flash_attn_decode_workspace_bytes(8, 32, 1, 32768, 128);
  EXPECT(flash_attn_decode_fwd(at(0), at(1), at(2), at(3), fat(4), at(5), dws, 8, 32, 1, 32768, 128, 0.088f, 0,
                               nullptr, nullptr),
         FA_OK);
  EXPECT(flash_attn_decode_fwd(at(0), at(1), at(2), at(3), fat(4), at(5), dws - 1, 8, 32, 1, 32768, 128, 0.088f, 0,
                               nullptr, nullptr),
         FA_ERR_INVALID_ARG);
  EXPECT(flash_attn_decode_fwd(at(0), at(1), at(2), at(3), fat(4), at(5), dws, 8, 32, 9, 32768, 128, 0.088f, 0,
                               nullptr, nullptr),
         FA_ERR_UNSUPPORTED);
  EXPECT(flash_attn_decode_fwd(at(0), at(1), at(2), at(3), fat(4), at(5), dws, 1, 1, 5, 4, 64, 0.125f, 1, nullptr,
                               nullptr),
         FA_ERR_INVALID_ARG);
  EXPECT((int)flash_attn_decode_workspace_bytes(1, 1, 0, 16, 64), 0);

  // dropout: the probability bound (round(256 p) < 256) and the mask call's own sizes
  EXPECT(flash_attn_fwd_dropout(at(0), at(1), at(2), at(3), fat(4), 1, 1, 64, 64, 0.125f, 0, nullptr, 0.998f, 7, 0,
                                nullptr),
         FA_OK);
  EXPECT(flash_attn_fwd_dropout(at(0), at(1), at(2), at(3), fat(4), 1, 1, 64, 64, 0.125f, 0, nullptr, 0.999f, 7, 0,
                                nullptr),
         FA_ERR_INVALID_ARG);
  EXPECT(flash_attn_fwd_dropout(at(0), at(1), at(2), at(3), fat(4), 1, 1, 64, 64, 0.125f, 0, nullptr, nan, 7, 0,
                                nullptr),
         FA_ERR_INVALID_ARG);
  EXPECT(flash_attn_bwd_dropout(at(0), at(1), at(2), at(3), at(4), fat(5), fat(6), fat(7), fat(8), at(9), 1 << 20, 1,
                                1, 64, 64, 0.125f, 0, nullptr, 0.1f, 7, 0, 2u, nullptr),
         FA_ERR_INVALID_ARG);
  EXPECT(flash_attn_dropout_mask(static_cast<uint8_t*>(at(0)), 65536, 65536, 4, 4, 0.1f, 7, 0, nullptr),
         FA_ERR_UNSUPPORTED);
  EXPECT(flash_attn_dropout_mask(static_cast<uint8_t*>(at(0)), 2, 3, 5, 7, 0.1f, 7, 0, nullptr), FA_OK);

  // block-sparse: mask span arithmetic in int64, overflow of (heads - 1) * stride, overlap with outputs
  const uint8_t* mask = static_cast<const uint8_t*>(at(10));
  EXPECT(flash_attn_fwd_block_sparse(at(0), at(1), at(2), at(3), fat(4), 1, 16, 65536, 128, 0.088f, 0, nullptr, mask,
                                     0, nullptr),
         FA_OK);
  EXPECT(flash_attn_fwd_block_sparse(at(0), at(1), at(2), at(3), fat(4), 1, 16, 65537, 128, 0.088f, 0, nullptr, mask,
                                     0, nullptr),
         FA_ERR_UNSUPPORTED);
  EXPECT(flash_attn_fwd_block_sparse(at(0), at(1), at(2), at(3), fat(4), 4, 16, 4096, 64, 0.125f, 0, nullptr, mask,
                                     std::numeric_limits<int64_t>::max(), nullptr),
         FA_ERR_INVALID_ARG);
  EXPECT(flash_attn_fwd_block_sparse(at(0), at(1), at(2), at(3), fat(4), 4, 16, 4096, 64, 0.125f, 0, nullptr, mask,
                                     int64_t(1) << 30, nullptr),
         FA_OK);
  // the same stride from below O: (heads - 1) * stride reaches into O
  EXPECT(flash_attn_fwd_block_sparse(at(0), at(1), at(2), at(3), fat(4), 4, 16, 4096, 64, 0.125f, 0, nullptr,
                                     static_cast<const uint8_t*>(at(2)), int64_t(1) << 31, nullptr),
         FA_ERR_INVALID_ARG);
  EXPECT(flash_attn_fwd_block_sparse(at(0), at(1), at(2), at(3), fat(4), 1, 1, 4096, 64, 0.125f, 0, nullptr, mask,
                                     -1, nullptr),
         FA_ERR_INVALID_ARG);
  EXPECT(flash_attn_fwd_block_sparse(at(0), at(1), at(2), at(3), fat(4), 1, 1, 4096, 64, 0.125f, 0, nullptr,
                                     static_cast<const uint8_t*>(at(3)), 0, nullptr),
         FA_ERR_INVALID_ARG);
  EXPECT(flash_attn_fwd_block_sparse(at(0), at(1), at(2), at(3), fat(4), 1, 1, 4096, 64, 0.125f, 0, nullptr,
                                     static_cast<const uint8_t*>(top(512)), 0, nullptr),
         FA_ERR_INVALID_ARG);

  // 8-bit forward: dequantisation factors and the N % 4 rule
  EXPECT(flash_attn_fwd_fp8(at(0), at(1), at(2), at(3), fat(4), 2, 2, 256, 128, 0.088f, 0, nullptr, 0.01f, 0.01f,
                            0.01f, nullptr),
         FA_OK);
  EXPECT(flash_attn_fwd_fp8(at(0), at(1), at(2), at(3), fat(4), 2, 2, 258, 128, 0.088f, 0, nullptr, 0.01f, 0.01f,
                            0.01f, nullptr),
         FA_ERR_UNSUPPORTED);
  EXPECT(flash_attn_fwd_fp8(at(0), at(1), at(2), at(3), fat(4), 2, 2, 256, 128, 0.088f, 0, nullptr, 0.f, 0.01f,
                            0.01f, nullptr),
         FA_ERR_INVALID_ARG);
  EXPECT(flash_attn_fwd_fp8(at(0), at(1), at(2), at(3), fat(4), 2, 2, 256, 128, 1e30f, 0, nullptr, 1e30f, 1e30f,
                            0.01f, nullptr),
         FA_ERR_INVALID_ARG);

  // status strings
  for (int st = -1; st <= 5; ++st) {
    ++checks;
    const char* s = flash_attn_status_string(st);
    if (!s || std::strlen(s) == 0) {
      std::printf("FAIL: empty status string for %d\n", st);
      ++failures;
    }
  }

  if (failures) {
    std::printf("%d of %d checks failed\n", failures, checks);
    return 1;
  }
  std::printf("all %d checks passed (%d launcher calls reached)\n", checks, fa::g_launches);
  return 0;
}
