// extern "C" entry points of libflashattn.so: argument checks on the host,
// then dispatch to the gfx950 launchers. Nothing is enqueued unless every
// check passes.
#include "flash_attn.h"

#include <math.h>
#include <stdint.h>

#include <initializer_list>

#include "fa_launch.h"

namespace {

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
};

Span span(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Span{a, a + bytes};
}

bool overlaps(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// A range whose end passes the top of the address space cannot be a real
// allocation; it would also defeat the overlap test.
bool wraps(Span a) { return a.hi < a.lo; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Whether the product of positive int factors stays within int32 (the
// kernels' element index range). Multiplied one factor at a time so that no
// intermediate can overflow int64.
bool fits_int32(std::initializer_list<int> factors) {
  int64_t p = 1;
  for (int f : factors) {
    p *= f;  // p <= INT32_MAX and f <= INT32_MAX: no overflow
    if (p > INT32_MAX) return false;
  }
  return true;
}

// Shape, scale and flag checks common to every entry point.
int check_shape(int B, int H, int N, int d, float scale) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (!fits_int32({B, H, N, d})) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// Pointer checks: non-NULL, 16-byte aligned, and no output overlapping any
// other tensor (inputs or outputs).
int check_ptrs(const Span* in, const void* const* in_p, int n_in, const Span* out,
               const void* const* out_p, int n_out) {
  for (int i = 0; i < n_in; ++i)
    if (!in_p[i] || !aligned16(in_p[i]) || wraps(in[i])) return FA_ERR_INVALID_ARG;
  for (int i = 0; i < n_out; ++i)
    if (!out_p[i] || !aligned16(out_p[i]) || wraps(out[i])) return FA_ERR_INVALID_ARG;
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlaps(out[i], in[j])) return FA_ERR_INVALID_ARG;
    for (int j = i + 1; j < n_out; ++j)
      if (overlaps(out[i], out[j])) return FA_ERR_INVALID_ARG;
  }
  return FA_OK;
}

size_t workspace_bytes(int B, int H, int N) {
  const size_t rows = (size_t)B * H * N;
  return (rows * sizeof(float) + 255) & ~(size_t)255;
}

int fwd_common(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int N,
               int d, float scale, int causal, size_t esize) {
  int st = check_shape(B, H, N, d, scale);
  if (st != FA_OK) return st;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  const size_t tbytes = (size_t)B * H * N * d * esize;
  const size_t lbytes = (size_t)B * H * N * sizeof(float);
  const void* in_p[3] = {Q, K, V};
  const Span in[3] = {span(Q, tbytes), span(K, tbytes), span(V, tbytes)};
  const void* out_p[2] = {O, LSE};
  const Span out[2] = {span(O, tbytes), span(LSE, lbytes)};
  return check_ptrs(in, in_p, 3, out, out_p, 2);
}

// Backward checks. has_ws = false: the caller passes no workspace (the
// allocation-free entry point), so only the tensors are checked.
int bwd_common(const void* Q, const void* K, const void* V, const void* O, const void* dO,
               const float* LSE, float* dQ, float* dK, float* dV, void* ws, size_t ws_bytes, int B,
               int H, int N, int d, float scale, int causal, unsigned flags, unsigned allowed_flags,
               size_t esize, bool has_ws = true) {
  int st = check_shape(B, H, N, d, scale);
  if (st != FA_OK) return st;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (flags & ~allowed_flags) return FA_ERR_INVALID_ARG;
  const size_t need = workspace_bytes(B, H, N);
  if (has_ws && ws_bytes < need) return FA_ERR_INVALID_ARG;
  const size_t tbytes = (size_t)B * H * N * d * esize;
  const size_t gbytes = (size_t)B * H * N * d * sizeof(float);
  const size_t lbytes = (size_t)B * H * N * sizeof(float);
  const void* in_p[6] = {Q, K, V, O, dO, LSE};
  const Span in[6] = {span(Q, tbytes), span(K, tbytes), span(V, tbytes),
                      span(O, tbytes), span(dO, tbytes), span(LSE, lbytes)};
  const void* out_p[4] = {dQ, dK, dV, ws};
  const Span out[4] = {span(dQ, gbytes), span(dK, gbytes), span(dV, gbytes), span(ws, need)};
  return check_ptrs(in, in_p, 6, out, out_p, has_ws ? 4 : 3);
}

size_t decode_ws_bytes(int B, int H, int Nq, int Nk, int d) {
  const size_t slots = (size_t)B * H * fa::decode_chunks(Nk) * Nq;
  return (slots * (size_t)(d + 1) * sizeof(float) + 255) & ~(size_t)255;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// Dropout parameters: 0 <= p < 1 with round(256 p) < 256.
int drop_params(float p, uint64_t seed, uint32_t offset, fa::DropParams* out) {
  if (!isfinite(p) || p < 0.f || !(p < 1.f)) return FA_ERR_INVALID_ARG;
  const double t = floor((double)p * 256.0 + 0.5);
  if (t >= 256.0) return FA_ERR_INVALID_ARG;
  out->k0 = (unsigned)(seed & 0xFFFFFFFFu);
  out->k1 = (unsigned)(seed >> 32);
  out->offset = offset;
  out->thresh = (unsigned)t;
  out->keep_scale = (float)(256.0 / (256.0 - t));
  return FA_OK;
}

}  // namespace

extern "C" {

int flash_attn_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                   int N, int d, float scale, int causal, const int32_t* kv_len, void* stream) {
  const int st = fwd_common(Q, K, V, O, LSE, B, H, N, d, scale, causal, 2);
  if (st != FA_OK) return st;
  const fa::AttnShape s{B, H, N, d, scale, causal, kv_len};
  return hip_status(fa::launch_fwd_bf16(Q, K, V, O, LSE, s, static_cast<hipStream_t>(stream)));
}

int flash_attn_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                   const float* LSE, float* dQ, float* dK, float* dV, void* workspace,
                   size_t workspace_bytes_, int B, int H, int N, int d, float scale, int causal,
                   const int32_t* kv_len, unsigned flags, void* stream) {
  const int st = bwd_common(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, workspace_bytes_, B, H, N, d,
                            scale, causal, flags, FA_BWD_PRECISE | FA_BWD_DQ_ATOMIC, 2);
  if (st != FA_OK) return st;
  const fa::AttnShape s{B, H, N, d, scale, causal, kv_len};
  return hip_status(fa::launch_bwd_bf16(Q, K, V, O, dO, LSE, dQ, dK, dV, static_cast<float*>(workspace),
                                        s, (flags & FA_BWD_PRECISE) != 0,
                                        (flags & FA_BWD_DQ_ATOMIC) != 0,
                                        static_cast<hipStream_t>(stream)));
}

int flash_attn_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                           const float* LSE, float* dQ, float* dK, float* dV, int B, int H, int N, int d,
                           float scale, int causal, const int32_t* kv_len, unsigned flags, void* stream) {
  const int st = bwd_common(Q, K, V, O, dO, LSE, dQ, dK, dV, nullptr, 0, B, H, N, d, scale, causal, flags,
                            FA_BWD_PRECISE | FA_BWD_DQ_ATOMIC, 2, false);
  if (st != FA_OK) return st;
  if ((size_t)B * H * N > fa::kNoAllocRows) return FA_ERR_SCRATCH_LIMIT;
  float* scratch = nullptr;
  const hipError_t e = fa::noalloc_scratch(&scratch);
  if (e != hipSuccess) return FA_ERR_HIP;
  const fa::AttnShape s{B, H, N, d, scale, causal, kv_len};
  return hip_status(fa::launch_bwd_bf16(Q, K, V, O, dO, LSE, dQ, dK, dV, scratch, s, (flags & FA_BWD_PRECISE) != 0,
                                        (flags & FA_BWD_DQ_ATOMIC) != 0, static_cast<hipStream_t>(stream)));
}

size_t flash_attn_bwd_workspace_bytes(int B, int H, int N, int d, unsigned flags) {
  (void)flags;
  if (B < 1 || H < 1 || N < 1 || d < 1) return 0;
  return workspace_bytes(B, H, N);
}

int flash_attn_fwd_f32(const float* Q, const float* K, const float* V, float* O, float* LSE, int B,
                       int H, int N, int d, float scale, int causal, const int32_t* kv_len,
                       void* stream) {
  const int st = fwd_common(Q, K, V, O, LSE, B, H, N, d, scale, causal, 4);
  if (st != FA_OK) return st;
  const fa::AttnShape s{B, H, N, d, scale, causal, kv_len};
  return hip_status(fa::launch_fwd_f32(Q, K, V, O, LSE, s, static_cast<hipStream_t>(stream)));
}

int flash_attn_bwd_f32(const float* Q, const float* K, const float* V, const float* O,
                       const float* dO, const float* LSE, float* dQ, float* dK, float* dV,
                       void* workspace, size_t workspace_bytes_, int B, int H, int N, int d,
                       float scale, int causal, const int32_t* kv_len, unsigned flags,
                       void* stream) {
  const int st = bwd_common(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, workspace_bytes_, B, H, N, d,
                            scale, causal, flags, 0u, 4);
  if (st != FA_OK) return st;
  const fa::AttnShape s{B, H, N, d, scale, causal, kv_len};
  return hip_status(fa::launch_bwd_f32(Q, K, V, O, dO, LSE, dQ, dK, dV, static_cast<float*>(workspace),
                                       s, static_cast<hipStream_t>(stream)));
}

size_t flash_attn_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return 0;
  return decode_ws_bytes(B, H, Nq, Nk, d);
}

int flash_attn_decode_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, void* workspace,
                          size_t workspace_bytes_, int B, int H, int Nq, int Nk, int d, float scale,
                          int causal, const int32_t* kv_len, void* stream) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (Nq > Nk) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (Nq > 8) return FA_ERR_UNSUPPORTED;
  if (!fits_int32({B, H, Nk, d})) return FA_ERR_UNSUPPORTED;
  const size_t need = decode_ws_bytes(B, H, Nq, Nk, d);
  if (workspace_bytes_ < need) return FA_ERR_INVALID_ARG;
  const size_t qbytes = (size_t)B * H * Nq * d * 2;
  const size_t kbytes = (size_t)B * H * Nk * d * 2;
  const size_t lbytes = (size_t)B * H * Nq * sizeof(float);
  const void* in_p[3] = {Q, K, V};
  const Span in[3] = {span(Q, qbytes), span(K, kbytes), span(V, kbytes)};
  const void* out_p[3] = {O, LSE, workspace};
  const Span out[3] = {span(O, qbytes), span(LSE, lbytes), span(workspace, need)};
  const int st = check_ptrs(in, in_p, 3, out, out_p, 3);
  if (st != FA_OK) return st;
  const fa::DecodeShape s{B, H, Nq, Nk, d, scale, causal, kv_len};
  return hip_status(fa::launch_decode_bf16(Q, K, V, O, LSE, static_cast<float*>(workspace), s,
                                           static_cast<hipStream_t>(stream)));
}

int flash_attn_fwd_dropout(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                           int N, int d, float scale, int causal, const int32_t* kv_len, float p_drop,
                           uint64_t seed, uint32_t offset, void* stream) {
  fa::DropParams dp;
  int st = drop_params(p_drop, seed, offset, &dp);
  if (st != FA_OK) return st;
  st = fwd_common(Q, K, V, O, LSE, B, H, N, d, scale, causal, 2);
  if (st != FA_OK) return st;
  const fa::AttnShape s{B, H, N, d, scale, causal, kv_len};
  return hip_status(fa::launch_fwd_drop_bf16(Q, K, V, O, LSE, s, dp, static_cast<hipStream_t>(stream)));
}

int flash_attn_bwd_dropout(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                           const float* LSE, float* dQ, float* dK, float* dV, void* workspace,
                           size_t workspace_bytes_, int B, int H, int N, int d, float scale, int causal,
                           const int32_t* kv_len, float p_drop, uint64_t seed, uint32_t offset, unsigned flags,
                           void* stream) {
  fa::DropParams dp;
  int st = drop_params(p_drop, seed, offset, &dp);
  if (st != FA_OK) return st;
  st = bwd_common(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, workspace_bytes_, B, H, N, d, scale, causal, flags,
                  FA_BWD_PRECISE, 2);
  if (st != FA_OK) return st;
  const fa::AttnShape s{B, H, N, d, scale, causal, kv_len};
  return hip_status(fa::launch_bwd_drop_bf16(Q, K, V, O, dO, LSE, dQ, dK, dV, static_cast<float*>(workspace), s,
                                             dp, (flags & FA_BWD_PRECISE) != 0, static_cast<hipStream_t>(stream)));
}

int flash_attn_fwd_block_sparse(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                                int N, int d, float scale, int causal, const int32_t* kv_len,
                                const uint8_t* block_mask, int64_t block_mask_head_stride, void* stream) {
  int st = fwd_common(Q, K, V, O, LSE, B, H, N, d, scale, causal, 2);
  if (st != FA_OK) return st;
  if (!block_mask || block_mask_head_stride < 0) return FA_ERR_INVALID_ARG;
  if (N > 65536) return FA_ERR_UNSUPPORTED;
  // The masks span (B*H - 1) * stride + nb^2 bytes and must not overlap an output.
  const int64_t nb = (N + 127) / 128, heads = (int64_t)B * H;
  if (block_mask_head_stride > 0 && heads - 1 > (INT64_MAX - nb * nb) / block_mask_head_stride)
    return FA_ERR_INVALID_ARG;
  const Span mask = span(block_mask, (size_t)((heads - 1) * block_mask_head_stride + nb * nb));
  if (wraps(mask)) return FA_ERR_INVALID_ARG;
  const size_t obytes = (size_t)B * H * N * d * 2, lbytes = (size_t)B * H * N * sizeof(float);
  if (overlaps(mask, span(O, obytes)) || overlaps(mask, span(LSE, lbytes))) return FA_ERR_INVALID_ARG;
  const fa::AttnShape s{B, H, N, d, scale, causal, kv_len};
  return hip_status(fa::launch_fwd_sparse_bf16(Q, K, V, O, LSE, s, block_mask, (long long)block_mask_head_stride,
                                               static_cast<hipStream_t>(stream)));
}

int flash_attn_fwd_fp8(const void* Q8, const void* K8, const void* Vt8, void* O, float* LSE, int B, int H, int N,
                       int d, float scale, int causal, const int32_t* kv_len, float descale_q, float descale_k,
                       float descale_v, void* stream) {
  int st = check_shape(B, H, N, d, scale);
  if (st != FA_OK) return st;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  for (float f : {descale_q, descale_k, descale_v})
    if (!isfinite(f) || !(f > 0.f)) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale * descale_q * descale_k)) return FA_ERR_INVALID_ARG;
  // V^T rows are N bytes long: a multiple of 4 keeps every row dword-aligned,
  // so no 16-byte tile load straddles the end of a head's range.
  if (N % 4 != 0) return FA_ERR_UNSUPPORTED;
  const size_t ebytes = (size_t)B * H * N * d;
  const size_t lbytes = (size_t)B * H * N * sizeof(float);
  const void* in_p[3] = {Q8, K8, Vt8};
  const Span in[3] = {span(Q8, ebytes), span(K8, ebytes), span(Vt8, ebytes)};
  const void* out_p[2] = {O, LSE};
  const Span out[2] = {span(O, 2 * ebytes), span(LSE, lbytes)};
  st = check_ptrs(in, in_p, 3, out, out_p, 2);
  if (st != FA_OK) return st;
  const fa::AttnShape s{B, H, N, d, scale, causal, kv_len};
  return hip_status(fa::launch_fwd_fp8(Q8, K8, Vt8, O, LSE, s, descale_q, descale_k, descale_v,
                                       static_cast<hipStream_t>(stream)));
}

int flash_attn_dropout_mask(uint8_t* mask, int B, int H, int N_q, int N_k, float p_drop, uint64_t seed,
                            uint32_t offset, void* stream) {
  fa::DropParams dp;
  int st = drop_params(p_drop, seed, offset, &dp);
  if (st != FA_OK) return st;
  if (!mask || B < 1 || H < 1 || N_q < 1 || N_k < 1) return FA_ERR_INVALID_ARG;
  if ((int64_t)B * H > INT32_MAX) return FA_ERR_UNSUPPORTED;
  return hip_status(fa::launch_dropout_mask(mask, B, H, N_q, N_k, dp, static_cast<hipStream_t>(stream)));
}

const char* flash_attn_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: an argument failed the host-side checks";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: request is well-formed but not implemented";
    case FA_ERR_HIP: return "FA_ERR_HIP: a kernel launch failed";
    case FA_ERR_SCRATCH_LIMIT:
      return "FA_ERR_SCRATCH_LIMIT: B*H*N exceeds the 4194304 rows of the allocation-free entry point's fixed scratch";
    default: return "unknown flash_attn status";
  }
}

}  // extern "C"
