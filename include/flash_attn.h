/*
 * flash_attn.h -- C ABI of libflashattn.so: exact attention forward and
 * backward on one AMD Instinct MI355X (gfx950).
 *
 * The forward computes O = softmax(scale * Q K^T + mask) V block by block
 * with a running softmax, so the N x N score and probability matrices never
 * reach device memory, and saves one log-sum-exp value per query row
 * ("FlashAttention and GPU Memory", chapters 07 Blocks and 08 A softmax with
 * a running tally; "48 FlashAttention", the sdpa snippet, for the
 * 1/sqrt(d) scaling). The backward rebuilds the score and probability tiles
 * from Q, K, V and the saved row statistics instead of reading a stored P
 * ("FlashAttention and GPU Memory", chapter 09 Backward: recomputing beats
 * reading; "FlashAttention does more arithmetic to move less data", section
 * "FlashAttention never writes the full score table to HBM", move 4).
 *
 * Conventions shared by every entry point:
 *   - Tensors are dense, row-major [B, H, N, d] with d innermost (element
 *     (b,h,n,c) at ((b*H + h)*N + n)*d + c). LSE and the backward workspace
 *     rows are [B, H, N].
 *   - All tensor pointers are DEVICE pointers, owned by the caller. The
 *     library allocates nothing, keeps no state between calls and never
 *     synchronises; every kernel is enqueued on `stream` (a hipStream_t,
 *     NULL = the default stream). Outputs must not alias inputs or each other.
 *   - Masking: key j is visible to query i iff j < kv_len[b] (when kv_len is
 *     not NULL) and, when causal != 0, j <= i (top-left aligned,
 *     self-attention: the query and key sequences have the same length N).
 *     kv_len is a DEVICE array of B int32 values; values outside [0, N] are
 *     clamped to it by the kernels. A query row with no visible key gets
 *     O = 0, LSE = -inf and contributes no gradient.
 *   - scale multiplies the scores; it must be finite and > 0 (1/sqrt(d) is
 *     the usual value).
 *   - d must be 64 or 128; N, B, H >= 1; B*H*N*d must fit in a signed
 *     32-bit element index.
 *   - Arguments are checked on the host before anything is enqueued; a bad
 *     argument returns FA_ERR_INVALID_ARG (or FA_ERR_UNSUPPORTED for a
 *     well-formed request this build does not implement) and launches
 *     nothing. A failed launch returns FA_ERR_HIP. Faults inside a kernel
 *     surface at the caller's next synchronisation.
 */
#ifndef FLASH_ATTN_H
#define FLASH_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1,
  FA_ERR_UNSUPPORTED = 2,
  FA_ERR_HIP = 3,
  FA_ERR_SCRATCH_LIMIT = 4
} fa_status;

/* flash_attn_bwd flags. */
enum {
  /* Compute the per-row term sum_j P_ij dP_ij exactly, by an extra pass that
   * recomputes the score and dP tiles, instead of from the bf16-rounded
   * output as rowsum(dO * O); and feed P and dS to the gradient products as
   * a bf16 high/low pair. Slower (about twice the matrix work), for inputs
   * whose gradients are large (e.g. outlier keys), where bf16 rounding of
   * O, P and dS dominates the error. */
  FA_BWD_PRECISE = 1u << 0,
  /* Accumulate dQ inside the key-outer kernel with fp32 atomics (one kernel
   * doing the 5 algorithmic products) instead of the default pair of kernels
   * that each write their outputs once (7 products' worth of work, no
   * atomics). Kept for comparison; dQ is then not bitwise reproducible. */
  FA_BWD_DQ_ATOMIC = 1u << 1
};

/*
 * Forward, bf16. Q, K, V: bf16 [B,H,N,d]. O: bf16 [B,H,N,d] output,
 * normalised. LSE: float [B,H,N] output, natural log:
 * LSE_i = ln sum_j exp(scale * q_i . k_j) over visible j.
 * Scores, the running maximum and sum, and both products accumulate in
 * fp32; P is rounded to bf16 only as the operand of the P V product.
 */
int flash_attn_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
                   int B, int H, int N, int d, float scale, int causal,
                   const int32_t* kv_len, void* stream);

/*
 * Backward, bf16 inputs, fp32 gradients. Q, K, V, O, dO: bf16 [B,H,N,d]
 * (O and LSE exactly as flash_attn_fwd wrote them). dQ, dK, dV: float
 * [B,H,N,d] outputs, fully overwritten. workspace: device memory of at least
 * flash_attn_bwd_workspace_bytes(B,H,N,d,flags) bytes, 256-byte aligned,
 * used for the per-row term D_i = sum_j P_ij dP_ij; its contents on entry
 * do not matter. flags: any combination of FA_BWD_PRECISE and
 * FA_BWD_DQ_ATOMIC; any other bit is FA_ERR_INVALID_ARG. By default every
 * gradient is written exactly once and all three are bitwise reproducible;
 * with FA_BWD_DQ_ATOMIC, dQ is accumulated with fp32 atomics and is not.
 */
int flash_attn_bwd(const void* Q, const void* K, const void* V, const void* O,
                   const void* dO, const float* LSE, float* dQ, float* dK, float* dV,
                   void* workspace, size_t workspace_bytes,
                   int B, int H, int N, int d, float scale, int causal,
                   const int32_t* kv_len, unsigned flags, void* stream);

/*
 * Allocation-free backward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same arguments, kernels, results and flags as flash_attn_bwd,
 * without the workspace: the per-row term D_i lives in a fixed 16 MiB device
 * array inside the library (one per GPU, held until the process ends),
 * whose address is looked up on the first call on each device. Nothing is
 * allocated or freed by the call. B*H*N above 4194304 rows returns
 * FA_ERR_SCRATCH_LIMIT and launches nothing. Every call on one GPU shares
 * that GPU's array: calls that overlap in time on one GPU (e.g. on two
 * streams without ordering between them) race and give wrong gradients.
 * The array's contents on entry do not matter.
 */
int flash_attn_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O,
                           const void* dO, const float* LSE, float* dQ, float* dK, float* dV,
                           int B, int H, int N, int d, float scale, int causal,
                           const int32_t* kv_len, unsigned flags, void* stream);

/* Workspace bytes flash_attn_bwd / flash_attn_bwd_f32 need (0 for bad sizes). */
size_t flash_attn_bwd_workspace_bytes(int B, int H, int N, int d, unsigned flags);

/*
 * fp32 twins: identical argument lists and semantics with float Q, K, V, O,
 * dO. Every step runs in fp32 on the vector ALUs (no matrix cores); meant
 * for small single-precision problems and as a precision reference path.
 * flash_attn_bwd_f32 accepts flags == 0 only.
 */
int flash_attn_fwd_f32(const float* Q, const float* K, const float* V, float* O, float* LSE,
                       int B, int H, int N, int d, float scale, int causal,
                       const int32_t* kv_len, void* stream);
int flash_attn_bwd_f32(const float* Q, const float* K, const float* V, const float* O,
                       const float* dO, const float* LSE, float* dQ, float* dK, float* dV,
                       void* workspace, size_t workspace_bytes,
                       int B, int H, int N, int d, float scale, int causal,
                       const int32_t* kv_len, unsigned flags, void* stream);

/*
 * Decoding forward, bf16: Nq new queries per (b, h) against a key/value
 * cache; each new token is a single query row that streams the whole cache,
 * so the call is bound by memory bandwidth ("FlashAttention — why it
 * mattered", closing note).
 *   Q:   bf16 [B,H,Nq,d], the new queries (1 <= Nq <= 8, Nq <= Nk);
 *   K,V: bf16 [B,H,Nk,d], the cache; slots j < kv_len[b] (all Nk when
 *        kv_len is NULL; values clamped to [0, Nk]) hold keys;
 *   O:   bf16 [B,H,Nq,d] output; LSE: float [B,H,Nq] output, natural log.
 * Query i may see key j iff j < L_b and, when causal != 0, j <= L_b - Nq + i
 * (the queries are the last Nq positions of the sequence). A query that
 * sees no key gets O = 0 and LSE = -inf. Scores, softmax statistics and the
 * output accumulate in fp32. The keys are processed in chunks whose partial
 * results are merged with the running-softmax rule ("FlashAttention and GPU
 * Memory", chapter 08); workspace (device, 256-byte aligned, at least
 * flash_attn_decode_workspace_bytes(...) bytes, contents on entry do not
 * matter) holds the per-chunk results. Nq > 8 or d outside {64, 128} is
 * FA_ERR_UNSUPPORTED; other conventions as above.
 */
int flash_attn_decode_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
                          void* workspace, size_t workspace_bytes, int B, int H, int Nq, int Nk,
                          int d, float scale, int causal, const int32_t* kv_len, void* stream);

/* Workspace bytes flash_attn_decode_fwd needs (0 for bad sizes). */
size_t flash_attn_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d);

/* Fused dropout ("FlashAttention and GPU Memory", chapter 07 Blocks, lists
 * dropout among the steps fused into one kernel; chapter 09 has the
 * backward regenerate the dropout mask from the generator state instead of
 * storing it). The mask is never written to memory by these two calls.
 *
 * Each weight P_ij of the softmax is kept with probability (256 - t)/256,
 * t = round(256 * p_drop), and kept weights are scaled by 256/(256 - t):
 * O = (P o Z * 256/(256 - t)) V, so the expected output is exact attention.
 * LSE is the log-sum-exp of the undropped scores, as in flash_attn_fwd.
 * Z comes from Philox4x32-10 (Salmon et al., SC 2011) keyed by `seed`
 * (low word, high word) with counter (j/4, i/4, b*H + h, offset) for query
 * i and key j: element (i, j) is kept iff byte j%4 of output word i%4 is
 * >= t. The same (seed, offset) must be passed to the backward; a new
 * offset draws an independent mask with the same seed.
 *
 * p_drop must satisfy 0 <= p_drop < 1 and round(256 p_drop) < 256,
 * otherwise FA_ERR_INVALID_ARG. bf16 tensors only; other arguments and
 * conventions as flash_attn_fwd / flash_attn_bwd. The backward accepts
 * FA_BWD_PRECISE (any other flag is FA_ERR_INVALID_ARG) and the workspace
 * of flash_attn_bwd_workspace_bytes(B, H, N, d, flags).
 */
int flash_attn_fwd_dropout(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                           int N, int d, float scale, int causal, const int32_t* kv_len, float p_drop,
                           uint64_t seed, uint32_t offset, void* stream);

int flash_attn_bwd_dropout(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                           const float* LSE, float* dQ, float* dK, float* dV, void* workspace,
                           size_t workspace_bytes, int B, int H, int N, int d, float scale, int causal,
                           const int32_t* kv_len, float p_drop, uint64_t seed, uint32_t offset, unsigned flags,
                           void* stream);

/* Writes the keep mask the two calls above use, as bytes (1 = kept), to the
 * DEVICE array mask[B][H][N_q][N_k] (caller-owned, B*H*N_q*N_k bytes), for
 * inspection and testing. Same p_drop, seed and offset rules; N_q, N_k >= 1. */
int flash_attn_dropout_mask(uint8_t* mask, int B, int H, int N_q, int N_k, float p_drop, uint64_t seed,
                            uint32_t offset, void* stream);

/* Block-sparse forward ("FlashAttention and GPU Memory", chapters 10 and 12:
 * the paper's approximate block-sparse variant, used for 64K-long inputs).
 * block_mask is a DEVICE array of bytes, one per (query block, key block) of
 * 128 x 128, row-major [nb][nb] with nb = ceil(N / 128) (query block index
 * first); consecutive (b, h) masks are block_mask_head_stride bytes apart
 * (0: every head uses the same mask). Key j is visible to query i iff
 * block_mask[i/128][j/128] != 0, in addition to kv_len and causal; O and
 * LSE are the exact softmax attention over the visible keys (O = 0,
 * LSE = -inf for a row with none). Only key tiles of non-zero blocks are
 * read from memory. The masks occupy (B*H - 1) * block_mask_head_stride +
 * nb * nb bytes, which must not overlap O or LSE. N <= 65536 (larger:
 * FA_ERR_UNSUPPORTED); NULL mask, a negative stride or an overlap:
 * FA_ERR_INVALID_ARG; other arguments as flash_attn_fwd. */
int flash_attn_fwd_block_sparse(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                                int N, int d, float scale, int causal, const int32_t* kv_len,
                                const uint8_t* block_mask, int64_t block_mask_head_stride, void* stream);

/* 8-bit floating-point forward ("FlashAttention — why it mattered" and
 * "FlashAttention and GPU Memory", chapter 11: the FlashAttention-3 8-bit
 * mode, the method's one source of error beyond rounding order). Q8 and K8
 * are OCP FP8 E4M3 codes (one byte each, [B, H, N, d]); Vt8 holds V
 * transposed, [B, H, d, N]; every value must be finite. The inputs stand for
 * Q = descale_q * Q8, K = descale_k * K8, V = descale_v * Vt8^T (fp32 factors,
 * finite and > 0). O (bf16, [B, H, N, d]) and LSE (fp32, natural log) are
 * the attention of those values: scores and softmax in fp32, the softmax
 * weights rounded to E4M3 for the P V product. N must be a multiple of 4
 * (the rows of Vt8 then start on 4-byte boundaries); other N is
 * FA_ERR_UNSUPPORTED. Other arguments and conventions as flash_attn_fwd. */
int flash_attn_fwd_fp8(const void* Q8, const void* K8, const void* Vt8, void* O, float* LSE, int B, int H, int N,
                       int d, float scale, int causal, const int32_t* kv_len, float descale_q, float descale_k,
                       float descale_v, void* stream);

/* Static, human-readable name of a status code. */
const char* flash_attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FLASH_ATTN_H */
