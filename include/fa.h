/*
 * fa.h -- C ABI of the fused exact-attention forward pass for AMD MI355X (gfx950).
 *
 * The library computes, for every batch b, query head h and query row i,
 *
 *     O[b,h,i,:] = sum_j P_ij V[b,kv(h),j,:],   P_ij = softmax_j(scale * <Q[b,h,i,:], K[b,kv(h),j,:]> + mask_ij)
 *     LSE[b,h,i] = ln sum_j exp(scale * <Q[b,h,i,:], K[b,kv(h),j,:]> + mask_ij)
 *
 * i.e. exact scaled-dot-product attention (page "FlashAttention (DE)",
 * systems-analysis.info, section "Problematik der Standard-Attention", the
 * attention formula; exactness: page "Flash Attention", 21medien.de, key
 * techniques), computed by one fused kernel that tiles Q and K/V, keeps a
 * running row maximum and a running sum of exponentials per query row (same
 * "FlashAttention (DE)" page, sections "Tiling und blockweise Verarbeitung"
 * and "Online-Softmax-Berechnung") and never writes the N x N score matrix to
 * device memory (same page, section "Zusammenfassen von Operationen in einem
 * CUDA-Kernel").  The per-row log-sum-exp is the statistic a recomputing
 * backward pass needs (page "Flash Attention", 21medien.de, overview:
 * recomputation in the backward pass).
 *
 * Conventions that the pages leave open:
 *  - causal masking (page "Flash Attention", 21medien.de, key techniques) is
 *    aligned to the bottom-right corner: key j is visible to query i iff
 *    j <= i + (Nk - Nq).  A row that sees no key gets O = 0 and LSE = -inf.
 *  - grouped-query / multi-query attention (same page, key techniques): the
 *    query head h reads key/value head kv(h) = h / (Hq / Hkv), i.e.
 *    consecutive groups of Hq/Hkv query heads share one key/value head.
 */
#ifndef FA_H
#define FA_H

#include <hip/hip_runtime_api.h>  /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of Q, K and V (fa_fwd: BF16 or FP8_E4M3; O is always
 * bfloat16, LSE always float32) and of the input of fa_rotate_quantize_e4m3
 * (BF16 or F32). */
typedef enum {
    FA_DTYPE_BF16 = 0,       /* bfloat16 (upper half of an IEEE binary32) */
    FA_DTYPE_FP8_E4M3 = 1,   /* OCP FP8 E4M3 (bias 7, max 448, no inf), per-tensor scales */
    FA_DTYPE_F32 = 2         /* IEEE binary32 */
} fa_dtype_t;

typedef enum {
    FA_SUCCESS = 0,
    FA_ERROR_INVALID_VALUE = 1,   /* an argument is out of its documented range */
    FA_ERROR_NOT_SUPPORTED = 2,   /* a valid combination this library has no kernel for */
    FA_ERROR_LAUNCH_FAILURE = 3   /* the HIP runtime reported an error at launch */
} fa_status_t;

/*
 * fa_fwd -- attention forward pass, asynchronous on `stream`.
 *
 * Pointers (all device memory, owned by the caller, 16-byte aligned,
 * row-major and contiguous):
 *   q    [B, Hq,  Nq, d]  elements of `dtype`
 *   k    [B, Hkv, Nk, d]  elements of `dtype`
 *   v    [B, Hkv, Nk, d]  elements of `dtype`
 *   o    [B, Hq,  Nq, d]  bfloat16 output (written)
 *   lse  [B, Hq,  Nq]     float32 output, natural-log log-sum-exp of the
 *                         scaled, masked scores (written); may be NULL when
 *                         the caller does not need it.
 * Sizes: B >= 0, Hq >= 1, Hkv >= 1 with Hq % Hkv == 0, Nq >= 0, Nk >= 0,
 *   d in {64, 128} for bf16 and d == 128 for fp8; every tensor must hold
 *   fewer than 2^31 elements.  Nk == 0 while B * Hq * Nq > 0 is an
 *   FA_ERROR_INVALID_VALUE (there are rows to compute and no key).
 * causal: 0 or 1 (bottom-right aligned mask, see above).
 * scale: multiplies the raw dot products; any finite value (callers
 *   normally pass 1/sqrt(d), the formula's 1/sqrt(d_k)).
 * descale_qkv: for FA_DTYPE_FP8_E4M3, a HOST pointer to three positive,
 *   finite float32 values {sq, sk, sv}: the real inputs are code * s.  Must
 *   be NULL for FA_DTYPE_BF16.
 *
 * Returns FA_SUCCESS after the kernel is enqueued (or when B*Hq*Nq == 0, in
 * which case nothing is launched).  On any error nothing is launched and
 * the outputs are untouched.  The library allocates no device memory and
 * keeps no mutable global state; concurrent calls on different streams are
 * safe.  The call does not synchronise; the caller orders later work on
 * `stream` (or synchronises) before reading o and lse.
 */
fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int Nq, int Nk, int d,
                   int causal, float scale, fa_dtype_t dtype,
                   const float* descale_qkv, hipStream_t stream);

/*
 * fa_fwd_validate -- the argument checks fa_fwd performs before launching,
 * as a pure host function (it makes no HIP call and touches no device
 * memory; for FP8 it reads the three host-side descale values).  Returns the
 * status fa_fwd would return for these arguments short of a launch failure.
 */
fa_status_t fa_fwd_validate(const void* q, const void* k, const void* v, const void* o,
                            const float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                            int causal, float scale, fa_dtype_t dtype,
                            const float* descale_qkv);

/*
 * fa_rotate_quantize_e4m3 -- incoherent processing before FP8 attention,
 * asynchronous on `stream`.
 *
 * Rotates every row of x by M = D H / sqrt(d) -- D = diag(sigma) with
 * sigma_j = -1 where bit j of sign_bits is set (+1 otherwise), H the d x d
 * Sylvester-Hadamard matrix, H[i][j] = (-1)^popcount(i & j) -- and quantises
 * the rotated tensor per tensor to OCP E4M3: s = max |x M| / 448 (1 when the
 * tensor is all zeros), codes = E4M3(x M / s), rounded to nearest even and
 * clamped to +-448 (page "FlashAttention-3 (DE)", systems-analysis.ru,
 * technical innovation 3: a random orthogonal transform of Q and K spreads
 * outlier features before the FP8 quantisation, and Q K^T is unchanged
 * because M is orthogonal).  Rotate Q and K with the same signs; V is
 * quantised without rotation (rotate = 0).  The codes and s are then the
 * q/k/v and descale arguments of fa_fwd with FA_DTYPE_FP8_E4M3.
 *
 * Pointers (device memory, owned by the caller):
 *   x      [rows, d] elements of x_dtype (FA_DTYPE_BF16 or FA_DTYPE_F32),
 *          row-major, aligned to 16 bytes
 *   codes  [rows, d] E4M3 codes (written), aligned to 16 bytes
 *   scale  one float (written): s
 *   work   one float of workspace the call overwrites; calls that share it
 *          must be ordered on one stream
 * sign_bits: HOST pointer to d / 32 words (bit j of word j / 32 negates
 *   feature j), read during the call; NULL means no sign flips.  Ignored
 *   when rotate == 0.
 * rows >= 0 with rows * d < 2^31; d in {64, 128}; rotate 0 or 1.
 *
 * Returns FA_SUCCESS after the kernels are enqueued (the scale is written
 * even for rows == 0), FA_ERROR_INVALID_VALUE for a null or misaligned
 * pointer or an out-of-range size, FA_ERROR_NOT_SUPPORTED for another d or
 * input dtype; on any error nothing is launched and the outputs are
 * untouched.  No device memory is allocated.
 */
fa_status_t fa_rotate_quantize_e4m3(const void* x, fa_dtype_t x_dtype, long long rows, int d,
                                    int rotate, const unsigned int* sign_bits,
                                    unsigned char* codes, float* scale, float* work,
                                    hipStream_t stream);

/* The argument checks of fa_rotate_quantize_e4m3 as a pure host function. */
fa_status_t fa_rotate_quantize_validate(const void* x, fa_dtype_t x_dtype, long long rows, int d,
                                        int rotate, const unsigned char* codes, const float* scale,
                                        const float* work);

/*
 * fa_fwd_varlen -- fa_fwd over a batch of sequences of different lengths,
 * packed without padding, asynchronous on `stream` (bf16).
 *
 * Sequence s has the query tokens cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1 and
 * the key/value tokens cu_seqlens_k[s] .. cu_seqlens_k[s+1]-1; each
 * sequence is an independent attention problem with the masking, head
 * grouping and bottom-right causal alignment of fa_fwd (page "Flash
 * Attention", 21medien.de, key techniques: variable sequence lengths).
 *
 * Pointers (device memory, owned by the caller), token-major packed layout:
 *   q, o   [total_q, Hq, d] bf16, aligned to 16 bytes
 *   k, v   [total_k, Hkv, d] bf16, aligned to 16 bytes
 *   lse    [Hq, total_q] fp32, or NULL
 *   cu_seqlens_q, cu_seqlens_k   n_seqs + 1 int32 offsets each, device memory,
 *          non-decreasing from 0 to total_q (total_k)
 * max_seqlen_q must be at least every query length (it sizes the grid);
 * query rows past it are not written.  The kernels clamp every offset to
 * [0, total], so malformed offsets give wrong results, never an access out of
 * bounds.  dtype must be FA_DTYPE_BF16 and d in {64, 128}.
 *
 * Returns as fa_fwd; nothing is launched on an argument error.
 */
fa_status_t fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                          const int* cu_seqlens_q, const int* cu_seqlens_k, int n_seqs, int max_seqlen_q,
                          int total_q, int total_k, int Hq, int Hkv, int d, int causal, float scale,
                          fa_dtype_t dtype, hipStream_t stream);

/* The argument checks of fa_fwd_varlen as a pure host function (the offsets
 * themselves live in device memory and are not read). */
fa_status_t fa_fwd_varlen_validate(const void* q, const void* k, const void* v, const void* o,
                                   const float* lse, const int* cu_seqlens_q, const int* cu_seqlens_k,
                                   int n_seqs, int max_seqlen_q, int total_q, int total_k, int Hq, int Hkv,
                                   int d, int causal, float scale, fa_dtype_t dtype);

/*
 * fa_fwd_splitkv -- fa_fwd for decode shapes with the keys split over
 * n_splits workgroups per (batch, key/value head), asynchronous on `stream`.
 *
 * Same result as fa_fwd (up to rounding order).  With few (batch, key/value
 * head) units the decode kernel's grid cannot fill the GPU; splitting the
 * keys gives every split its own workgroup, which writes a normalised
 * partial O and its log-sum-exp to `workspace`; a merge kernel then combines
 * the splits with the online-softmax rescaling rule (page "FlashAttention
 * (DE)", systems-analysis.info, section "Online-Softmax-Berechnung").
 *
 * Arguments as fa_fwd (bf16, d = 128, Nq <= 16; other shapes return
 * FA_ERROR_NOT_SUPPORTED), plus:
 *   n_splits   1 .. 256; 1 is fa_fwd's decode path and ignores workspace
 *   workspace  device memory of n_splits * B * Hq * Nq * (d + 1) floats,
 *              aligned to 16 bytes, overwritten; calls that share it must be
 *              ordered on one stream
 * Returns as fa_fwd.  No device memory is allocated.
 */
fa_status_t fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                           int Hkv, int Nq, int Nk, int d, int causal, float scale, fa_dtype_t dtype,
                           int n_splits, float* workspace, hipStream_t stream);

/* The argument checks of fa_fwd_splitkv as a pure host function. */
fa_status_t fa_fwd_splitkv_validate(const void* q, const void* k, const void* v, const void* o,
                                    const float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                                    int causal, float scale, fa_dtype_t dtype, int n_splits,
                                    const float* workspace);

/*
 * fa_fwd_splitkv_noalloc -- fa_fwd_splitkv without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, hosts that forbid allocation.
 *
 * The split partials go to a scratch array of FA_SPLITKV_SCRATCH_FLOATS
 * floats (16 MiB) that the library holds in each GPU's memory from load until
 * the process ends; the call allocates nothing (no hipMalloc, no allocating
 * library routine).  Arguments and result as fa_fwd_splitkv; a call with
 * n_splits > 1 whose n_splits * B * Hq * Nq * (d + 1) floats exceed
 * FA_SPLITKV_SCRATCH_FLOATS returns FA_ERROR_INVALID_VALUE before any launch
 * (n_splits = 1 uses no scratch), and one whose scratch array cannot be
 * located on the current device FA_ERROR_LAUNCH_FAILURE.  The scratch array
 * keeps the last call's contents (every split overwrites its partial before
 * the merge reads it).  All calls on one GPU share its array: calls that
 * overlap in time on one GPU (on different streams, or from several host
 * threads without ordering) race and give wrong results; order them on one
 * stream.
 */
#define FA_SPLITKV_SCRATCH_FLOATS (4u << 20)
fa_status_t fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                   int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                                   fa_dtype_t dtype, int n_splits, hipStream_t stream);

/*
 * fa_bwd -- backward pass of fa_fwd (bf16), asynchronous on `stream`.
 *
 * Given the forward inputs q, k, v, the forward outputs o and lse (as
 * written by fa_fwd with the same arguments) and the gradient dout of a loss
 * with respect to o, writes the gradients dq, dk, dv.  Attention
 * probabilities are recomputed from q, k and lse, not stored (page "Flash
 * Attention", 21medien.de, key techniques, recomputation).  With
 * S = scale q k^T + mask and P = exp(S - lse) row by row:
 *   dv = P^T dout,  dP = dout v^T,  dS = P * (dP - D) with D_i = <dout_i, o_i>,
 *   dq = scale dS k,  dk = scale dS^T q,
 * where a key/value head's dk and dv sum over every query head that reads
 * it.  Masking, head grouping and the bottom-right causal alignment are those
 * of fa_fwd; rows that see no key (lse = -inf) contribute nothing.
 *
 * Pointers (device memory, owned by the caller; layouts as in fa_fwd):
 *   q, o, dout, dq   [B, Hq, Nq, d] bf16, aligned to 16 bytes
 *   k, v, dk, dv     [B, Hkv, Nk, d] bf16, aligned to 16 bytes
 *   lse              [B, Hq, Nq] fp32
 *   workspace        2 * B * Hq * Nq floats the call overwrites (D and a
 *                    base-2 copy of lse); calls that share it must be ordered
 * dq, dk and dv are written in full (keys no query sees get zero gradients).
 * dtype must be FA_DTYPE_BF16; d in {64, 128}; other sizes as in fa_fwd
 * (Nk == 0 while B * Hq * Nq > 0 is an FA_ERROR_INVALID_VALUE, as there).
 *
 * Returns FA_SUCCESS once the kernels are enqueued, FA_ERROR_INVALID_VALUE
 * for a null or misaligned pointer or an out-of-range size,
 * FA_ERROR_NOT_SUPPORTED for another dtype or d, FA_ERROR_LAUNCH_FAILURE if a
 * launch fails.  On an argument error nothing is launched.  No device memory
 * is allocated.
 */
fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, float* workspace, int B, int Hq,
                   int Hkv, int Nq, int Nk, int d, int causal, float scale, fa_dtype_t dtype,
                   hipStream_t stream);

/* The argument checks of fa_bwd as a pure host function. */
fa_status_t fa_bwd_validate(const void* q, const void* k, const void* v, const void* o,
                            const float* lse, const void* dout, const void* dq, const void* dk,
                            const void* dv, const float* workspace, int B, int Hq, int Hkv, int Nq,
                            int Nk, int d, int causal, float scale, fa_dtype_t dtype);

/*
 * fa_bwd_varlen -- fa_bwd for the packed variable-length layout of
 * fa_fwd_varlen, asynchronous on `stream` (bf16).
 *
 * q, o, dout, dq [total_q, Hq, d]; k, v, dk, dv [total_k, Hkv, d]; lse
 * [Hq, total_q] as written by fa_fwd_varlen; cu_seqlens_q / cu_seqlens_k
 * the same device offsets (n_seqs + 1 each); max_seqlen_q / max_seqlen_k at
 * least every query / key length (they size the grids).  workspace:
 * 2 * Hq * total_q floats, overwritten.  Every sequence is an independent
 * problem; the gradients are those of fa_bwd for each sequence.  dk and dv
 * are written for every key of every sequence (zero where no query sees the
 * key); rows past the max lengths are not written.  Offsets are clamped to
 * [0, total] in the kernels.  Returns as fa_bwd.
 */
fa_status_t fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv, float* workspace,
                          const int* cu_seqlens_q, const int* cu_seqlens_k, int n_seqs, int max_seqlen_q,
                          int max_seqlen_k, int total_q, int total_k, int Hq, int Hkv, int d, int causal,
                          float scale, fa_dtype_t dtype, hipStream_t stream);

/* The argument checks of fa_bwd_varlen as a pure host function. */
fa_status_t fa_bwd_varlen_validate(const void* q, const void* k, const void* v, const void* o,
                                   const float* lse, const void* dout, const void* dq, const void* dk,
                                   const void* dv, const float* workspace, const int* cu_seqlens_q,
                                   const int* cu_seqlens_k, int n_seqs, int max_seqlen_q, int max_seqlen_k,
                                   int total_q, int total_k, int Hq, int Hkv, int d, int causal, float scale,
                                   fa_dtype_t dtype);

/* A static, human-readable description of a status code. */
const char* fa_status_string(fa_status_t status);

/* Library version, major * 10000 + minor * 100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
