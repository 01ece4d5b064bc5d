/*
 * gptq.h -- C ABI of the MI355X (gfx950) GPTQ layer-quantization library.
 *
 * The operation is GPTQ as derived on the pages
 *   [derivation] hbblog.cn  "GPTQ 从零推导：4-bit 权重量化为什么能“量化一列，补偿一列”"
 *   [teardown]   pinghaoyang.com.cn "GPTQ 完全拆解：二阶信息驱动的权重量化"
 * for one linear layer y = W x, W in R^{m x d}:
 *   1. H = (2/N) X X^T from N calibration inputs           ([derivation] eq. (9))
 *   2. dead-feature fix, optional act-order, damping       ([derivation] section 10, eq. (12), (34))
 *   3. R = upper Cholesky factor of (H + damp I)^-1        ([derivation] eq. (37)-(40))
 *   4. column-by-column b-bit affine quantization with the OBS feedback
 *      eta = (w - q) / R_jj folded into later columns, all rows in parallel,
 *      and the lazy block update W[:, T] -= E R[B, T]        ([derivation] eq. (36), (42), (46);
 *                                                            [teardown] Algorithm 1)
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless marked [host].  The caller owns every
 *     buffer; the library never allocates or frees memory.  Its only state
 *     is one internal stream and two events per device, created on the first
 *     factor and kept until the process ends.  Calls that share a workspace
 *     must not overlap.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it in order.  The factor also runs part of the
 *     triangular inverse on the internal stream, forked from `stream` and
 *     joined back into it by events before the call's later work, so the
 *     call stays ordered on `stream` as a whole.  gptq_cholesky_inverse and
 *     gptq_quantize_layer (when it factors) enqueue all of a damping
 *     attempt's work, then synchronise `stream` once to read the
 *     positive-definiteness flag; a failed attempt is redone whole.
 *   - Matrices are row-major with an explicit leading dimension.
 *   - Every argument is validated before anything is enqueued; a call that
 *     fails validation returns a status and leaves outputs untouched (NOT_SPD
 *     is reported after the work ran; see the factor).  Nothing is thrown
 *     across the ABI.
 */
#ifndef GPTQ_MI355_H
#define GPTQ_MI355_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gptq_status {
  GPTQ_OK = 0,
  GPTQ_ERR_INVALID_ARG = 1, /* bad size, pointer, dtype or parameter           */
  GPTQ_ERR_NOT_SPD = 2,     /* damped Hessian not positive definite after the
                               retries ([derivation] section 10: raise the
                               damping and retry; here damp *= 10, 5 times)   */
  GPTQ_ERR_WORKSPACE = 3,   /* ws_bytes smaller than the matching *_bytes query */
  GPTQ_ERR_HIP = 4          /* a HIP launch or runtime call failed              */
} gptq_status;

typedef enum gptq_dtype { GPTQ_BF16 = 0, GPTQ_F32 = 1 } gptq_dtype;

/* Quantizer settings; names follow the GPTQConfig fields the pages mention
 * (bits, group_size, desc_act) plus the algorithm's block size and damping. */
typedef struct gptq_params {
  int32_t bits;       /* 2, 3, 4 or 8                                           */
  int32_t group_size; /* -1: one grid per row, fitted on the original row.
                         >0: dynamic groups of g columns in processing order,
                         refitted at each group start on the compensated
                         working weights ([derivation] 8.3/8.4).  Every group
                         that starts inside a block must end inside it.       */
  int32_t blocksize;  /* lazy-update block, >= 1 (the pages use 128)           */
  float percdamp;     /* damp = max(percdamp * mean(diag H), 2^-23), >= 0       */
  int32_t act_order;  /* 0: natural order; 1: descending diag(H), stable       */
} gptq_params;

const char* gptq_status_string(gptq_status s);

/* ---------------------------------------------------------------------------
 * Hessian statistics ([derivation] eq. (5), (9); accumulable over chunks, 9.4)
 *
 *   S[d, d] += sum_t x_t x_t^T   over the n_tok rows x_t of X.
 *
 * X: token-major activations [n_tok, d], row stride ldx >= d elements, dtype
 *    GPTQ_BF16 (products exact in fp32, accumulated in fp32 on the matrix
 *    cores) or GPTQ_F32 (accumulated in fp64).
 * S: fp32 [d, d] row-major, dense and symmetric on return.  Zero it before the
 *    first chunk; the caller keeps the running token count N.
 * ws: device scratch of at least gptq_hessian_workspace_bytes(d, n_tok) bytes
 *    (may be 0 bytes, then ws may be NULL).
 * Errors: INVALID_ARG for d <= 0, n_tok < 0, ldx < d, NULL S/X (X may be NULL
 * when n_tok == 0), bad dtype; WORKSPACE; HIP.
 * ------------------------------------------------------------------------- */
size_t gptq_hessian_workspace_bytes(int64_t d, int64_t n_tok);
gptq_status gptq_hessian_accumulate(float* S, int64_t d, const void* X,
                                    gptq_dtype x_dtype, int64_t n_tok,
                                    int64_t ldx, void* ws, size_t ws_bytes,
                                    void* stream);

/* ---------------------------------------------------------------------------
 * Factor ([derivation] section 10 steps 5-6, eq. (37)-(40)).
 *
 * From S (fp32 [d, d], as accumulated above) and the token count n:
 *   H = (2/n) S; dead[j] = (S[j][j] == 0), H[j][j] = 1 for dead j;
 *   perm = identity, or the stable order of descending diag(H) (act_order);
 *   H' = H[perm][:, perm] + damp I, damp = max(percdamp * mean diag H, 2^-23);
 *   R  = upper Cholesky factor of H'^-1, i.e. R^T R = H'^-1.
 * Computed in fp64 as H' = U U^T (U upper) and R = U^-1.  On failure the
 * damping is multiplied by 10 and the factorisation retried, at most 5 times.
 *
 * Outputs: R fp32 [d, d] row-major, processing order, lower triangle 0;
 *          perm int32 [d] (perm[j] = original column processed j-th);
 *          dead uint8 [d] (original order); *damp_used [host] (may be NULL).
 * ws: at least gptq_factor_workspace_bytes(d).
 * Errors: INVALID_ARG (d <= 0, n <= 0, percdamp < 0 or NaN, NULL outputs);
 *         WORKSPACE; NOT_SPD (*damp_used = last damping tried; R, perm and
 *         dead then hold the last attempt's values, R meaningless); HIP.
 * ------------------------------------------------------------------------- */
size_t gptq_factor_workspace_bytes(int64_t d);
gptq_status gptq_cholesky_inverse(const float* S, int64_t n, int64_t d,
                                  float percdamp, int32_t act_order, float* R,
                                  int32_t* perm, uint8_t* dead,
                                  float* damp_used, void* ws, size_t ws_bytes,
                                  void* stream);

/* ---------------------------------------------------------------------------
 * Quantize one layer ([teardown] Algorithm 1; [derivation] section 10 with
 * dynamic groups and act-order per 8.3-8.4).
 *
 * W: [m, d] row-major (row stride ldw >= d), GPTQ_BF16 or GPTQ_F32; read only.
 * Factor input, one of:
 *   - R, perm, dead all NULL: S (fp32 [d, d]) and n are used and the factor
 *     is computed internally exactly as gptq_cholesky_inverse does;
 *   - R, perm, dead all non-NULL: a factor from gptq_cholesky_inverse for the
 *     same S, percdamp and act_order (layers sharing one Hessian); S may be
 *     NULL and n is ignored.
 * Outputs (all in ORIGINAL column order, fully overwritten):
 *   qweight uint32 [m, ceil(d*bits/32)]: per row an LSB-first bit stream,
 *           column c's code in stream bits [c*bits, (c+1)*bits), stream bit p
 *           in bit p%32 of word p/32; unused trailing bits are 0;
 *   scales  fp32  [m, n_g]  step Delta of each (row, processing group);
 *   zeros   uint8 [m, n_g]  integer zero point z;
 *           n_g = 1 for group_size -1, else ceil(d / group_size);
 *   g_idx   int32 [d]       group of each original column (0 for -1);
 *   w_hat   fp32  [m, d]    dequantized Delta * (code - z); may be NULL.
 * Codes c = clip(round_half_even(w / Delta) + z, 0, 2^bits - 1) (eq. (36)).
 * ws: at least gptq_workspace_bytes(m, d, p) (includes the factor workspace
 *     only when the factor is computed internally: pass factor_inside = 1).
 * Errors: INVALID_ARG (m, d <= 0, ldw < d, bad params, mixed NULL-ness of
 *         R/perm/dead, NULL S when factoring, NULL outputs); WORKSPACE;
 *         NOT_SPD (the outputs then hold meaningless values); HIP.
 * ------------------------------------------------------------------------- */
size_t gptq_workspace_bytes(int64_t m, int64_t d, const gptq_params* p,
                            int32_t factor_inside);
gptq_status gptq_quantize_layer(const void* W, gptq_dtype w_dtype, int64_t m,
                                int64_t d, int64_t ldw, const float* S,
                                int64_t n, const gptq_params* p,
                                const float* R, const int32_t* perm,
                                const uint8_t* dead, uint32_t* qweight,
                                float* scales, uint8_t* zeros, int32_t* g_idx,
                                float* w_hat, void* ws, size_t ws_bytes,
                                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_MI355_H */
