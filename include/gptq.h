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
 *     buffer; the library never allocates or frees device memory.  State it
 *     keeps between calls, per device, until the process ends: one internal
 *     non-blocking stream and two events (created, under a mutex, by the
 *     first factorisation on that device, with the caller stream's device
 *     current); a library-owned static scratch array and its address (see
 *     gptq_hessian_accumulate_noalloc).  Calls that share a workspace must
 *     not overlap.
 *   - Sizes: every matrix dimension (d, and m for the quantizer) is at most
 *     65535 (one grid dimension per row/column in several launches); larger
 *     values are rejected with GPTQ_ERR_INVALID_ARG.
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

typedef enum gptq_dtype { GPTQ_BF16 = 0, GPTQ_F32 = 1, GPTQ_F16 = 2 } gptq_dtype;

/* The quantization grid ([derivation] 1.1 fit, eq. (36) encoder). */
typedef enum gptq_grid {
  /* min-max over the group, widened to contain 0: Delta = (hi - lo) /
     (2^b - 1), z = round(-lo / Delta); unsigned codes 0 .. 2^b - 1.        */
  GPTQ_GRID_MINMAX = 0,
  /* symmetric ([derivation] 1.1 names it; 8.4 the signed code form): range
     [-a, a], a = max |w|, 2^b - 1 levels -h..h around an exact 0 (h =
     2^(b-1) - 1), Delta = a / h.  Codes are stored SIGNED, c - h as b-bit
     two's complement; zeros[] is written as 0; w_hat = Delta * code.  At
     bits = 2 this is the ternary grid {-1, 0, +1} * Delta of [teardown]
     "extreme quantization: 2-bit and ternary".                              */
  GPTQ_GRID_SYMMETRIC = 1,
  /* given by the caller (fixed_scales / fixed_zeros below), e.g. the fixed
     grid of the [derivation] section 11 example; unsigned codes as for
     MINMAX.  With group_size > 0 the grids are on the static layout.       */
  GPTQ_GRID_FIXED = 2
} gptq_grid;

/* Quantizer settings; names follow the GPTQConfig fields the pages mention
 * (bits, group_size, desc_act) plus the algorithm's block size and damping. */
typedef struct gptq_params {
  int32_t bits;       /* 2, 3, 4 or 8                                           */
  int32_t group_size; /* -1: one grid per row, fitted on the original row.
                         >0: groups of g columns: dynamic (refitted at each
                         group start, in processing order, on the
                         compensated working weights, [derivation] 8.3/8.4;
                         every group that starts inside a block must end
                         inside it) or static (see static_groups).          */
  int32_t blocksize;  /* lazy-update block, >= 1 (the pages use 128)           */
  float percdamp;     /* damp = max(percdamp * mean(diag H), 2^-23), >= 0       */
  int32_t act_order;  /* 0: natural order; 1: descending diag(H), stable       */
  int32_t grid;       /* gptq_grid                                              */
  int32_t static_groups; /* 0/1, with group_size > 0: groups fitted once, before
                         GPTQ, on the ORIGINAL contiguous columns
                         [G g, (G+1) g) of the original row; processing
                         position j uses group floor(perm[j] / g)
                         ([derivation] 8.3), so g_idx[c] = c / g.  Any
                         (g, blocksize) pair.  Implied by GPTQ_GRID_FIXED.  */
  const float* fixed_scales;  /* GPTQ_GRID_FIXED only (else NULL): DEVICE
                         [m, n_g] fp32, positive finite steps               */
  const uint8_t* fixed_zeros; /* GPTQ_GRID_FIXED only (else NULL): DEVICE
                         [m, n_g] zero points <= 2^bits - 1                   */
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
 * Errors: INVALID_ARG for d <= 0, d > 65535, n_tok < 0, ldx < d, NULL S/X
 * (X may be NULL when n_tok == 0), bad dtype; WORKSPACE; HIP.
 * ------------------------------------------------------------------------- */
size_t gptq_hessian_workspace_bytes(int64_t d, int64_t n_tok);
gptq_status gptq_hessian_accumulate(float* S, int64_t d, const void* X,
                                    gptq_dtype x_dtype, int64_t n_tok,
                                    int64_t ldx, void* ws, size_t ws_bytes,
                                    void* stream);

/* ---------------------------------------------------------------------------
 * Allocation-free variant of gptq_hessian_accumulate, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same operation, arguments and errors,
 * without ws: the token-split partial sums live in a static device array of
 * GPTQ_NOALLOC_SCRATCH_BYTES that the library owns (one per GPU it runs on,
 * held until the process ends).  The split plan is chosen to fit that array,
 * so larger problems run with fewer (longer) token splits than
 * gptq_hessian_accumulate may use: S agrees with it to fp32 summation
 * rounding, bit for bit when both plans coincide.  Every partial the call
 * reads it has written itself, so no clearing is needed between calls.  The
 * array is shared by every call on one GPU: calls that overlap on one GPU
 * (other streams, other host threads) race on it and must be serialised by
 * the caller.  Calls no hipMalloc/hipFree.
 * ------------------------------------------------------------------------- */
#define GPTQ_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
gptq_status gptq_hessian_accumulate_noalloc(float* S, int64_t d, const void* X,
                                            gptq_dtype x_dtype, int64_t n_tok,
                                            int64_t ldx, void* stream);

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
 * A non-finite S (NaN or inf on the diagonal) is reported as NOT_SPD; perm
 * is still a permutation (NaN keys order after every number, by index).
 * Errors: INVALID_ARG (d <= 0, d > 65535, n <= 0, percdamp < 0 or NaN, NULL
 *         outputs); WORKSPACE; NOT_SPD (*damp_used = last damping tried; R,
 *         perm and dead then hold the last attempt's values, R meaningless);
 *         HIP.
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
 *   scales  fp32  [m, n_g]  step Delta of each (row, group): processing
 *           groups for dynamic groups, original contiguous groups for
 *           static ones;
 *   zeros   uint8 [m, n_g]  integer zero point z (0 for GPTQ_GRID_SYMMETRIC,
 *           whose codes are signed);
 *           n_g = 1 for group_size -1, else ceil(d / group_size);
 *   g_idx   int32 [d]       group of each original column (0 for -1);
 *   w_hat   fp32  [m, d]    dequantized Delta * (code - z); may be NULL.
 * Codes c = clip(round_half_even(w / Delta) + z, 0, maxq) (eq. (36)),
 * maxq = 2^bits - 1 (2^bits - 2 for the symmetric grid).
 * ws: at least gptq_workspace_bytes(m, d, p) (includes the factor workspace
 *     only when the factor is computed internally: pass factor_inside = 1).
 * Errors: INVALID_ARG (m, d <= 0, m or d > 65535, ldw < d, bad params --
 *         including grid / static_groups out of range, GPTQ_GRID_FIXED
 *         without both fixed arrays or with them for another grid --, mixed
 *         NULL-ness of R/perm/dead, NULL S when factoring, NULL outputs);
 *         WORKSPACE; NOT_SPD (the outputs then hold meaningless values); HIP.
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

/* ---------------------------------------------------------------------------
 * Inference on the stored format: the fused dequantizing matmul
 * ([wiki] "inference": W4A16 -- 4-bit weights expanded inside the matmul
 * kernel -- and 3-/2-bit likewise; format of [derivation] 3.1 / 8.3).
 *
 *   Y[k][r] = sum_c X[k][c] * W_hat[r][c],
 *   W_hat[r][c] = scales[r][g] * (code[r][c] - zeros[r][g]),  g = g_idx[c]
 *   (signed_codes = 1: code sign-extended from `bits` bits, zeros ignored).
 *
 * X: bf16 activations [n, d] token-major, row stride ldx >= d (GPTQ_BF16
 *    only); 0 <= n <= 524280.  Up to 16 rows: the vector units, one weight
 *    pass per 8 rows; more: bf16 matrix cores on tiles of 128 rows.
 * qweight, scales, zeros, g_idx: as gptq_quantize_layer writes them
 *    (qweight [m, ceil(d*bits/32)] uint32, scales / zeros uint8 [m, n_g]
 *    with n_g from group_size, g_idx int32 [d], values < n_g).
 * scale_dtype: GPTQ_F32 (the scales as written) or GPTQ_F16 (the compact
 *    16-bit storage of the steps: fp16 scales [m, n_g], e.g. the fp32 ones
 *    rounded to nearest; each is widened exactly to fp32 in the kernel).
 * Y: fp32 [n, m], row stride ldy >= m; fully overwritten.
 * Sums in fp32, every product of an activation and a code exact: each
 * group's grid is factored out of the group's sums (Delta (sum x c - z sum x)),
 * the codes entering the products as exact small numbers, never as rounded
 * weights.
 * Errors: INVALID_ARG (bad sizes, dtype, scale_dtype, bits, group_size,
 *         NULL pointers when n > 0); HIP.  Allocates nothing; no workspace.
 * ------------------------------------------------------------------------- */
gptq_status gptq_dequant_matmul(const void* X, gptq_dtype x_dtype, int64_t n,
                                int64_t d, int64_t ldx, const uint32_t* qweight,
                                const void* scales, gptq_dtype scale_dtype,
                                const uint8_t* zeros,
                                const int32_t* g_idx, int64_t m, int32_t bits,
                                int32_t group_size, int32_t signed_codes,
                                float* Y, int64_t ldy, void* stream);

/* ---------------------------------------------------------------------------
 * Layer by layer ([derivation] 3.2 steps 1-2 and 10: capture each layer's
 * inputs, quantize it, verify its reconstruction error, go on to the next;
 * [teardown] "layer-wise quantization").
 *
 * For l = 0 .. n_layers-1, with X_0 = X_in:
 *   S_l = X_l^T X_l (gptq_hessian_accumulate);
 *   layer l quantized from S_l and N = n_tok (gptq_quantize_layer, factor
 *   inside, layers[l].params) into layers[l]'s outputs;
 *   layer_err[l] = (1/N) ||(W_l - W_hat_l) X_l||_F^2 ([derivation] eq. (6),
 *   from S_l in fp32 products with fp64 partial sums);
 *   X_{l+1} = bf16(act(X_l W_hat_l^T)) (gptq_dequant_matmul's arithmetic,
 *   then the activation, rounded to nearest even bf16).
 * X_out receives X_{n_layers}: the inputs the next layer would see, so a
 * stack is resumed at any layer by calling again with the remaining layers
 * and that X as X_in (the result is the same bits as one call).
 *
 * layers [host]: n_layers >= 1 descriptors; layers[l].d == layers[l-1].m.
 * X_in: bf16 [n_tok, layers[0].d] contiguous; X_out: bf16 [n_tok,
 * layers[n-1].m] contiguous; 1 <= n_tok <= 524280.  activation: gptq_activation.
 * layer_err [host]: n_layers doubles, may be NULL.
 * ws: at least gptq_stack_workspace_bytes(layers, n_layers, n_tok).
 * Synchronises `stream` once per layer (the factor's flag) and at the end.
 * Errors: INVALID_ARG (any layer's arguments as for gptq_quantize_layer,
 *         mismatched dimensions, bad activation, NULL X_in / X_out);
 *         WORKSPACE; NOT_SPD (from the failing layer; earlier layers'
 *         outputs are final); HIP.
 * ------------------------------------------------------------------------- */
typedef enum gptq_activation {
  GPTQ_ACT_NONE = 0, GPTQ_ACT_RELU = 1, GPTQ_ACT_SILU = 2
} gptq_activation;

typedef struct gptq_stack_layer {
  const void* W;        /* [m, d] row-major, row stride ldw >= d; read only */
  gptq_dtype w_dtype;
  int64_t m, d, ldw;
  gptq_params params;
  uint32_t* qweight;    /* outputs, as gptq_quantize_layer writes them */
  float* scales;
  uint8_t* zeros;
  int32_t* g_idx;
} gptq_stack_layer;

size_t gptq_stack_workspace_bytes(const gptq_stack_layer* layers, int32_t n_layers,
                                  int64_t n_tok);
gptq_status gptq_quantize_stack(const gptq_stack_layer* layers, int32_t n_layers,
                                const void* X_in, int64_t n_tok, int32_t activation,
                                void* X_out, double* layer_err, void* ws,
                                size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Tracing: per-phase GPU time.  While enabled, each launch group of a phase
 * is bracketed by two hipEvents recorded on the caller's stream (a few
 * microseconds per group; leave it off when timing the whole path).
 * Phases: GPTQ_TRACE_STATS (the statistics kernels of one
 * gptq_hessian_accumulate call), GPTQ_TRACE_FACTOR (one damping attempt's
 * factorisation, H through R), GPTQ_TRACE_CHAIN (each in-block column-chain
 * launch), GPTQ_TRACE_LAZY (each lazy block update), GPTQ_TRACE_OTHER (grid
 * fits, working-copy set-up, output re-layout of a layer).
 * gptq_trace_read waits for the recorded events and writes the summed
 * milliseconds (and the number of launch groups) per phase since the last
 * reset; reset = 1 clears them.  Host-side state guarded by a mutex.
 * ------------------------------------------------------------------------- */
#define GPTQ_TRACE_PHASES 5
enum { GPTQ_TRACE_STATS = 0, GPTQ_TRACE_FACTOR = 1, GPTQ_TRACE_CHAIN = 2,
       GPTQ_TRACE_LAZY = 3, GPTQ_TRACE_OTHER = 4 };
gptq_status gptq_trace_enable(int32_t enable);
gptq_status gptq_trace_read(double* ms /*[host] 5*/, int64_t* launches /*[host] 5, may be NULL*/,
                            int32_t reset);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_MI355_H */
