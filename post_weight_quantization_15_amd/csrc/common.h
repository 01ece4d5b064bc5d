// Shared helpers of the gfx950 GPTQ library: vector types, workspace carving,
// launch checking and the declarations of the per-file launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/gptq.h"

namespace gptq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr size_t kAlign = 256;

inline size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

// Carves typed sub-buffers out of the caller's workspace.  With base == NULL
// it only measures (used by the *_workspace_bytes queries).
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <class T>
  T* take(size_t count) {
    off = align_up(off);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
  size_t bytes() const { return align_up(off); }
};

#define GPTQ_CHECK_LAUNCH()                         \
  do {                                              \
    if (hipGetLastError() != hipSuccess) return GPTQ_ERR_HIP; \
  } while (0)

#define GPTQ_CHECK_HIP(call)                        \
  do {                                              \
    if ((call) != hipSuccess) return GPTQ_ERR_HIP;  \
  } while (0)

// ---------------------------------------------------------------------------
// Launchers (each returns GPTQ_OK or GPTQ_ERR_HIP; arguments pre-validated)
// ---------------------------------------------------------------------------

// Hessian: S += X^T X.  Partial sums for split tokens live in `ws`.
size_t hessian_ws_bytes(int64_t d, int64_t n_tok);
gptq_status launch_hessian(float* S, int64_t d, const void* X, gptq_dtype dt,
                           int64_t n_tok, int64_t ldx, void* ws,
                           hipStream_t st);

// Factor pieces (fp64).
struct FactorWs {
  double* H;      // [d, d] damped, permuted Hessian; overwritten by U (upper)
  double* R;      // [d, d] U^-1 (upper)
  double* T;      // scratch for the triangular inverse (caller's stream)
  double* Tb;     // the same, for the part on the second stream
  double* keys;   // [d] diag(H) after the dead fix
  double* damp;   // [1] damping used
  int* flag;      // [1] set when a pivot is not positive
};
size_t factor_ws_bytes(int64_t d);
FactorWs carve_factor_ws(Carver& c, int64_t d);
gptq_status launch_prep_stats(const float* S, int64_t d, int64_t n,
                              double percdamp, int attempt, const FactorWs& f,
                              uint8_t* dead, hipStream_t st);
gptq_status launch_perm(int64_t d, int act_order, const FactorWs& f,
                        int32_t* perm, hipStream_t st);
gptq_status launch_build_h(const float* S, int64_t d, int64_t n,
                           const int32_t* perm, const uint8_t* dead,
                           const FactorWs& f, hipStream_t st);
// U (in H) and R = U^-1 (in R), the inverse partly beside the factor on a
// second stream; the caller's stream has waited for it on return.
gptq_status launch_factor_inverse(int64_t d, const FactorWs& f, hipStream_t st);
gptq_status launch_r_to_f32(int64_t d, const FactorWs& f, float* R,
                            hipStream_t st);

// Quantization pieces.
// Whole-row grid (group_size -1): scale[r], zero[r] of the original row r.
gptq_status launch_fit_rows(const void* W, gptq_dtype dt, int64_t m, int64_t d,
                            int64_t ldw, int bits, float* scale, uint8_t* zero,
                            hipStream_t st);
gptq_status launch_init_work(const void* W, gptq_dtype dt, int64_t m,
                             int64_t d, int64_t ldw, const int32_t* perm,
                             const uint8_t* dead, float* WT, int32_t* pinv,
                             hipStream_t st);
// RL[blk] = R's diagonal block blk (blocks of bi <= 128 columns) in the chain
// kernel's lane order, 128 x 128 floats per block.
gptq_status launch_rbt(const float* R, int64_t d, int bi, float* RL,
                       hipStream_t st);
// Block [i0, i0 + bw) of the column loop (bw <= bi <= 128).  scalesP/zerosP
// are [n_g][m] (processing-group major); for group_size -1 row 0 holds the
// row grids.  Writes the block's codes and its residuals E [bw][m].  The
// block belongs to a lazy batch starting at column sb0 (a multiple of 32
// columns before i0) whose earlier blocks' residuals Esb [i0 - sb0][m] have
// not been applied to WT yet: the kernel applies them to its own columns
// first (R: fp32 [d][d]).
gptq_status launch_chain(float* WT, int64_t m, int64_t d, const float* RL,
                         int64_t i0, int bw, int bi, int bits, int64_t gsize,
                         float* scalesP, uint8_t* zerosP, uint8_t* codesP,
                         float* E, const float* R, int64_t sb0, const float* Esb,
                         hipStream_t st);
// WT[:, i0 + bw:] -= E^T R[i0:i0 + bw, i0 + bw:] for a lazy batch of bw <= 512
// columns; E [bw][m] with room for its rows padded to the product's k steps.
gptq_status launch_lazy_update(float* WT, int64_t m, int64_t d, const float* R,
                               int64_t i0, int bw, float* E,
                               hipStream_t st);
gptq_status launch_outputs(int64_t m, int64_t d, int bits, int gsize,
                           const uint8_t* codesP, const float* scalesP,
                           const uint8_t* zerosP, const int32_t* pinv,
                           uint8_t* codesO, uint32_t* qweight, float* scales,
                           uint8_t* zeros, int32_t* g_idx, float* w_hat,
                           hipStream_t st);

}  // namespace gptq
