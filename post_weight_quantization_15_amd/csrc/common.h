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

// Hessian: S += X^T X.  Partial sums for split tokens live in `ws`; the
// token split is planned so that they take at most max_part bytes (the
// same bound must be passed to both calls).
constexpr double kHessianMaxPartBytes = 16.0 * (1 << 30);
size_t hessian_ws_bytes(int64_t d, int64_t n_tok,
                        double max_part = kHessianMaxPartBytes);
gptq_status launch_hessian(float* S, int64_t d, const void* X, gptq_dtype dt,
                           int64_t n_tok, int64_t ldx, void* ws,
                           hipStream_t st,
                           double max_part = kHessianMaxPartBytes);

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
                           const int32_t* perm, const uint8_t* dead, bool ident,
                           const FactorWs& f, hipStream_t st);
// U (in H) and R = U^-1 (in R), the inverse partly beside the factor on a
// second stream; the caller's stream has waited for it on return.
gptq_status launch_factor_inverse(int64_t d, const FactorWs& f, hipStream_t st);
gptq_status launch_r_to_f32(int64_t d, const FactorWs& f, float* R,
                            hipStream_t st);

// Quantization pieces.
// Grids fitted on the ORIGINAL weights before the loop: groups of g
// contiguous columns (g = d: the whole-row grid), scale / zero at [G][r].
gptq_status launch_fit_grids(const void* W, gptq_dtype dt, int64_t m, int64_t d,
                             int64_t ldw, int64_t g, float maxq, int sym,
                             float* scalesP, uint8_t* zerosP, hipStream_t st);
// A caller-given grid [m, n_g] into the [n_g][m] layout.
gptq_status launch_grid_in(const float* s_in, const uint8_t* z_in, int64_t m,
                           int64_t ng, float* scalesP, uint8_t* zerosP,
                           hipStream_t st);
gptq_status launch_init_work(const void* W, gptq_dtype dt, int64_t m,
                             int64_t d, int64_t ldw, const int32_t* perm,
                             const uint8_t* dead, bool ident, float* WT,
                             int32_t* pinv, hipStream_t st);
// RL[blk] = R's diagonal block blk (blocks of bi <= 128 columns) in the chain
// kernel's lane order, 128 x 128 floats per block.
gptq_status launch_rbt(const float* R, int64_t d, int bi, float* RL,
                       hipStream_t st);
// Block [i0, i0 + bw) of the column loop (bw <= bi <= 128).  scalesP/zerosP
// are [n_g][m] (group major); for the whole-row grid row 0 holds the row
// grids.  Writes the block's codes and its residuals E [bw][m].  The block
// belongs to a lazy batch starting at column sb0 (a multiple of 32 columns
// before i0, kn = i0 - sb0) whose earlier blocks' residuals Esb [kn][m] have
// not been applied to WT yet: the kernel applies them to its own columns
// first (R: fp32 [d][d]).
struct ChainArgs {
  float* WT;
  int64_t m, d;
  const float* RL;
  int64_t i0;
  int bw, bi;
  float maxq;          // top unsigned code (2^b - 1, or 2^b - 2 symmetric)
  int64_t gsize;       // group size (dynamic or static), -1 for the row grid
  int fs;              // 0: row grid; -1: static per-column grids; 1: dynamic
  int sym;             // dynamic refits use the symmetric grid
  int sgn;             // store signed codes c - z (low bits)
  int cmask;           // 2^b - 1
  const int32_t* perm; // processing position -> original column
  float* scalesP;
  uint8_t* zerosP;
  uint8_t* codesP;
  float* E;
  const float* R;
  int64_t sb0;
  int kn;
  const float* Esb;
  int nblk = 1;        // full blocks i0, i0 + bi, ... run by one launch (1 or 2)
};
// The chain's 16-byte global accesses need these alignments.
inline bool chain_vec(const ChainArgs& a) {
  return a.m % 4 == 0 && reinterpret_cast<uintptr_t>(a.WT) % 16 == 0 &&
         reinterpret_cast<uintptr_t>(a.E) % 16 == 0 &&
         reinterpret_cast<uintptr_t>(a.codesP) % 4 == 0;
}
gptq_status launch_chain(const ChainArgs& a, hipStream_t st);
// per-variant launchers (one instantiation unit each)
gptq_status launch_chain_row(const ChainArgs& a, hipStream_t st);
gptq_status launch_chain_static(const ChainArgs& a, hipStream_t st);
gptq_status launch_chain_g1(const ChainArgs& a, hipStream_t st);
gptq_status launch_chain_g8(const ChainArgs& a, hipStream_t st);
gptq_status launch_chain_g64(const ChainArgs& a, hipStream_t st);
gptq_status launch_chain_g128(const ChainArgs& a, hipStream_t st);
// WT[:, i0 + bw:] -= E^T R[i0:i0 + bw, i0 + bw:] for a lazy batch of bw <= 512
// columns; E [bw][m] with room for its rows padded to the product's k steps.
gptq_status launch_lazy_update(float* WT, int64_t m, int64_t d, const float* R,
                               int64_t i0, int bw, float* E,
                               hipStream_t st);
// Outputs in the original column order.  sgn: codes are signed (zeros
// written as 0, w_hat = Delta * code); stat: static groups (g_idx = c / g).
gptq_status launch_outputs(int64_t m, int64_t d, int bits, int gsize, int sgn,
                           int stat, const uint8_t* codesP,
                           const float* scalesP, const uint8_t* zerosP,
                           const int32_t* pinv, uint8_t* codesO,
                           uint32_t* qweight, float* scales, uint8_t* zeros,
                           int32_t* g_idx, float* w_hat, hipStream_t st);

// Y[k][r] = sum_c X[k][c] W_hat[r][c] for bf16 activations X [n][ldx] and
// the stored format (qweight [m][ceil(d bits / 32)], scales / zeros
// [m][ng], g_idx [d]); Y fp32 [n][ldy], or (out_bf16) bf16 after the
// activation act (0 none, 1 ReLU, 2 SiLU).  n <= 524280.
gptq_status launch_dequant_matmul(const uint16_t* X, int64_t ldx, int64_t n,
                                  const uint32_t* qweight, int64_t m, int64_t d,
                                  int bits, const void* scales, int scale_f16,
                                  const uint8_t* zeros, int64_t ng,
                                  const int32_t* g_idx, int sgn, void* Y,
                                  int64_t ldy, int out_bf16, int act,
                                  hipStream_t st);

// Tracing (trace.hip): per-phase event pairs on the caller's stream while
// enabled.  trace_begin returns a token (-1 when off) for trace_end.
constexpr int kTracePhases = GPTQ_TRACE_PHASES;
bool trace_on();
int trace_begin(hipStream_t st, int phase);
void trace_end(hipStream_t st, int token);

// Layer error (1/n) sum_r (W - W_hat)_r^T S (W - W_hat)_r into *out (fp64);
// part: layer_error_part_count(m, d) doubles of scratch.
size_t layer_error_part_count(int64_t m, int64_t d);
gptq_status launch_layer_error(const void* W, gptq_dtype wdt, int64_t ldw,
                               const float* W_hat, const float* S, int64_t m,
                               int64_t d, int64_t n, double* part, double* out,
                               hipStream_t st);
gptq_status launch_zero_f32(float* p, int64_t n, hipStream_t st);

}  // namespace gptq
