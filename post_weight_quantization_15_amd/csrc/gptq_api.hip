// Host runtime behind include/gptq.h: argument validation, workspace carving,
// launch sequencing on the caller's stream and the damping retry.
#include <algorithm>
#include <cmath>

#include "common.h"

namespace gptq {
namespace {

constexpr int64_t kMaxDim = 65535;   // grid.y limit of the per-row launches
constexpr int kChainMaxBlock = 128;
constexpr int kLazyBatch = 2;        // chain blocks per lazy (far) update
constexpr int kMaxRetries = 5;

bool valid_dtype(gptq_dtype t) { return t == GPTQ_BF16 || t == GPTQ_F32; }

// Every dynamic group that starts inside a block of `b` columns (blocks
// start at multiples of b) must end inside that block.
bool groups_fit_blocks(int64_t d, int64_t g, int64_t b) {
  if (g == -1) return true;
  for (int64_t j = 0; j < d; j += g) {
    const int64_t off = j % b;
    if (off != 0 && off + std::min<int64_t>(g, d - j) > b) return false;
  }
  return true;
}

bool valid_params(const gptq_params* p, int64_t d) {
  if (!p) return false;
  if (!(p->bits == 2 || p->bits == 3 || p->bits == 4 || p->bits == 8)) return false;
  if (!(p->group_size == -1 || p->group_size > 0)) return false;
  if (p->blocksize < 1) return false;
  if (!(p->percdamp >= 0.0f) || !std::isfinite(p->percdamp)) return false;
  if (p->act_order != 0 && p->act_order != 1) return false;
  return groups_fit_blocks(d, p->group_size, p->blocksize);
}

// Internal block width of the column loop: the requested block size when it
// fits the chain kernel, else its largest divisor <= 128 that keeps the
// group rule (lazy batching is exact algebra, so any grouping of the same
// updates is the same method).
int internal_block(int64_t d, const gptq_params* p) {
  if (p->blocksize <= kChainMaxBlock) return p->blocksize;
  for (int bi = kChainMaxBlock; bi >= 1; --bi)
    if (p->blocksize % bi == 0 && groups_fit_blocks(d, p->group_size, bi)) return bi;
  return 1;
}

struct QuantWs {
  float* WT;
  float* E;
  uint8_t* codesP;
  uint8_t* codesO;
  float* scalesP;
  uint8_t* zerosP;
  int32_t* pinv;
  float* RbT;
  float* R;
  int32_t* perm;
  uint8_t* dead;
  FactorWs f;
};

QuantWs carve_quant_ws(Carver& c, int64_t m, int64_t d, const gptq_params* p,
                       bool factor_inside) {
  QuantWs q{};
  const int64_t ng = p->group_size > 0 ? (d + p->group_size - 1) / p->group_size : 1;
  const int bi = internal_block(d, p);
  const int64_t nblk = (d + bi - 1) / bi;
  q.WT = c.take<float>(size_t(d) * size_t(m));
  q.E = c.take<float>(size_t(kLazyBatch) * size_t(kChainMaxBlock) * size_t(m));
  q.codesP = c.take<uint8_t>(size_t(d) * size_t(m));
  q.codesO = c.take<uint8_t>(size_t(d) * size_t(m));
  q.scalesP = c.take<float>(size_t(ng) * size_t(m));
  q.zerosP = c.take<uint8_t>(size_t(ng) * size_t(m));
  q.pinv = c.take<int32_t>(size_t(d));
  q.RbT = c.take<float>(size_t(nblk) * size_t(kChainMaxBlock) * size_t(kChainMaxBlock));
  if (factor_inside) {
    q.R = c.take<float>(size_t(d) * size_t(d));
    q.perm = c.take<int32_t>(size_t(d));
    q.dead = c.take<uint8_t>(size_t(d));
    q.f = carve_factor_ws(c, d);
  }
  return q;
}

// One damping attempt of the factor: enqueues everything up to R (fp32).
// The Cholesky raises f.flag on a non-positive pivot; the kernels after it
// do plain arithmetic (no value-dependent addressing), so they may run on a
// failed factor and the caller reads the flag once, after the whole
// attempt's work -- the factor and whatever consumes R -- is enqueued.
gptq_status enqueue_factor(const float* S, int64_t n, int64_t d, float percdamp,
                           int act_order, int attempt, float* R, int32_t* perm,
                           uint8_t* dead, const FactorWs& f, hipStream_t st) {
  gptq_status s;
  if ((s = launch_prep_stats(S, d, n, percdamp, attempt, f, dead, st)) != GPTQ_OK) return s;
  if (attempt == 0 && (s = launch_perm(d, act_order, f, perm, st)) != GPTQ_OK) return s;
  if ((s = launch_build_h(S, d, n, perm, dead, f, st)) != GPTQ_OK) return s;
  if ((s = launch_factor_inverse(d, f, st)) != GPTQ_OK) return s;
  return launch_r_to_f32(d, f, R, st);
}

// Waits for the stream and reads the attempt's outcome.
gptq_status read_factor_outcome(const FactorWs& f, hipStream_t st, bool* ok,
                                double* damp) {
  int flag = 0;
  GPTQ_CHECK_HIP(hipMemcpyAsync(&flag, f.flag, sizeof(int), hipMemcpyDeviceToHost, st));
  GPTQ_CHECK_HIP(hipMemcpyAsync(damp, f.damp, sizeof(double), hipMemcpyDeviceToHost, st));
  GPTQ_CHECK_HIP(hipStreamSynchronize(st));
  *ok = flag == 0;
  return GPTQ_OK;
}

gptq_status run_factor(const float* S, int64_t n, int64_t d, float percdamp,
                       int act_order, float* R, int32_t* perm, uint8_t* dead,
                       float* damp_used, const FactorWs& f, hipStream_t st) {
  double damp = 0.0;
  for (int attempt = 0; attempt <= kMaxRetries; ++attempt) {
    gptq_status s;
    if ((s = enqueue_factor(S, n, d, percdamp, act_order, attempt, R, perm, dead, f, st)) != GPTQ_OK)
      return s;
    bool ok = false;
    if ((s = read_factor_outcome(f, st, &ok, &damp)) != GPTQ_OK) return s;
    if (ok) {
      if (damp_used) *damp_used = static_cast<float>(damp);
      return GPTQ_OK;
    }
  }
  if (damp_used) *damp_used = static_cast<float>(damp);
  return GPTQ_ERR_NOT_SPD;
}

// The column loop and the outputs for one layer, given the factor.
gptq_status enqueue_columns(const void* W, gptq_dtype w_dtype, int64_t m,
                            int64_t d, int64_t ldw, const gptq_params* p,
                            const float* Ru, const int32_t* pu,
                            const uint8_t* du, const QuantWs& q,
                            uint32_t* qweight, float* scales, uint8_t* zeros,
                            int32_t* g_idx, float* w_hat, hipStream_t st) {
  gptq_status s;
  const int64_t gsize = p->group_size;
  // whole-row grid on the original row, before dead columns are zeroed
  if (gsize == -1 &&
      (s = launch_fit_rows(W, w_dtype, m, d, ldw, p->bits, q.scalesP, q.zerosP, st)) != GPTQ_OK)
    return s;
  if ((s = launch_init_work(W, w_dtype, m, d, ldw, pu, du, q.WT, q.pinv, st)) != GPTQ_OK)
    return s;
  const int bi = internal_block(d, p);
  if ((s = launch_rbt(Ru, d, bi, q.RbT, st)) != GPTQ_OK) return s;
  // Lazy batches of nb blocks: each block's chain first applies the batch's
  // earlier residuals to its own columns, and one update per batch carries
  // the whole batch to the columns after it (the same sums regrouped, as
  // lazy batching itself is).  Batches need full 128-column blocks and no
  // group reaching past its block, whose fit would read columns of the
  // batch that have not received the batch's residuals yet.
  const bool batch = bi == kChainMaxBlock && (gsize == -1 || bi % gsize == 0);
  const int nb = batch ? kLazyBatch : 1;
  for (int64_t s0 = 0; s0 < d; s0 += int64_t(nb) * bi) {
    int64_t i0 = s0;
    for (int j = 0; j < nb && i0 < d; ++j, i0 += bi) {
      const int bw = static_cast<int>(std::min<int64_t>(bi, d - i0));
      if ((s = launch_chain(q.WT, m, d, q.RbT, i0, bw, bi, p->bits, gsize,
                            q.scalesP, q.zerosP, q.codesP, q.E + (i0 - s0) * m, Ru,
                            s0, q.E, st)) != GPTQ_OK)
        return s;
    }
    const int kw = static_cast<int>(std::min<int64_t>(int64_t(nb) * bi, d - s0));
    if ((s = launch_lazy_update(q.WT, m, d, Ru, s0, kw, q.E, st)) != GPTQ_OK)
      return s;
  }
  return launch_outputs(m, d, p->bits, static_cast<int>(gsize), q.codesP,
                        q.scalesP, q.zerosP, q.pinv, q.codesO, qweight, scales,
                        zeros, g_idx, w_hat, st);
}

}  // namespace
}  // namespace gptq

using namespace gptq;

extern "C" {

const char* gptq_status_string(gptq_status s) {
  switch (s) {
    case GPTQ_OK: return "ok";
    case GPTQ_ERR_INVALID_ARG: return "invalid argument";
    case GPTQ_ERR_NOT_SPD: return "damped Hessian not positive definite";
    case GPTQ_ERR_WORKSPACE: return "workspace too small";
    case GPTQ_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

size_t gptq_hessian_workspace_bytes(int64_t d, int64_t n_tok) {
  if (d <= 0 || n_tok < 0) return 0;
  return hessian_ws_bytes(d, n_tok);
}

gptq_status gptq_hessian_accumulate(float* S, int64_t d, const void* X,
                                    gptq_dtype x_dtype, int64_t n_tok,
                                    int64_t ldx, void* ws, size_t ws_bytes,
                                    void* stream) {
  if (!S || d <= 0 || d > kMaxDim || n_tok < 0 || ldx < d || !valid_dtype(x_dtype))
    return GPTQ_ERR_INVALID_ARG;
  if (n_tok > 0 && !X) return GPTQ_ERR_INVALID_ARG;
  const size_t need = hessian_ws_bytes(d, n_tok);
  if (ws_bytes < need || (need > 0 && !ws)) return GPTQ_ERR_WORKSPACE;
  return launch_hessian(S, d, X, x_dtype, n_tok, ldx, ws,
                        static_cast<hipStream_t>(stream));
}

size_t gptq_factor_workspace_bytes(int64_t d) {
  if (d <= 0) return 0;
  return factor_ws_bytes(d);
}

gptq_status gptq_cholesky_inverse(const float* S, int64_t n, int64_t d,
                                  float percdamp, int32_t act_order, float* R,
                                  int32_t* perm, uint8_t* dead,
                                  float* damp_used, void* ws, size_t ws_bytes,
                                  void* stream) {
  if (!S || !R || !perm || !dead || n <= 0 || d <= 0 || d > kMaxDim ||
      !(percdamp >= 0.0f) || !std::isfinite(percdamp) ||
      (act_order != 0 && act_order != 1))
    return GPTQ_ERR_INVALID_ARG;
  Carver c(ws);
  const FactorWs f = carve_factor_ws(c, d);
  if (!ws || ws_bytes < c.bytes()) return GPTQ_ERR_WORKSPACE;
  return run_factor(S, n, d, percdamp, act_order, R, perm, dead, damp_used, f,
                    static_cast<hipStream_t>(stream));
}

size_t gptq_workspace_bytes(int64_t m, int64_t d, const gptq_params* p,
                            int32_t factor_inside) {
  if (m <= 0 || d <= 0 || !valid_params(p, d)) return 0;
  Carver c(nullptr);
  carve_quant_ws(c, m, d, p, factor_inside != 0);
  return c.bytes();
}

gptq_status gptq_quantize_layer(const void* W, gptq_dtype w_dtype, int64_t m,
                                int64_t d, int64_t ldw, const float* S,
                                int64_t n, const gptq_params* p,
                                const float* R, const int32_t* perm,
                                const uint8_t* dead, uint32_t* qweight,
                                float* scales, uint8_t* zeros, int32_t* g_idx,
                                float* w_hat, void* ws, size_t ws_bytes,
                                void* stream) {
  if (!W || m <= 0 || d <= 0 || m > kMaxDim || d > kMaxDim || ldw < d ||
      !valid_dtype(w_dtype) || !valid_params(p, d) || !qweight || !scales ||
      !zeros || !g_idx)
    return GPTQ_ERR_INVALID_ARG;
  const int given = (R != nullptr) + (perm != nullptr) + (dead != nullptr);
  if (given != 0 && given != 3) return GPTQ_ERR_INVALID_ARG;
  const bool factor_inside = given == 0;
  if (factor_inside && (!S || n <= 0)) return GPTQ_ERR_INVALID_ARG;
  Carver c(ws);
  QuantWs q = carve_quant_ws(c, m, d, p, factor_inside);
  if (!ws || ws_bytes < c.bytes()) return GPTQ_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!factor_inside)
    return enqueue_columns(W, w_dtype, m, d, ldw, p, R, perm, dead, q, qweight,
                           scales, zeros, g_idx, w_hat, st);
  // The whole layer is enqueued behind each damping attempt and the flag read
  // once at the end; a failed attempt's outputs are recomputed.
  double damp = 0.0;
  for (int attempt = 0; attempt <= kMaxRetries; ++attempt) {
    gptq_status s;
    if ((s = enqueue_factor(S, n, d, p->percdamp, p->act_order, attempt, q.R,
                            q.perm, q.dead, q.f, st)) != GPTQ_OK)
      return s;
    if ((s = enqueue_columns(W, w_dtype, m, d, ldw, p, q.R, q.perm, q.dead, q,
                             qweight, scales, zeros, g_idx, w_hat, st)) != GPTQ_OK)
      return s;
    bool ok = false;
    if ((s = read_factor_outcome(q.f, st, &ok, &damp)) != GPTQ_OK) return s;
    if (ok) return GPTQ_OK;
  }
  return GPTQ_ERR_NOT_SPD;
}

}  // extern "C"
