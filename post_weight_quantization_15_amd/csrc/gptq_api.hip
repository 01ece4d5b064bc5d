// Host runtime behind include/gptq.h: argument validation, workspace carving,
// launch sequencing on the caller's stream and the damping retry.
#include <algorithm>
#include <cmath>
#include <mutex>

#include "common.h"

namespace gptq {
namespace {

// Scratch of the allocation-free Hessian entry point: the split partial
// tiles.  Every GPU the library runs on holds its own copy until the process
// ends.  In host code `scratch` names a host-side stand-in, not the device
// array: its device address is looked up once per device (with that device
// current) and only that address is passed to kernels.
constexpr size_t kScratchBytes = GPTQ_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of `scratch` on the device that runs `st` (the current
// device for the null stream).
gptq_status scratch_address(hipStream_t st, void** out) {
  *out = nullptr;
  int dev = 0;
  if (st)
    GPTQ_CHECK_HIP(hipStreamGetDevice(st, &dev));
  else
    GPTQ_CHECK_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxScratchDevices) return GPTQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    GPTQ_CHECK_HIP(hipGetDevice(&cur));
    if (cur != dev) GPTQ_CHECK_HIP(hipSetDevice(dev));
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) GPTQ_CHECK_HIP(hipSetDevice(cur));
    if (e != hipSuccess || !p) return GPTQ_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GPTQ_OK;
}

constexpr int64_t kMaxDim = 65535;   // grid.y limit of the per-row launches
constexpr int kChainMaxBlock = 128;
constexpr int kLazyBatch = 4;        // chain blocks per lazy (far) update
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

// Groups fitted before the loop (static or caller-given grids) rather than
// refitted in processing order.
bool static_grids(const gptq_params* p) {
  return p->group_size > 0 && (p->static_groups == 1 || p->grid == GPTQ_GRID_FIXED);
}

bool valid_params(const gptq_params* p, int64_t d) {
  if (!p) return false;
  if (!(p->bits == 2 || p->bits == 3 || p->bits == 4 || p->bits == 8)) return false;
  if (!(p->group_size == -1 || p->group_size > 0)) return false;
  if (p->blocksize < 1) return false;
  if (!(p->percdamp >= 0.0f) || !std::isfinite(p->percdamp)) return false;
  if (p->act_order != 0 && p->act_order != 1) return false;
  if (p->grid != GPTQ_GRID_MINMAX && p->grid != GPTQ_GRID_SYMMETRIC &&
      p->grid != GPTQ_GRID_FIXED)
    return false;
  if (p->static_groups != 0 && p->static_groups != 1) return false;
  const bool fixed = p->grid == GPTQ_GRID_FIXED;
  if (fixed != (p->fixed_scales != nullptr) || fixed != (p->fixed_zeros != nullptr))
    return false;
  return static_grids(p) || groups_fit_blocks(d, p->group_size, p->blocksize);
}

// Internal block width of the column loop: the requested block size when it
// fits the chain kernel, else its largest divisor <= 128 that keeps the
// group rule (lazy batching is exact algebra, so any grouping of the same
// updates is the same method).
int internal_block(int64_t d, const gptq_params* p) {
  if (p->blocksize <= kChainMaxBlock) return p->blocksize;
  for (int bi = kChainMaxBlock; bi >= 1; --bi)
    if (p->blocksize % bi == 0 &&
        (static_grids(p) || groups_fit_blocks(d, p->group_size, bi)))
      return bi;
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
  const int tk = trace_begin(st, GPTQ_TRACE_FACTOR);
  if ((s = launch_prep_stats(S, d, n, percdamp, attempt, f, dead, st)) != GPTQ_OK) return s;
  if (attempt == 0 && (s = launch_perm(d, act_order, f, perm, st)) != GPTQ_OK) return s;
  if ((s = launch_build_h(S, d, n, perm, dead, act_order == 0, f, st)) != GPTQ_OK) return s;
  if ((s = launch_factor_inverse(d, f, st)) != GPTQ_OK) return s;
  s = launch_r_to_f32(d, f, R, st);
  trace_end(st, tk);
  return s;
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
                            int32_t* g_idx, float* w_hat, bool ident, hipStream_t st) {
  gptq_status s;
  int tk = trace_begin(st, GPTQ_TRACE_OTHER);
  const int64_t gsize = p->group_size;
  const bool sym = p->grid == GPTQ_GRID_SYMMETRIC;
  const bool stat = static_grids(p);
  const float maxq = static_cast<float>((1 << p->bits) - (sym ? 2 : 1));
  // grids fixed before the loop: given, or fitted on the original weights
  // (the whole row, or the static groups) before dead columns are zeroed
  if (p->grid == GPTQ_GRID_FIXED) {
    const int64_t ng = gsize > 0 ? (d + gsize - 1) / gsize : 1;
    if ((s = launch_grid_in(p->fixed_scales, p->fixed_zeros, m, ng, q.scalesP,
                            q.zerosP, st)) != GPTQ_OK)
      return s;
  } else if (gsize == -1 || stat) {
    if ((s = launch_fit_grids(W, w_dtype, m, d, ldw, gsize == -1 ? d : gsize, maxq,
                              sym, q.scalesP, q.zerosP, st)) != GPTQ_OK)
      return s;
  }
  if ((s = launch_init_work(W, w_dtype, m, d, ldw, pu, du, ident, q.WT, q.pinv, st)) != GPTQ_OK)
    return s;
  const int bi = internal_block(d, p);
  if ((s = launch_rbt(Ru, d, bi, q.RbT, st)) != GPTQ_OK) return s;
  trace_end(st, tk);
  // Lazy batches of nb blocks: each block's chain first applies the batch's
  // earlier residuals to its own columns, and one update per batch carries
  // the whole batch to the columns after it (the same sums regrouped, as
  // lazy batching itself is).  Batches need full 128-column blocks and no
  // dynamic group reaching past its block, whose fit would read columns of
  // the batch that have not received the batch's residuals yet.
  const bool batch = bi == kChainMaxBlock && (gsize == -1 || stat || bi % gsize == 0);
  const int nb = batch ? kLazyBatch : 1;
  ChainArgs a{};
  a.WT = q.WT;
  a.m = m;
  a.d = d;
  a.RL = q.RbT;
  a.bi = bi;
  a.maxq = maxq;
  a.gsize = gsize;
  a.fs = stat ? -1 : (gsize == -1 ? 0 : 1);
  a.sym = sym;
  a.sgn = sym;
  a.cmask = (1 << p->bits) - 1;
  a.perm = pu;
  a.scalesP = q.scalesP;
  a.zerosP = q.zerosP;
  a.codesP = q.codesP;
  a.R = Ru;
  a.Esb = q.E;
  for (int64_t s0 = 0; s0 < d; s0 += int64_t(nb) * bi) {
    int64_t i0 = s0;
    // a batch of full blocks runs in one launch (rows are independent, so
    // each workgroup carries its rows through the batch's blocks in turn)
    a.i0 = s0;
    a.E = q.E;
    a.bw = bi;
    const bool one_launch = nb > 1 && s0 + int64_t(nb) * bi <= d && chain_vec(a);
    for (int j = 0; j < nb && i0 < d; ++j, i0 += bi) {
      a.i0 = i0;
      a.bw = static_cast<int>(std::min<int64_t>(bi, d - i0));
      a.E = q.E + (i0 - s0) * m;
      a.sb0 = s0;
      a.kn = static_cast<int>(i0 - s0);
      a.nblk = one_launch ? nb : 1;
      tk = trace_begin(st, GPTQ_TRACE_CHAIN);
      if ((s = launch_chain(a, st)) != GPTQ_OK) return s;
      trace_end(st, tk);
      if (one_launch) break;
    }
    const int kw = static_cast<int>(std::min<int64_t>(int64_t(nb) * bi, d - s0));
    if (d - s0 - kw > 0) {
      tk = trace_begin(st, GPTQ_TRACE_LAZY);
      if ((s = launch_lazy_update(q.WT, m, d, Ru, s0, kw, q.E, st)) != GPTQ_OK) return s;
      trace_end(st, tk);
    }
  }
  tk = trace_begin(st, GPTQ_TRACE_OTHER);
  s = launch_outputs(m, d, p->bits, static_cast<int>(gsize), sym, stat, q.codesP,
                     q.scalesP, q.zerosP, q.pinv, q.codesO, qweight, scales, zeros,
                     g_idx, w_hat, st);
  trace_end(st, tk);
  return s;
}

constexpr int64_t kMaxStackTokens = int64_t(65535) * 8;   // dequant grid.y

struct StackWs {
  float* S;
  void* hws;
  size_t hws_bytes;
  void* qws;
  size_t qws_bytes;
  float* w_hat;
  uint16_t* buf[2];
  double* part;
  double* errs;
};

bool valid_stack(const gptq_stack_layer* L, int32_t nl, int64_t n_tok) {
  if (!L || nl < 1 || n_tok < 1 || n_tok > kMaxStackTokens) return false;
  for (int32_t l = 0; l < nl; ++l) {
    const gptq_stack_layer& a = L[l];
    if (!a.W || a.m <= 0 || a.d <= 0 || a.m > kMaxDim || a.d > kMaxDim || a.ldw < a.d ||
        !valid_dtype(a.w_dtype) || !valid_params(&a.params, a.d) || !a.qweight ||
        !a.scales || !a.zeros || !a.g_idx)
      return false;
    if (l > 0 && a.d != L[l - 1].m) return false;
  }
  return true;
}

StackWs carve_stack_ws(Carver& c, const gptq_stack_layer* L, int32_t nl, int64_t n) {
  int64_t dmax = 0, mmax = 0, wmax = 0;
  size_t hb = 0, qb = 0, pc = 0;
  for (int32_t l = 0; l < nl; ++l) {
    dmax = std::max(dmax, L[l].d);
    mmax = std::max(mmax, L[l].m);
    wmax = std::max(wmax, L[l].m * L[l].d);
    hb = std::max(hb, hessian_ws_bytes(L[l].d, n));
    Carver q(nullptr);
    carve_quant_ws(q, L[l].m, L[l].d, &L[l].params, true);
    qb = std::max(qb, q.bytes());
    pc = std::max(pc, layer_error_part_count(L[l].m, L[l].d));
  }
  StackWs w{};
  w.S = c.take<float>(size_t(dmax) * size_t(dmax));
  w.hws = c.take<char>(hb);
  w.hws_bytes = hb;
  w.qws = c.take<char>(qb);
  w.qws_bytes = qb;
  w.w_hat = c.take<float>(size_t(wmax));
  w.buf[0] = c.take<uint16_t>(size_t(n) * size_t(mmax));
  w.buf[1] = c.take<uint16_t>(size_t(n) * size_t(mmax));
  w.part = c.take<double>(pc);
  w.errs = c.take<double>(size_t(nl));
  return w;
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
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int tk = trace_begin(st, GPTQ_TRACE_STATS);
  const gptq_status s = launch_hessian(S, d, X, x_dtype, n_tok, ldx, ws, st);
  trace_end(st, tk);
  return s;
}

gptq_status gptq_hessian_accumulate_noalloc(float* S, int64_t d, const void* X,
                                            gptq_dtype x_dtype, int64_t n_tok,
                                            int64_t ldx, void* stream) {
  if (!S || d <= 0 || d > kMaxDim || n_tok < 0 || ldx < d || !valid_dtype(x_dtype))
    return GPTQ_ERR_INVALID_ARG;
  if (n_tok > 0 && !X) return GPTQ_ERR_INVALID_ARG;
  const double cap = static_cast<double>(kScratchBytes);
  // the token split is planned within the scratch size, so no size needs
  // more; the check guards the plan itself
  if (hessian_ws_bytes(d, n_tok, cap) > kScratchBytes) return GPTQ_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  gptq_status s;
  if ((s = scratch_address(st, &ws)) != GPTQ_OK) return s;
  const int tk = trace_begin(st, GPTQ_TRACE_STATS);
  s = launch_hessian(S, d, X, x_dtype, n_tok, ldx, ws, st, cap);
  trace_end(st, tk);
  return s;
}

gptq_status gptq_dequant_matmul(const void* X, gptq_dtype x_dtype, int64_t n,
                                int64_t d, int64_t ldx, const uint32_t* qweight,
                                const void* scales, gptq_dtype scale_dtype,
                                const uint8_t* zeros,
                                const int32_t* g_idx, int64_t m, int32_t bits,
                                int32_t group_size, int32_t signed_codes,
                                float* Y, int64_t ldy, void* stream) {
  if (x_dtype != GPTQ_BF16 || (scale_dtype != GPTQ_F32 && scale_dtype != GPTQ_F16) ||
      n < 0 || d <= 0 || m <= 0 || d > kMaxDim ||
      ldx < d || ldy < m || !(bits == 2 || bits == 3 || bits == 4 || bits == 8) ||
      !(group_size == -1 || group_size > 0) ||
      (signed_codes != 0 && signed_codes != 1))
    return GPTQ_ERR_INVALID_ARG;
  if (n > 0 && (!X || !qweight || !scales || !zeros || !g_idx || !Y))
    return GPTQ_ERR_INVALID_ARG;
  const int64_t ng = group_size > 0 ? (d + group_size - 1) / group_size : 1;
  if (n > int64_t(65535) * 8) return GPTQ_ERR_INVALID_ARG;
  return launch_dequant_matmul(static_cast<const uint16_t*>(X), ldx, n, qweight, m,
                               d, bits, scales, scale_dtype == GPTQ_F16, zeros, ng, g_idx,
                               signed_codes, Y, ldy, 0, 0, static_cast<hipStream_t>(stream));
}

size_t gptq_stack_workspace_bytes(const gptq_stack_layer* layers, int32_t n_layers,
                                  int64_t n_tok) {
  if (!layers || n_layers < 1 || n_tok < 1) return 0;
  for (int32_t l = 0; l < n_layers; ++l) {
    if (layers[l].m <= 0 || layers[l].d <= 0 || !valid_params(&layers[l].params, layers[l].d))
      return 0;
  }
  Carver c(nullptr);
  carve_stack_ws(c, layers, n_layers, n_tok);
  return c.bytes();
}

gptq_status gptq_quantize_stack(const gptq_stack_layer* layers, int32_t n_layers,
                                const void* X_in, int64_t n_tok, int32_t activation,
                                void* X_out, double* layer_err, void* ws,
                                size_t ws_bytes, void* stream) {
  if (!valid_stack(layers, n_layers, n_tok) || !X_in || !X_out ||
      activation < GPTQ_ACT_NONE || activation > GPTQ_ACT_SILU)
    return GPTQ_ERR_INVALID_ARG;
  Carver c(ws);
  const StackWs w = carve_stack_ws(c, layers, n_layers, n_tok);
  if (!ws || ws_bytes < c.bytes()) return GPTQ_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  gptq_status s;
  for (int32_t l = 0; l < n_layers; ++l) {
    const gptq_stack_layer& a = layers[l];
    const void* Xc = l == 0 ? X_in : w.buf[(l - 1) & 1];
    void* Xn = l == n_layers - 1 ? X_out : w.buf[l & 1];
    // statistics of this layer's inputs (the previous quantized layer's
    // outputs after the activation)
    if ((s = launch_zero_f32(w.S, a.d * a.d, st)) != GPTQ_OK) return s;
    if ((s = launch_hessian(w.S, a.d, Xc, GPTQ_BF16, n_tok, a.d, w.hws, st)) != GPTQ_OK)
      return s;
    if ((s = gptq_quantize_layer(a.W, a.w_dtype, a.m, a.d, a.ldw, w.S, n_tok, &a.params,
                                 nullptr, nullptr, nullptr, a.qweight, a.scales, a.zeros,
                                 a.g_idx, w.w_hat, w.qws, w.qws_bytes, stream)) != GPTQ_OK)
      return s;
    if ((s = launch_layer_error(a.W, a.w_dtype, a.ldw, w.w_hat, w.S, a.m, a.d, n_tok,
                                w.part, w.errs + l, st)) != GPTQ_OK)
      return s;
    const int64_t ng = a.params.group_size > 0 ? (a.d + a.params.group_size - 1) / a.params.group_size : 1;
    if ((s = launch_dequant_matmul(static_cast<const uint16_t*>(Xc), a.d, n_tok, a.qweight,
                                   a.m, a.d, a.params.bits, a.scales, 0, a.zeros, ng, a.g_idx,
                                   a.params.grid == GPTQ_GRID_SYMMETRIC, Xn, a.m, 1,
                                   activation, st)) != GPTQ_OK)
      return s;
  }
  if (layer_err)
    GPTQ_CHECK_HIP(hipMemcpyAsync(layer_err, w.errs, sizeof(double) * size_t(n_layers),
                                  hipMemcpyDeviceToHost, st));
  GPTQ_CHECK_HIP(hipStreamSynchronize(st));
  return GPTQ_OK;
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
                           scales, zeros, g_idx, w_hat, false, st);
  // The whole layer is enqueued behind each damping attempt and the flag read
  // once at the end; a failed attempt's outputs are recomputed.
  double damp = 0.0;
  for (int attempt = 0; attempt <= kMaxRetries; ++attempt) {
    gptq_status s;
    if ((s = enqueue_factor(S, n, d, p->percdamp, p->act_order, attempt, q.R,
                            q.perm, q.dead, q.f, st)) != GPTQ_OK)
      return s;
    // the order computed here is the identity without act-order
    if ((s = enqueue_columns(W, w_dtype, m, d, ldw, p, q.R, q.perm, q.dead, q,
                             qweight, scales, zeros, g_idx, w_hat, p->act_order == 0,
                             st)) != GPTQ_OK)
      return s;
    bool ok = false;
    if ((s = read_factor_outcome(q.f, st, &ok, &damp)) != GPTQ_OK) return s;
    if (ok) return GPTQ_OK;
  }
  return GPTQ_ERR_NOT_SPD;
}

}  // extern "C"
