// Pre-processing and factorisation of the damped Hessian, in fp64.
//
// [derivation] section 10, steps 5-6: H = (2/N) S; never-seen features get
// H_jj = 1 (their weights are zeroed later); act-order = descending diag(H);
// damp = max(percdamp * mean diag H, eps); R = upper Cholesky factor of
// (H + damp I)^-1 so that R^T R = H^-1 (eq. (37)), whose tails hold every
// conditional inverse the column loop needs (eq. (40)).
//
// Route taken here: H = U U^T with U upper triangular ("reverse" Cholesky,
// the lower Cholesky factor of H with its index order reversed), then
// R = U^-1: R is upper with a positive diagonal and R^T R = U^-T U^-1 = H^-1,
// so by uniqueness it is the factor the pages build (chol -> invert ->
// chol_upper), with one factorisation instead of two.
//
// Blocked right-looking, from the last 64-column block to the first:
//   1. factor the diagonal block A_KK = U_KK U_KK^T in LDS;
//   2. panel: U_iK = A_iK U_KK^-T for every row i above the block;
//   3. trailing update A_ij -= U_iK U_jK^T (upper tiles only).
// Steps 1-2 are one kernel: every workgroup refactors the 64x64 diagonal
// block in LDS (cheap, avoids a launch) and then solves its own rows.
// U_KK^-1 for every diagonal block is then formed in parallel, and the
// off-diagonal blocks of R come from R_12 = -R_11 U_12 R_22 applied level by
// level (block size 64, 128, 256, ...).
#include <algorithm>
#include <cmath>

#include "common.h"

namespace gptq {
namespace {

constexpr int kNb = 64;          // diagonal block / panel width
constexpr double kEpsFloor = 1.1920928955078125e-07;   // 2^-23

// ---------------------------------------------------------------------------
// Statistics, permutation, damped permuted H
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(1024) void prep_stats_kernel(
    const float* __restrict__ S, int64_t d, int64_t n, double percdamp,
    int attempt, double* __restrict__ keys, double* __restrict__ damp_out,
    uint8_t* __restrict__ dead) {
  __shared__ double red[1024];
  const double scale = 2.0 / double(n);
  double sum = 0.0;
  for (int64_t j = threadIdx.x; j < d; j += 1024) {
    const float sjj = S[j * d + j];
    const bool dd = sjj == 0.0f;
    const double h = dd ? 1.0 : scale * double(sjj);
    keys[j] = h;
    dead[j] = dd ? 1 : 0;
    sum += h;
  }
  red[threadIdx.x] = sum;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    double damp = fmax(percdamp * (red[0] / double(d)), kEpsFloor);
    for (int a = 0; a < attempt; ++a) damp *= 10.0;
    *damp_out = damp;
  }
}

// Stable descending order of the keys by rank counting:
// rank(j) = #{k : key_k > key_j} + #{k < j : key_k == key_j}.
__global__ __launch_bounds__(256) void rank_sort_kernel(
    const double* __restrict__ keys, int64_t d, int32_t* __restrict__ perm) {
  __shared__ double tile[256];
  const int64_t j = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const double kj = j < d ? keys[j] : 0.0;
  int64_t rank = 0;
  for (int64_t t0 = 0; t0 < d; t0 += 256) {
    tile[threadIdx.x] = (t0 + threadIdx.x < d) ? keys[t0 + threadIdx.x] : 0.0;
    __syncthreads();
    const int lim = static_cast<int>(min<int64_t>(256, d - t0));
    for (int k = 0; k < lim; ++k) {
      const double kk = tile[k];
      rank += (kk > kj) || (kk == kj && t0 + k < j);
    }
    __syncthreads();
  }
  if (j < d) perm[rank] = static_cast<int32_t>(j);
}

__global__ void zero_flag_kernel(int* flag) { *flag = 0; }

__global__ void identity_perm_kernel(int64_t d, int32_t* __restrict__ perm) {
  const int64_t j = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (j < d) perm[j] = static_cast<int32_t>(j);
}

// H[a][b] = (2/n) S[perm a][perm b] (+ damp on the diagonal; dead diagonal
// entries are 1 before damping).  Upper triangle only.
__global__ __launch_bounds__(256) void build_h_kernel(
    const float* __restrict__ S, int64_t d, int64_t n,
    const int32_t* __restrict__ perm, const uint8_t* __restrict__ dead,
    const double* __restrict__ damp, double* __restrict__ H) {
  const int64_t a = blockIdx.y;
  const int64_t b = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (b >= d || b < a) return;
  const double scale = 2.0 / double(n);
  const int64_t pa = perm[a];
  double h;
  if (a == b) {
    h = dead[pa] ? 1.0 : scale * double(S[pa * d + pa]);
    h += *damp;
  } else {
    h = scale * double(S[pa * d + perm[b]]);
  }
  H[a * d + b] = h;
}

// ---------------------------------------------------------------------------
// Step 1 + 2: diagonal block factor (every workgroup, in LDS) + panel solve
// ---------------------------------------------------------------------------

// A_KK (nbk x nbk, upper triangle in Ad) = U U^T with U upper, in place.
// Step c (from the last column down) eliminates column c from the leading
// block with the unscaled column, A_ij -= A_ic A_jc / A_cc (i <= j < c);
// column c is final after its step, so U is formed at the end:
// U_cc = sqrt(A_cc), U_ic = A_ic / U_cc.  One barrier per column.
__device__ void factor_diag_block(double (*Ad)[kNb + 1], double* piv, int nbk,
                                  int* flag, bool report) {
  static_assert(kNb == 64, "index split below assumes 64 columns");
  for (int c = nbk - 1; c >= 0; --c) {
    double p = Ad[c][c];
    const bool bad = !(p > 0.0);
    if (bad) p = 1.0;
    if (threadIdx.x == 0) {
      piv[c] = p;
      if (bad && report) atomicOr(flag, 1);
    }
    const double pinv = 1.0 / p;
    for (int e = threadIdx.x; e < kNb * kNb; e += blockDim.x) {
      const int i = e >> 6, j = e & 63;
      if (i <= j && j < c) Ad[i][j] -= Ad[i][c] * Ad[j][c] * pinv;
    }
    __syncthreads();
  }
  for (int e = threadIdx.x; e < kNb * kNb; e += blockDim.x) {
    const int i = e >> 6, j = e & 63;
    if (i <= j && j < nbk) Ad[i][j] = (i == j) ? sqrt(piv[i]) : Ad[i][j] / sqrt(piv[j]);
  }
  __syncthreads();
}

// Block K = [k0, k0 + nbk).  Workgroup w solves rows [256w, 256w + 256) of
// the panel: x U_KK^T = A_iK, in place, one row per thread.
__global__ __launch_bounds__(256) void chol_panel_kernel(
    double* __restrict__ H, int64_t d, int64_t k0, int nbk,
    int* __restrict__ flag) {
  __shared__ double Ad[kNb][kNb + 1];
  __shared__ double piv[kNb];
  for (int e = threadIdx.x; e < kNb * kNb; e += 256) {
    const int i = e >> 6, j = e & 63;
    Ad[i][j] = (i < nbk && j < nbk && i <= j) ? H[(k0 + i) * d + k0 + j] : 0.0;
  }
  __syncthreads();
  factor_diag_block(Ad, piv, nbk, flag, blockIdx.x == 0);
  if (blockIdx.x == 0) {
    for (int e = threadIdx.x; e < kNb * kNb; e += 256) {
      const int i = e >> 6, j = e & 63;
      if (i <= j && j < nbk) H[(k0 + i) * d + k0 + j] = Ad[i][j];
    }
  }
  const int64_t r = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (r >= k0) return;
  double* row = H + r * d + k0;
  double x[kNb];
#pragma unroll
  for (int c = 0; c < kNb; ++c) x[c] = (c < nbk) ? row[c] : 0.0;
  // x U^T = a  <=>  sum_{c' >= c} x[c'] U[c][c'] = a[c]; solve from the end
#pragma unroll
  for (int c = kNb - 1; c >= 0; --c) {
    if (c < nbk) {
      x[c] /= Ad[c][c];
#pragma unroll
      for (int c2 = 0; c2 < c; ++c2) x[c2] -= x[c] * Ad[c2][c];
    }
  }
#pragma unroll
  for (int c = 0; c < kNb; ++c)
    if (c < nbk) row[c] = x[c];
}

// ---------------------------------------------------------------------------
// fp64 tile GEMM core: 64x64 output tile, 256 threads x (4x4), k-step 16
// ---------------------------------------------------------------------------

template <class FA, class FB>
__device__ inline void tile_gemm(int64_t kbeg, int64_t kend, FA fa, FB fb,
                                 double acc[4][4]) {
  __shared__ double As[16][68];
  __shared__ double Bs[16][68];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  for (int64_t k0 = kbeg; k0 < kend; k0 += 16) {
    for (int e = threadIdx.x; e < 16 * 64; e += 256) {
      const int kk = e >> 6, ii = e & 63;
      const int64_t k = k0 + kk;
      As[kk][ii] = k < kend ? fa(ii, k) : 0.0;
      Bs[kk][ii] = k < kend ? fb(k, ii) : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      double av[4], bv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        av[u] = As[kk][ty * 4 + u];
        bv[u] = Bs[kk][tx * 4 + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[u][w] = fma(av[u], bv[w], acc[u][w]);
    }
    __syncthreads();
  }
}

// Step 3: A[i][j] -= sum_c P[i][c] P[j][c] over the upper 64x64 tiles of
// [0, k0)^2, P = H[:, k0:k0+nbk].
__global__ __launch_bounds__(256) void syrk_update_kernel(
    double* __restrict__ H, int64_t d, int64_t k0, int nbk) {
  const int64_t ti = blockIdx.y, tj = blockIdx.x;
  if (ti > tj) return;
  const int64_t I0 = ti * 64, J0 = tj * 64;
  const double* P = H + k0;
  auto fa = [&](int ii, int64_t k) -> double {
    const int64_t i = I0 + ii;
    return i < k0 ? P[i * d + k] : 0.0;
  };
  auto fb = [&](int64_t k, int jj) -> double {
    const int64_t j = J0 + jj;
    return j < k0 ? P[j * d + k] : 0.0;
  };
  double acc[4][4] = {};
  tile_gemm(0, nbk, fa, fb, acc);
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int64_t i = I0 + ty * 4 + u, j = J0 + tx * 4 + w;
      if (i < k0 && j < k0 && i <= j) H[i * d + j] -= acc[u][w];
    }
}

// ---------------------------------------------------------------------------
// R = U^-1
// ---------------------------------------------------------------------------

// Each 64x64 diagonal block: R_KK = U_KK^-1 (upper).  Thread j solves
// U x = e_j by back substitution for column j.
__global__ __launch_bounds__(64) void trtri_diag_kernel(
    const double* __restrict__ U, double* __restrict__ R, int64_t d) {
  __shared__ double Ud[kNb][kNb + 1];
  const int64_t k0 = int64_t(blockIdx.x) * kNb;
  const int nbk = static_cast<int>(min<int64_t>(kNb, d - k0));
  for (int e = threadIdx.x; e < kNb * kNb; e += 64) {
    const int i = e >> 6, j = e & 63;
    Ud[i][j] = (i < nbk && j < nbk && i <= j) ? U[(k0 + i) * d + k0 + j] : (i == j ? 1.0 : 0.0);
  }
  __syncthreads();
  const int j = threadIdx.x;
  double x[kNb];
#pragma unroll
  for (int i = 0; i < kNb; ++i) x[i] = (i == j) ? 1.0 : 0.0;
#pragma unroll
  for (int i = kNb - 1; i >= 0; --i) {
    if (i <= j) {
      x[i] /= Ud[i][i];
#pragma unroll
      for (int i2 = 0; i2 < i; ++i2) x[i2] -= Ud[i2][i] * x[i];
    }
  }
  if (j < nbk) {
#pragma unroll
    for (int i = 0; i < kNb; ++i)
      if (i < nbk) R[(k0 + i) * d + k0 + j] = (i <= j) ? x[i] : 0.0;
  }
}

// Level s: pairs p of adjacent diagonal blocks I = [2ps, 2ps+s),
// J = [2ps+s, min(2ps+2s, d)).  T_p = U_IJ R_JJ  (R_JJ upper: k <= j).
__global__ __launch_bounds__(256) void trtri_t_kernel(
    const double* __restrict__ U, const double* __restrict__ R,
    double* __restrict__ T, int64_t d, int64_t s) {
  const int64_t p = blockIdx.z;
  const int64_t I0 = 2 * p * s, J0 = I0 + s;
  if (J0 >= d) return;
  const int64_t sJ = min<int64_t>(s, d - J0);
  const int64_t ti = blockIdx.y, tj = blockIdx.x;
  if (ti * 64 >= s || tj * 64 >= sJ) return;
  const int64_t i0 = ti * 64, j0 = tj * 64;
  auto fa = [&](int ii, int64_t k) -> double {
    return (k < sJ) ? U[(I0 + i0 + ii) * d + J0 + k] : 0.0;
  };
  auto fb = [&](int64_t k, int jj) -> double {
    const int64_t j = j0 + jj;
    return (k <= j && j < sJ) ? R[(J0 + k) * d + J0 + j] : 0.0;
  };
  double acc[4][4] = {};
  tile_gemm(0, min<int64_t>(sJ, j0 + 64), fa, fb, acc);
  double* Tp = T + p * s * s;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int64_t i = i0 + ty * 4 + u, j = j0 + tx * 4 + w;
      if (i < s && j < sJ) Tp[i * s + j] = acc[u][w];
    }
}

// R_IJ = -R_II T_p  (R_II upper: k >= i).
__global__ __launch_bounds__(256) void trtri_r_kernel(
    double* __restrict__ R, const double* __restrict__ T, int64_t d,
    int64_t s) {
  const int64_t p = blockIdx.z;
  const int64_t I0 = 2 * p * s, J0 = I0 + s;
  if (J0 >= d) return;
  const int64_t sJ = min<int64_t>(s, d - J0);
  const int64_t ti = blockIdx.y, tj = blockIdx.x;
  if (ti * 64 >= s || tj * 64 >= sJ) return;
  const int64_t i0 = ti * 64, j0 = tj * 64;
  const double* Tp = T + p * s * s;
  auto fa = [&](int ii, int64_t k) -> double {
    const int64_t i = i0 + ii;
    return (k >= i) ? R[(I0 + i) * d + I0 + k] : 0.0;
  };
  auto fb = [&](int64_t k, int jj) -> double {
    const int64_t j = j0 + jj;
    return (j < sJ) ? Tp[k * s + j] : 0.0;
  };
  double acc[4][4] = {};
  tile_gemm(i0, s, fa, fb, acc);
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int64_t i = i0 + ty * 4 + u, j = j0 + tx * 4 + w;
      if (i < s && j < sJ) R[(I0 + i) * d + J0 + j] = -acc[u][w];
    }
}

__global__ __launch_bounds__(256) void r_to_f32_kernel(
    const double* __restrict__ R64, int64_t d, float* __restrict__ R) {
  const int64_t a = blockIdx.y;
  const int64_t b = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (b >= d) return;
  R[a * d + b] = (b >= a) ? static_cast<float>(R64[a * d + b]) : 0.0f;
}

unsigned cdiv(int64_t a, int64_t b) { return static_cast<unsigned>((a + b - 1) / b); }

}  // namespace

size_t factor_ws_bytes(int64_t d) {
  Carver c(nullptr);
  carve_factor_ws(c, d);
  return c.bytes();
}

FactorWs carve_factor_ws(Carver& c, int64_t d) {
  FactorWs f;
  f.H = c.take<double>(size_t(d) * size_t(d));
  f.R = c.take<double>(size_t(d) * size_t(d));
  // largest level: ceil(d / 2s) pairs of s x s with s < d
  int64_t tmax = 0;
  for (int64_t s = kNb; s < d; s *= 2) {
    const int64_t pairs = (d + 2 * s - 1) / (2 * s);
    tmax = std::max(tmax, pairs * s * s);
  }
  f.T = c.take<double>(size_t(std::max<int64_t>(tmax, 1)));
  f.keys = c.take<double>(size_t(d));
  f.damp = c.take<double>(1);
  f.flag = c.take<int>(1);
  return f;
}

gptq_status launch_prep_stats(const float* S, int64_t d, int64_t n,
                              double percdamp, int attempt, const FactorWs& f,
                              uint8_t* dead, hipStream_t st) {
  prep_stats_kernel<<<1, 1024, 0, st>>>(S, d, n, percdamp, attempt, f.keys,
                                        f.damp, dead);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

gptq_status launch_perm(int64_t d, int act_order, const FactorWs& f,
                        int32_t* perm, hipStream_t st) {
  if (act_order)
    rank_sort_kernel<<<cdiv(d, 256), 256, 0, st>>>(f.keys, d, perm);
  else
    identity_perm_kernel<<<cdiv(d, 256), 256, 0, st>>>(d, perm);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

gptq_status launch_build_h(const float* S, int64_t d, int64_t n,
                           const int32_t* perm, const uint8_t* dead,
                           const FactorWs& f, hipStream_t st) {
  build_h_kernel<<<dim3(cdiv(d, 256), static_cast<unsigned>(d)), 256, 0, st>>>(
      S, d, n, perm, dead, f.damp, f.H);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

gptq_status launch_cholesky_upper(int64_t d, const FactorWs& f,
                                  hipStream_t st) {
  zero_flag_kernel<<<1, 1, 0, st>>>(f.flag);
  GPTQ_CHECK_LAUNCH();
  // blocks from the bottom-right corner; the first one absorbs d % 64
  int64_t k1 = d;
  while (k1 > 0) {
    const int nbk = static_cast<int>((k1 % kNb) ? (k1 % kNb) : kNb);
    const int64_t k0 = k1 - nbk;
    chol_panel_kernel<<<std::max(1u, cdiv(k0, 256)), 256, 0, st>>>(f.H, d, k0, nbk, f.flag);
    GPTQ_CHECK_LAUNCH();
    if (k0 > 0) {
      const unsigned nt = cdiv(k0, 64);
      syrk_update_kernel<<<dim3(nt, nt), 256, 0, st>>>(f.H, d, k0, nbk);
      GPTQ_CHECK_LAUNCH();
    }
    k1 = k0;
  }
  return GPTQ_OK;
}

gptq_status launch_triangular_inverse(int64_t d, const FactorWs& f,
                                      hipStream_t st) {
  // Diagonal blocks are aligned to multiples of 64 from the top; the
  // Cholesky's block boundaries do not matter for the inverse.
  trtri_diag_kernel<<<cdiv(d, kNb), 64, 0, st>>>(f.H, f.R, d);
  GPTQ_CHECK_LAUNCH();
  for (int64_t s = kNb; s < d; s *= 2) {
    const unsigned pairs = cdiv(d, 2 * s);
    const dim3 grid(cdiv(s, 64), cdiv(s, 64), pairs);
    trtri_t_kernel<<<grid, 256, 0, st>>>(f.H, f.R, f.T, d, s);
    GPTQ_CHECK_LAUNCH();
    trtri_r_kernel<<<grid, 256, 0, st>>>(f.R, f.T, d, s);
    GPTQ_CHECK_LAUNCH();
  }
  return GPTQ_OK;
}

gptq_status launch_r_to_f32(int64_t d, const FactorWs& f, float* R,
                            hipStream_t st) {
  r_to_f32_kernel<<<dim3(cdiv(d, 256), static_cast<unsigned>(d)), 256, 0, st>>>(f.R, d, R);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

}  // namespace gptq
