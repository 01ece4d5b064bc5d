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
//   1. factor the diagonal block A_KK = U_KK U_KK^T and invert it,
//      W_KK = U_KK^-1 (= R's diagonal block), in one workgroup;
//   2. panel: U_iK = A_iK W_KK^T for every row i above the block (GEMM);
//   3. trailing update A_ij -= U_iK U_jK^T (upper tiles only), applied to
//      the next blocks' own columns at once and to the rest of the matrix
//      once per group of four blocks (k = 256).
// The off-diagonal blocks of R then come from R_12 = -R_11 U_12 R_22
// applied level by level (block size 64, 128, 256, ...).
#include <algorithm>
#include <cmath>
#include <functional>
#include <mutex>

#include "common.h"

namespace gptq {
namespace {

constexpr int kNb = 64;          // diagonal block / panel width
constexpr int kGroup = 4;        // blocks per trailing update (k = 256)
constexpr int64_t kCUs = 256;     // MI355X compute units
constexpr int64_t kBgTiles = 1;   // deferred trailing tiles per idle workgroup
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
    const double mean = red[0] / double(d);
    double damp = fmax(percdamp * mean, kEpsFloor);
    for (int a = 0; a < attempt; ++a) damp *= 10.0;
    // a non-finite diagonal (NaN or inf) makes every pivot NaN, which the
    // factor flags as not positive definite
    *damp_out = isfinite(mean) ? damp : __builtin_nan("");
  }
}

// Stable descending order of the keys by rank counting:
// rank(j) = #{k : key_k > key_j} + #{k < j : key_k == key_j}.
// NaN keys (a non-finite statistic) are ordered after every number, among
// themselves by index, so the ranks are always a permutation of 0..d-1 and
// every later gather through perm stays in bounds; the factor then reports
// the non-finite matrix as not positive definite.
__global__ __launch_bounds__(256) void rank_sort_kernel(
    const double* __restrict__ keys, int64_t d, int32_t* __restrict__ perm) {
  __shared__ double tile[256];
  const int64_t j = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const double kj = j < d ? keys[j] : 0.0;
  const bool nj = kj != kj;
  int64_t rank = 0;
  for (int64_t t0 = 0; t0 < d; t0 += 256) {
    tile[threadIdx.x] = (t0 + threadIdx.x < d) ? keys[t0 + threadIdx.x] : 0.0;
    __syncthreads();
    const int lim = static_cast<int>(min<int64_t>(256, d - t0));
    for (int k = 0; k < lim; ++k) {
      const double kk = tile[k];
      const bool nk = kk != kk;
      const bool same = nk == nj && (nk || kk == kj);
      rank += (!nk && (nj || kk > kj)) || (same && t0 + k < j);
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
// entries are 1 before damping).  Upper triangle only: one workgroup per
// row a, its threads taking the columns b >= a, four per pass (independent
// loads in flight); ident: perm is the identity (no gather of perm[b]).
__global__ __launch_bounds__(256) void build_h_kernel(
    const float* __restrict__ S, int64_t d, int64_t n,
    const int32_t* __restrict__ perm, const uint8_t* __restrict__ dead,
    const double* __restrict__ damp, int ident, double* __restrict__ H) {
  const int64_t a = blockIdx.x;
  const double scale = 2.0 / double(n);
  const int64_t pa = ident ? a : perm[a];
  const float* Srow = S + pa * d;
  double* Hrow = H + a * d;
  const int64_t b0 = (a & ~int64_t(255)) + threadIdx.x;
  for (int64_t bb = b0; bb < d; bb += 1024) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t b = bb + 256 * u;
      v[u] = (b >= a && b < d) ? Srow[ident ? b : perm[b]] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t b = bb + 256 * u;
      if (b < a || b >= d) continue;
      double h = scale * double(v[u]);
      if (b == a) h = (dead[pa] ? 1.0 : h) + *damp;
      Hrow[b] = h;
    }
  }
}

// ---------------------------------------------------------------------------
// Step 1: diagonal block factor + inverse (one workgroup)
// ---------------------------------------------------------------------------

typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ inline double read_lane(double x, int l) {
  const long long v = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(v), l);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(v >> 32), l);
  return __longlong_as_double((static_cast<long long>(hi) << 32) |
                              static_cast<unsigned>(lo));
}

// 1/sqrt(p) from the hardware estimate and two Newton steps
// 1/sqrt(p): the hardware estimate (relative error about 2^-24) and one
// third-order step r (1 + e/2 + 3e^2/8), e = 1 - p r^2, whose truncation
// error (about 5e^3/16) is far below the fp64 rounding.
__device__ inline double rsqrt_refined(double p) {
  const double r = __builtin_amdgcn_rsq(p);
  const double e = fma(-(p * r), r, 1.0);
  return fma(r * e, fma(e, 0.375, 0.5), r);
}

constexpr int kWp = kNb + 2;     // LDS pitch of the U / W arrays (16-B rows)

// Step 1 for the block K = [k0, k0 + nbk), nbk <= 64, one 256-thread
// workgroup; rows/columns past nbk are padded with the identity.
//
// A_KK = U_KK U_KK^T, four columns per barrier: thread (wave w, lane i)
// holds A[i][j] for the columns j = w + 4u (u = 0..15), upper part i <= j.
// For each group G = {g0..g0+3}, from the last one, the owners publish the
// group's columns, every wave factors the 64 x 4 panel in registers (lane =
// row; pivots from the right: U_cc = sqrt(A_cc), U_ic = A_ic / U_cc, then
// the group's remaining columns lose U_:c U_c'c) and applies the rank-4
// update A_ij -= sum_{c in G} U_ic U_jc to its columns j < g0: at once to
// its column in the next group (the only one the next barrier waits for),
// the others during the next group's pivot chain.  Each column receives the
// groups' updates in the same order either way.
//
// W_KK = U_KK^-1 (R's diagonal block, R = U^-1): the four 16 x 16 diagonal
// blocks by back substitution, then W_12 = -W_11 U_12 W_22 at sizes 16 and
// 32 on the matrix cores.
struct DiagLds {
  double Us[kNb][kWp];   // block staging, then U
  double Wl[kNb][kWp];   // W = U^-1
  double pan[2][4][kNb];
  double rsl[kNb];       // 1 / U_cc
  double Tl[32][34];
};

// Stages the diagonal block [k0, k0 + nbk) of H in L.Us (upper part, the
// rest identity) and clears L.Wl.
__device__ inline void diag_load(const double* __restrict__ H, int64_t d,
                                 int64_t k0, int nbk, DiagLds& L) {
  for (int e = threadIdx.x; e < kNb * kNb; e += 256) {
    const int r = e >> 6, c = e & 63;
    double v = (r == c) ? 1.0 : 0.0;
    if (r < nbk && c < nbk && r <= c) v = H[(k0 + r) * d + k0 + c];
    L.Us[r][c] = v;
    L.Wl[r][c] = 0.0;
  }
}

// Factors and inverts the block staged in L.Us (upper triangle read; L.Wl
// cleared) into L.Us (U, upper) and L.Wl (W = U^-1); returns true when a
// pivot was not positive.
__device__ __attribute__((always_inline)) inline bool diag_factor(DiagLds& L) {
  static_assert(kNb == 64, "thread/element split assumes 64 columns");
  auto& Us = L.Us;
  auto& Wl = L.Wl;
  auto& pan = L.pan;
  auto& rsl = L.rsl;
  auto& Tl = L.Tl;
  const int t = threadIdx.x;
  const int w = t >> 6, i = t & 63;
  __syncthreads();
  double a[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) a[u] = Us[i][w + 4 * u];
  __syncthreads();
  double ok = 1.0;        // -1 once a pivot was not positive (or NaN)
  double Up[4];           // previous group's U[i][g0 + cc] (deferred updates)
#pragma unroll
  for (int g = 15; g >= 0; --g) {
    const int g0 = 4 * g;
    pan[g & 1][w][i] = a[g];             // column g0 + w
    __syncthreads();
    // P[cc]: this lane's row of the group's columns.  q[r][cc]: the group's
    // 4 x 4 diagonal block and qn[cc]: row g0 - 4 + w (the row of this
    // wave's column in the next group), both the same in every lane of the
    // wave (broadcast LDS reads), so the pivots and the next group's column
    // need no cross-lane moves.
    double P[4], Uc[4], q[4][4], qn[4];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      P[cc] = pan[g & 1][cc][i];
#pragma unroll
      for (int r = 0; r <= cc; ++r) q[r][cc] = pan[g & 1][cc][g0 + r];
      qn[cc] = g > 0 ? pan[g & 1][cc][g0 - 4 + w] : 0.0;
    }
    double2 ud[15][2];     // rows w + 4u of the previous group's U columns
    if (g < 15) {
#pragma unroll
      for (int u = g - 1; u >= 0; --u) {
        const int jr = w + 4 * u;
        ud[u][0] = *reinterpret_cast<const double2*>(&Us[jr][g0 + 4]);
        ud[u][1] = *reinterpret_cast<const double2*>(&Us[jr][g0 + 6]);
      }
    }
    double un[4], rsw[4];
#pragma unroll
    for (int cc = 3; cc >= 0; --cc) {
      // a pivot that is not positive leaves non-finite values behind; the
      // flag discards the whole factor then
      const double p = q[cc][cc];
      ok = fmin(ok, (p > 0.0) ? p : -1.0);
      const double rs = rsqrt_refined(p);
      rsw[cc] = rs;
      // rows below the pivot (i > c) carry values that are never read: the
      // lower triangle of U is not used
      Uc[cc] = P[cc] * rs;
      // U[g0 + r][c] and U[g0 - 4 + w][c] as their own lanes compute them
      double uq[4];
#pragma unroll
      for (int r = 0; r < cc; ++r) uq[r] = q[r][cc] * rs;
      un[cc] = qn[cc] * rs;
#pragma unroll
      for (int c2 = cc - 1; c2 >= 0; --c2) {
        P[c2] = fma(-Uc[cc], uq[c2], P[c2]);
        qn[c2] = fma(-un[cc], uq[c2], qn[c2]);
#pragma unroll
        for (int r = 0; r <= c2; ++r) q[r][c2] = fma(-uq[r], uq[c2], q[r][c2]);
      }
    }
    // the previous group's update of this wave's other columns, deferred to
    // this group: its operands were read with the pivot block, its FMAs fill
    // the pivot chain's latency
    if (g < 15) {
#pragma unroll
      for (int u = g - 1; u >= 0; --u) {
        double v = a[u];
        v = fma(-Up[0], ud[u][0].x, v);
        v = fma(-Up[1], ud[u][0].y, v);
        v = fma(-Up[2], ud[u][1].x, v);
        v = fma(-Up[3], ud[u][1].y, v);
        a[u] = v;
      }
    }
    // every wave writes the same values; a wave reads back only after its
    // own writes (LDS operations of one wave complete in order)
    *reinterpret_cast<double2*>(&Us[i][g0]) = double2{Uc[0], Uc[1]};
    *reinterpret_cast<double2*>(&Us[i][g0 + 2]) = double2{Uc[2], Uc[3]};
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (g > 0) {                         // the next group's column now
      double v = a[g - 1];
      v = fma(-Uc[0], un[0], v);
      v = fma(-Uc[1], un[1], v);
      v = fma(-Uc[2], un[2], v);
      v = fma(-Uc[3], un[3], v);
      a[g - 1] = v;
    }
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) Up[cc] = Uc[cc];
    if (t < 4) {
      double v = rsw[0];
      v = (t == 1) ? rsw[1] : v;
      v = (t == 2) ? rsw[2] : v;
      v = (t == 3) ? rsw[3] : v;
      rsl[g0 + t] = v;
    }
  }
  __syncthreads();
  const bool bad = !(ok > 0.0);
  const int lane = i, lr = lane & 15, lk = lane >> 4;
  // 16 x 16 diagonal blocks of W: wave w, lanes 0..15 solve one column each
  if (lane < 16) {
    const int o = 16 * w, jj = lane;
    double x[16];
#pragma unroll
    for (int ii = 15; ii >= 0; --ii) {
      double acc = (ii == jj) ? 1.0 : 0.0;
#pragma unroll
      for (int k = ii + 1; k < 16; ++k) acc = fma(-Us[o + ii][o + k], x[k], acc);
      x[ii] = acc * rsl[o + ii];
    }
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) Wl[o + ii][o + jj] = x[ii];
  }
  __syncthreads();
  // size 16: pairs (0,1) and (2,3), one wave each
  if (w < 2) {
    const int A0 = 32 * w, B0 = A0 + 16;
    f64x4 T = {0.0, 0.0, 0.0, 0.0}, Y = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      T = __builtin_amdgcn_mfma_f64_16x16x4f64(Us[A0 + lr][B0 + 4 * ks + lk],
                                                Wl[B0 + 4 * ks + lk][B0 + lr], T, 0, 0, 0);
    // T's output row l/16 + 4v is the B operand row of k step v
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      Y = __builtin_amdgcn_mfma_f64_16x16x4f64(Wl[A0 + lr][A0 + 4 * ks + lk], T[ks], Y, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < 4; ++v) Wl[A0 + lk + 4 * v][B0 + lr] = -Y[v];
  }
  __syncthreads();
  // size 32: T = U_AB W_BB, then W_AB = -W_AA T; wave w owns tile (w/2, w%2)
  {
    const int r0 = 16 * (w >> 1), c0 = 16 * (w & 1);
    f64x4 T = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      T = __builtin_amdgcn_mfma_f64_16x16x4f64(Us[r0 + lr][32 + 4 * ks + lk],
                                                Wl[32 + 4 * ks + lk][32 + c0 + lr], T, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < 4; ++v) Tl[r0 + lk + 4 * v][c0 + lr] = T[v];
  }
  __syncthreads();
  {
    const int r0 = 16 * (w >> 1), c0 = 16 * (w & 1);
    f64x4 Y = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      Y = __builtin_amdgcn_mfma_f64_16x16x4f64(Wl[r0 + lr][4 * ks + lk],
                                                Tl[4 * ks + lk][c0 + lr], Y, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < 4; ++v) Wl[r0 + lk + 4 * v][32 + c0 + lr] = -Y[v];
  }
  __syncthreads();
  return bad;
}

// Writes W_KK (R's diagonal block; U_KK itself is not needed later) and
// raises the flag on a non-positive pivot.
__device__ inline void diag_store(double* __restrict__ R, int64_t d, int64_t k0,
                                  int nbk, bool bad, const DiagLds& L,
                                  int* __restrict__ flag) {
  const int t = threadIdx.x;
  if (bad && t == 0) atomicOr(flag, 1);
  for (int e = t; e < kNb * kNb; e += 256) {
    const int r = e >> 6, c = e & 63;
    // upper part only: every reader of R masks the lower triangle
    if (r < nbk && c < nbk && r <= c) R[(k0 + r) * d + k0 + c] = L.Wl[r][c];
  }
}

__global__ __launch_bounds__(256) void chol_diag_kernel(
    double* __restrict__ H, double* __restrict__ R, int64_t d, int64_t k0,
    int nbk, int* __restrict__ flag) {
  __shared__ __align__(16) DiagLds L;
  diag_load(H, d, k0, nbk, L);
  const bool bad = diag_factor(L);
  diag_store(R, d, k0, nbk, bad, L, flag);
}

// ---------------------------------------------------------------------------
// fp64 tile GEMM core on the matrix cores: a 64x64 output tile per 256-thread
// workgroup, each wave a 32x32 quarter of 2x2 v_mfma_f64_16x16x4_f64 blocks.
// Lane l feeds A[row = l%16][k = l/16] and B[k = l/16][col = l%16] and
// receives D[row = l/16 + 4v][col = l%16] (the fp64 instruction interleaves
// its output rows differently from the fp32 one).  K is staged through LDS in
// chunks of 32 with the next chunk's loads issued before the current one is
// consumed.  fa(i, k) / fb(k, j) return operand elements (0 outside);
// B_KC: B's memory order has k contiguous (else j contiguous), which picks
// the coalesced thread-to-element map for loading it.
// ---------------------------------------------------------------------------

constexpr int kKc = 32;            // k chunk
constexpr int kLp = kKc + 2;       // LDS pitch (doubles)

struct GemmLds {
  double As[64][kLp];
  double Bs[64][kLp];
};

// One staging area per kernel, shared by every tile_gemm instantiation in it.
__device__ inline GemmLds& gemm_lds() {
  __shared__ GemmLds g;
  return g;
}

template <bool B_KC, class FA, class FB>
__device__ inline void tile_gemm(int64_t kbeg, int64_t kend, FA fa, FB fb,
                                 f64x4 acc[2][2]) {
  static_assert(kKc == 32, "the fetch map below covers 64 x 32 operands per chunk");
  auto& As = gemm_lds().As;
  auto& Bs = gemm_lds().Bs;
  const int t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;
  const int wr = (wv >> 1) * 32, wc = (wv & 1) * 32;
  const int lr = lane & 15, lk = lane >> 4;
  double ra[8], rb[8];
  auto fetch = [&](int64_t k0) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = t + 256 * u;
      {
        const int i = e >> 5, kk = e & 31;
        const int64_t k = k0 + kk;
        ra[u] = k < kend ? fa(i, k) : 0.0;
      }
      if (B_KC) {
        const int j = e >> 5, kk = e & 31;
        const int64_t k = k0 + kk;
        rb[u] = k < kend ? fb(k, j) : 0.0;
      } else {
        const int kk = e >> 6, j = e & 63;
        const int64_t k = k0 + kk;
        rb[u] = k < kend ? fb(k, j) : 0.0;
      }
    }
  };
  if (kbeg < kend) fetch(kbeg);
  for (int64_t k0 = kbeg; k0 < kend; k0 += kKc) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = t + 256 * u;
      As[e >> 5][e & 31] = ra[u];
      if (B_KC)
        Bs[e >> 5][e & 31] = rb[u];
      else
        Bs[e & 63][e >> 6] = rb[u];
    }
    __syncthreads();
    if (k0 + kKc < kend) fetch(k0 + kKc);
#pragma unroll
    for (int ks = 0; ks < kKc; ks += 4) {
      const double a0 = As[wr + lr][ks + lk], a1 = As[wr + 16 + lr][ks + lk];
      const double b0 = Bs[wc + lr][ks + lk], b1 = Bs[wc + 16 + lr][ks + lk];
      acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc[1][1], 0, 0, 0);
    }
    __syncthreads();
  }
}

// Output element (i, j) of the 64x64 tile held by this lane as acc[h][g][v].
template <class F>
__device__ inline void tile_store(const f64x4 acc[2][2], F f) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wr = (wv >> 1) * 32, wc = (wv & 1) * 32;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        f(wr + 16 * h + (lane >> 4) + 4 * v, wc + 16 * g + (lane & 15), acc[h][g][v]);
}

__device__ inline void zero_acc(f64x4 acc[2][2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int g = 0; g < 2; ++g) acc[h][g] = f64x4{0.0, 0.0, 0.0, 0.0};
}

// The trailing update after a group: A[i][j] -= sum_c P[i][c] P[j][c] over
// the upper 64x64 tiles of [0, k0)^2 in tile columns tj0.., P = H[:,
// k0:k0+nbk], except the last diagonal tile (the group's step kernels
// updated and factored it).
__global__ __launch_bounds__(256) void syrk_update_kernel(
    double* __restrict__ H, int64_t d, int64_t k0, int nbk, int64_t tj0) {
  const int64_t ti = blockIdx.y, tj = tj0 + blockIdx.x;
  if (ti > tj || (ti == tj && (ti + 1) * 64 >= k0)) return;
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
  f64x4 acc[2][2];
  zero_acc(acc);
  tile_gemm<true>(0, nbk, fa, fb, acc);
  tile_store(acc, [&](int ii, int jj, double v) {
    const int64_t i = I0 + ii, j = J0 + jj;
    if (i < k0 && j < k0 && i <= j) H[i * d + j] -= v;
  });
}

// One block K = [k0, k0 + nbk) of a group of blocks [kg, kend), one
// workgroup per 64-row tile i above it (I0 < k0).  The group's blocks are
// taken from the bottom; P = [kp, kp + nbp) is the one before K (kp < 0 for
// the group's first block).  Every row tile:
//   A_iC -= U_iP U_CP^T   for the group's column tiles C = K and the ones to
//                         its left down to kg (C above the diagonal): P's
//                         share, one block late, so that these updates never
//                         wait on another workgroup;
//   U_iK  = A_iK W_KK^T   (the panel; W_KK from the diagonal factor).
// The row tiles J in [kg - 64, k0) -- the group's later blocks and the next
// group's first one -- also take K's share of their own diagonal tile,
// A_JJ -= U_JK U_JK^T, and the one right above K (J = k0 - 64, whose block
// comes next) then factors and inverts it; the trailing update after the
// group leaves that tile out.  A_iK and U_iK stay in LDS between the steps.
// Workgroups past the row tiles apply part of the previous group's trailing
// update to the tiles this group never reads (see trailing_tiles).
// 64 x 64 products with k <= 64 in one LDS stage, for the step kernel: A(i,
// k) and B(j, k) (B k-contiguous) both [64][kWp], zero past the k range.
// Thread t holds operand elements e = t + 256u (u < 16) at (e / 64, e % 64),
// which keeps the global loads row-contiguous.
struct Tile64Lds {
  double As[kNb][kWp];
  double Bs[kNb][kWp];
};

__device__ inline Tile64Lds& tile64_lds() {
  __shared__ __align__(16) Tile64Lds g;
  return g;
}

template <class F>
__device__ inline void load64(F f, double r[16]) {
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int e = threadIdx.x + 256 * u;
    r[u] = f(e >> 6, e & 63);
  }
}

__device__ inline void stage64(const double r[16], double (&S)[kNb][kWp]) {
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int e = threadIdx.x + 256 * u;
    S[e >> 6][e & 63] = r[u];
  }
}

// acc += A B^T over k < 64 (same output map as tile_gemm / tile_store).
__device__ inline void mma64(const double (&A)[kNb][kWp], const double (&B)[kNb][kWp],
                             f64x4 acc[2][2]) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wr = (wv >> 1) * 32, wc = (wv & 1) * 32;
  const int lr = lane & 15, lk = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < kNb; ks += 4) {
    const double a0 = A[wr + lr][ks + lk], a1 = A[wr + 16 + lr][ks + lk];
    const double b0 = B[wc + lr][ks + lk], b1 = B[wc + 16 + lr][ks + lk];
    acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc[0][0], 0, 0, 0);
    acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, acc[0][1], 0, 0, 0);
    acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, acc[1][0], 0, 0, 0);
    acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc[1][1], 0, 0, 0);
  }
}

// Loads a 64 x 64 tile in the product output map (see tile_store).
template <class F>
__device__ inline void load_out(F f, double r[16]) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wr = (wv >> 1) * 32, wc = (wv & 1) * 32;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        r[(h * 2 + g) * 4 + v] = f(wr + 16 * h + (lane >> 4) + 4 * v, wc + 16 * g + (lane & 15));
}

// The previous group's trailing update on the tiles no step of this group
// touches, A_ij -= P_i P_j^T with P = H[:, bk:bk+bK] (bK <= 256): upper
// tiles numbered column-major, L = tj (tj + 1) / 2 + ti, this workgroup
// taking L = t0 + b, t0 + b + nbg, ... below t0 + nt.
__device__ inline void trailing_tiles(double* __restrict__ H, int64_t d,
                                      int64_t bk, int bK, int64_t t0, int64_t nt,
                                      int64_t b, int64_t nbg) {
  auto& T = tile64_lds();
  for (int64_t q = b; q < nt; q += nbg) {
    const int64_t Lq = t0 + q;
    int64_t tj = static_cast<int64_t>((sqrt(8.0 * double(Lq) + 1.0) - 1.0) * 0.5);
    while (tj * (tj + 1) / 2 > Lq) --tj;
    while ((tj + 1) * (tj + 2) / 2 <= Lq) ++tj;
    const int64_t ti = Lq - tj * (tj + 1) / 2;
    const double* Pi = H + ti * 64 * d + bk;
    const double* Pj = H + tj * 64 * d + bk;
    f64x4 acc[2][2];
    zero_acc(acc);
    double ra[16], rb[16];
    auto fetch = [&](int kc) {
      load64([&](int i, int k) { return kc + k < bK ? Pi[int64_t(i) * d + kc + k] : 0.0; }, ra);
      load64([&](int j, int k) { return kc + k < bK ? Pj[int64_t(j) * d + kc + k] : 0.0; }, rb);
    };
    fetch(0);
    for (int kc = 0; kc < bK; kc += 64) {
      __syncthreads();                         // the previous chunk's products are done
      stage64(ra, T.As);
      stage64(rb, T.Bs);
      __syncthreads();
      if (kc + 64 < bK) fetch(kc + 64);
      mma64(T.As, T.Bs, acc);
    }
    double* Dt = H + ti * 64 * d + tj * 64;
    tile_store(acc, [&](int ii, int jj, double v) {
      if (ti != tj || ii <= jj) Dt[int64_t(ii) * d + jj] -= v;
    });
  }
}

__global__ __launch_bounds__(256) void chol_step_kernel(
    double* __restrict__ H, double* __restrict__ R, int64_t d, int64_t k0,
    int nbk, int64_t kp, int nbp, int64_t kg, int* __restrict__ flag,
    int64_t bk, int bK, int64_t t0, int64_t nt) {
  __shared__ __align__(16) DiagLds L;
  auto& T = tile64_lds();
  const int64_t nrow = k0 / 64;
  if (int64_t(blockIdx.x) >= nrow) {           // the chip's idle workgroups
    trailing_tiles(H, d, bk, bK, t0, nt, blockIdx.x - nrow, gridDim.x - nrow);
    return;
  }
  auto& At = L.Us;                 // A_iK, then (next block's tile) its U
  auto& Pt = L.Wl;                 // U_iK, then (next block's tile) its W
  const int64_t I0 = int64_t(blockIdx.x) * 64;
  const bool diag_later = I0 >= kg - kNb;     // a diagonal tile still to come
  const double* W = R + k0 * d + k0;
  double* D = H + I0 * d + I0;
  f64x4 acc[2][2];
  // every global operand of the chain is requested up front
  double ra[16], rb[16], rw[16], rk[16], rd[16];
  if (kp >= 0) {
    load64([&](int i, int k) { return k < nbp ? H[(I0 + i) * d + kp + k] : 0.0; }, ra);
    load64([&](int j, int k) {
      return (j < nbk && k < nbp) ? H[(k0 + j) * d + kp + k] : 0.0;
    }, rb);
  }
  load64([&](int j, int k) {                   // B(k, j) = W[j][k], upper
    return (j < nbk && k < nbk && k >= j) ? W[int64_t(j) * d + k] : 0.0;
  }, rw);
  load_out([&](int i, int j) { return j < nbk ? H[(I0 + i) * d + k0 + j] : 0.0; }, rk);
  if (diag_later)
    load_out([&](int i, int j) { return i <= j ? D[int64_t(i) * d + j] : 0.0; }, rd);
  // P's share: C = k0 first (into At), then C = k0 - 64, ... (in place)
  if (kp >= 0) {
    stage64(ra, T.As);
    for (int64_t c = k0; c >= kg && c > I0; c -= 64) {
      if (c != k0) {
        load64([&](int j, int k) { return k < nbp ? H[(c + j) * d + kp + k] : 0.0; }, rb);
        __syncthreads();                       // the previous product read T.Bs
      }
      stage64(rb, T.Bs);
      __syncthreads();
      zero_acc(acc);
      mma64(T.As, T.Bs, acc);
      if (c == k0) {
        int q = 0;
        tile_store(acc, [&](int ii, int jj, double v) { At[ii][jj] = rk[q++] - v; });
      } else {
        tile_store(acc, [&](int ii, int jj, double v) { H[(I0 + ii) * d + c + jj] -= v; });
      }
    }
  } else {
    zero_acc(acc);
    int q = 0;
    tile_store(acc, [&](int ii, int jj, double) { At[ii][jj] = rk[q++]; });
  }
  __syncthreads();                             // T.Bs free, At complete
  stage64(rw, T.Bs);
  __syncthreads();
  zero_acc(acc);
  mma64(At, T.Bs, acc);
  tile_store(acc, [&](int ii, int jj, double v) {
    if (jj < nbk) H[(I0 + ii) * d + k0 + jj] = v;
    Pt[ii][jj] = v;
  });
  if (!diag_later) return;
  __syncthreads();
  zero_acc(acc);
  mma64(Pt, Pt, acc);
  if (I0 + kNb < k0) {
    int q = 0;
    tile_store(acc, [&](int ii, int jj, double v) {
      const double x = rd[q++] - v;
      if (ii <= jj) D[int64_t(ii) * d + jj] = x;
    });
    return;
  }
  // the next block's diagonal tile (64 wide: only the bottom block of the
  // matrix is narrower, and it comes first)
  __syncthreads();                             // every product read At / Pt
  {
    int q = 0;
    tile_store(acc, [&](int ii, int jj, double v) {
      At[ii][jj] = ii <= jj ? rd[q] - v : 0.0;
      Pt[ii][jj] = 0.0;
      ++q;
    });
  }
  const bool bad = diag_factor(L);
  diag_store(R, d, I0, kNb, bad, L, flag);
}

// ---------------------------------------------------------------------------
// R = U^-1
// ---------------------------------------------------------------------------

// Level s: pairs p of adjacent diagonal blocks I = [2ps, 2ps+s),
// J = [2ps+s, min(2ps+2s, d)).  T_p = U_IJ R_JJ  (R_JJ upper: k <= j).
// A launch covers the 64x64 tiles of pairs p0 .. p0 + np - 1, item w =
// (tile column, tile row, pair) with the first fastest, each workgroup
// taking items blockIdx.x, blockIdx.x + gridDim.x, ... (a grid smaller than
// the item count leaves the rest of the chip to other work); pair p's T
// block starts (p - p0) s^2 into T.
__global__ __launch_bounds__(256) void trtri_t_kernel(
    const double* __restrict__ U, const double* __restrict__ R,
    double* __restrict__ T, int64_t d, int64_t s, int64_t p0, int64_t np) {
  const int64_t g = (s + 63) / 64, nitems = g * g * np;
  for (int64_t w = blockIdx.x; w < nitems; w += gridDim.x) {
    __syncthreads();                           // the previous item's LDS reads
    const int64_t p = p0 + w / (g * g);
    const int64_t I0 = 2 * p * s, J0 = I0 + s;
    if (J0 >= d) continue;
    const int64_t sJ = min<int64_t>(s, d - J0);
    // k runs to the end of tile column tj: the heavy columns (large tj) come
    // first, so the last items are the short ones
    const int64_t ti = w % g, tj = g - 1 - (w / g) % g;
    if (ti * 64 >= s || tj * 64 >= sJ) continue;
    const int64_t i0 = ti * 64, j0 = tj * 64;
    auto fa = [&](int ii, int64_t k) -> double {
      return (k < sJ) ? U[(I0 + i0 + ii) * d + J0 + k] : 0.0;
    };
    auto fb = [&](int64_t k, int jj) -> double {
      const int64_t j = j0 + jj;
      return (k <= j && j < sJ) ? R[(J0 + k) * d + J0 + j] : 0.0;
    };
    f64x4 acc[2][2];
    zero_acc(acc);
    tile_gemm<false>(0, min<int64_t>(sJ, j0 + 64), fa, fb, acc);
    double* Tp = T + (p - p0) * s * s;
    tile_store(acc, [&](int ii, int jj, double v) {
      const int64_t i = i0 + ii, j = j0 + jj;
      if (i < s && j < sJ) Tp[i * s + j] = v;
    });
  }
}

// R_IJ = -R_II T_p  (R_II upper: k >= i); items as above, tile rows with the
// longest k range (small ti) first.
__global__ __launch_bounds__(256) void trtri_r_kernel(
    double* __restrict__ R, const double* __restrict__ T, int64_t d,
    int64_t s, int64_t p0, int64_t np) {
  const int64_t g = (s + 63) / 64, nitems = g * g * np;
  for (int64_t w = blockIdx.x; w < nitems; w += gridDim.x) {
    __syncthreads();
    const int64_t p = p0 + w / (g * g);
    const int64_t I0 = 2 * p * s, J0 = I0 + s;
    if (J0 >= d) continue;
    const int64_t sJ = min<int64_t>(s, d - J0);
    const int64_t ti = (w / g) % g, tj = w % g;
    if (ti * 64 >= s || tj * 64 >= sJ) continue;
    const int64_t i0 = ti * 64, j0 = tj * 64;
    const double* Tp = T + (p - p0) * s * s;
    auto fa = [&](int ii, int64_t k) -> double {
      const int64_t i = i0 + ii;
      return (k >= i) ? R[(I0 + i) * d + I0 + k] : 0.0;
    };
    auto fb = [&](int64_t k, int jj) -> double {
      const int64_t j = j0 + jj;
      return (j < sJ) ? Tp[k * s + j] : 0.0;
    };
    f64x4 acc[2][2];
    zero_acc(acc);
    tile_gemm<false>(i0, s, fa, fb, acc);
    tile_store(acc, [&](int ii, int jj, double v) {
      const int64_t i = i0 + ii, j = j0 + jj;
      if (i < s && j < sJ) R[(I0 + i) * d + J0 + j] = -v;
    });
  }
}

// fp32 copy of R with its lower triangle zeroed: one workgroup per row,
// four columns per thread and pass.
__global__ __launch_bounds__(256) void r_to_f32_kernel(
    const double* __restrict__ R64, int64_t d, float* __restrict__ R) {
  const int64_t a = blockIdx.x;
  const double* src = R64 + a * d;
  float* dst = R + a * d;
  for (int64_t bb = threadIdx.x; bb < d; bb += 1024) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t b = bb + 256 * u;
      v[u] = (b >= a && b < d) ? static_cast<float>(src[b]) : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t b = bb + 256 * u;
      if (b < d) dst[b] = v[u];
    }
  }
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
  f.Tb = c.take<double>(size_t(std::max<int64_t>(tmax, 1)));
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
                           const int32_t* perm, const uint8_t* dead, bool ident,
                           const FactorWs& f, hipStream_t st) {
  build_h_kernel<<<static_cast<unsigned>(d), 256, 0, st>>>(S, d, n, perm, dead, f.damp,
                                                           ident ? 1 : 0, f.H);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

// at_split, when given, is called right after the launch of the step kernel
// of the block starting at column split_k: from there on the columns
// [split_k, d) of U (and R's diagonal blocks in them) are final.
gptq_status launch_cholesky_upper(int64_t d, const FactorWs& f, hipStream_t st,
                                  int64_t split_k,
                                  const std::function<gptq_status()>& at_split) {
  zero_flag_kernel<<<1, 1, 0, st>>>(f.flag);
  GPTQ_CHECK_LAUNCH();
  // 64-column blocks, 64-aligned from the top (the bottom one absorbs
  // d % 64), taken from the bottom in groups of kGroup.  Inside a group the
  // step kernels update only the group's own columns (and the diagonal tile
  // of the block after it); the rest of the trailing matrix receives the
  // whole group at once, one update with k = up to 64 kGroup.  Only the
  // bottom block's diagonal factor has a launch of its own: each step kernel
  // factors the next block's.
  int64_t k1 = d;
  {
    const int nb0 = static_cast<int>((d % kNb) ? (d % kNb) : kNb);
    chol_diag_kernel<<<1, 256, 0, st>>>(f.H, f.R, d, d - nb0, nb0, f.flag);
    GPTQ_CHECK_LAUNCH();
  }
  // the previous group's deferred trailing tiles: P = H[:, bk:bk+bK],
  // upper tiles with tile column < defer_tj
  int64_t bk = 0, defer_tj = 0;
  int bK = 0;
  while (k1 > 0) {
    const int64_t kend = k1;
    int64_t bk0[kGroup];
    int bnb[kGroup];
    int nb = 0;
    for (int64_t k = k1; nb < kGroup && k > 0; ++nb) {
      bnb[nb] = static_cast<int>((k % kNb) ? (k % kNb) : kNb);
      bk0[nb] = k - bnb[nb];
      k = bk0[nb];
    }
    const int64_t kg = bk0[nb - 1];
    int nl = 0;
    while (nl < nb && bk0[nl] > 0) ++nl;
    const int64_t ntask = defer_tj * (defer_tj + 1) / 2;
    // deferred tiles shared out in proportion to each launch's idle
    // workgroups (every launch has some: see the cap below)
    int64_t idle[kGroup], idle_sum = 0;
    for (int x = 0; x < nl; ++x) {
      idle[x] = std::max<int64_t>(0, kCUs - bk0[x] / 64);
      idle_sum += idle[x];
    }
    int64_t tdone = 0, idle_acc = 0;
    for (int x = 0; x < nl; ++x) {
      const int64_t nrow = bk0[x] / 64;
      idle_acc += idle[x];
      const int64_t ta = tdone;
      const int64_t tb = idle_sum > 0 ? ntask * idle_acc / idle_sum : 0;
      tdone = tb;
      const int64_t nbg = std::min<int64_t>(tb - ta, idle[x]);
      chol_step_kernel<<<static_cast<unsigned>(nrow + nbg), 256, 0, st>>>(
          f.H, f.R, d, bk0[x], bnb[x], x > 0 ? bk0[x - 1] : -1, x > 0 ? bnb[x - 1] : 0,
          kg, f.flag, bk, bK, ta, tb - ta);
      GPTQ_CHECK_LAUNCH();
      if (bk0[x] == split_k && at_split) {
        const gptq_status rc = at_split();
        if (rc != GPTQ_OK) return rc;
      }
    }
    // deferred work must have found a launch: it exists only when the next
    // group has all of its blocks below row 0
    if (ntask > 0 && nl == 0) return GPTQ_ERR_HIP;
    k1 = kg;
    defer_tj = 0;
    if (k1 > kNb) {
      // now: the tile columns the next group reads (its own columns and the
      // first block of the one after); the rest rides along with the next
      // group's step kernels
      const int64_t nt = cdiv(k1, 64);
      // deferred tiles must fit the next group's idle workgroups, at most
      // kBgTiles each: its launches have k1 / 64 - x - 1 row tiles
      int64_t cap = 0;
      for (int x = 0; x < kGroup; ++x)
        cap += kBgTiles * std::max<int64_t>(0, kCUs - (k1 / 64 - x - 1));
      int64_t tj0 = std::max<int64_t>(0, nt - (kGroup + 1));
      while (tj0 > 0 && tj0 * (tj0 + 1) / 2 > cap) --tj0;
      syrk_update_kernel<<<dim3(static_cast<unsigned>(nt - tj0), static_cast<unsigned>(nt)), 256, 0, st>>>(
          f.H, d, k1, static_cast<int>(kend - k1), tj0);
      GPTQ_CHECK_LAUNCH();
      defer_tj = tj0;
      bk = k1;
      bK = static_cast<int>(kend - k1);
    }
  }
  return GPTQ_OK;
}

namespace {

// One product of level s for pairs p0 .. p0 + np - 1 (T blocks in T), on
// at most max_wg workgroups.
gptq_status launch_trtri_t(int64_t d, const FactorWs& f, double* T, int64_t s,
                           int64_t p0, int64_t np, int64_t max_wg, hipStream_t st) {
  if (np <= 0) return GPTQ_OK;
  const int64_t g = (s + 63) / 64;
  const unsigned grid = static_cast<unsigned>(std::min<int64_t>(g * g * np, max_wg));
  trtri_t_kernel<<<grid, 256, 0, st>>>(f.H, f.R, T, d, s, p0, np);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

gptq_status launch_trtri_r(int64_t d, const FactorWs& f, const double* T, int64_t s,
                           int64_t p0, int64_t np, int64_t max_wg, hipStream_t st) {
  if (np <= 0) return GPTQ_OK;
  const int64_t g = (s + 63) / 64;
  const unsigned grid = static_cast<unsigned>(std::min<int64_t>(g * g * np, max_wg));
  trtri_r_kernel<<<grid, 256, 0, st>>>(f.R, T, d, s, p0, np);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

// Workgroups of the inverse's launches beside the factor: the step kernels
// keep the rest of the chip.
constexpr int64_t kSideWg = 160;
constexpr int64_t kAllWg = int64_t(1) << 30;

// A second stream per device (default priority, created on first use) and
// the two events that order it against the caller's stream.
struct SideStream {
  hipStream_t st = nullptr;
  hipEvent_t ready = nullptr, done = nullptr;
};
constexpr int kMaxDevices = 64;
std::mutex g_side_mu;
SideStream g_side[kMaxDevices];

// The second stream of the device that runs `caller` (the current device for
// the null stream), created with that device current.
gptq_status side_stream(hipStream_t caller, SideStream** out) {
  *out = nullptr;
  int dev = 0;
  if (caller)
    GPTQ_CHECK_HIP(hipStreamGetDevice(caller, &dev));
  else
    GPTQ_CHECK_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return GPTQ_OK;
  SideStream& sd = g_side[dev];
  if (!sd.st) {
    int cur = 0;
    GPTQ_CHECK_HIP(hipGetDevice(&cur));
    if (cur != dev) GPTQ_CHECK_HIP(hipSetDevice(dev));
    hipStream_t st = nullptr;
    hipEvent_t ready = nullptr, done = nullptr;
    const bool ok = hipStreamCreateWithFlags(&st, hipStreamNonBlocking) == hipSuccess &&
                    hipEventCreateWithFlags(&ready, hipEventDisableTiming) == hipSuccess &&
                    hipEventCreateWithFlags(&done, hipEventDisableTiming) == hipSuccess;
    if (cur != dev) GPTQ_CHECK_HIP(hipSetDevice(cur));
    if (!ok) return GPTQ_ERR_HIP;
    sd.ready = ready;
    sd.done = done;
    sd.st = st;
  }
  *out = &sd;
  return GPTQ_OK;
}

}  // namespace

// The reverse Cholesky H = U U^T followed by R = U^-1.  The inverse combines
// R's 64x64 diagonal blocks level by level; its top level pairs I = [0, s)
// with J = [s, d) (s the largest level).  The factor runs from the bottom
// up, so U's columns J are final once it has passed column s: from there
// the levels below the top inside J and the top level's T = U_IJ R_JJ run on
// a second stream, beside the factor of the columns I, which is latency
// bound and leaves most of the chip idle.  The rest (the levels inside I,
// then R_IJ = -R_II T) follows the factor on the caller's stream, after it
// has waited for the second stream.  The two streams touch disjoint parts of
// H, R and the scratch (T for the caller's stream, Tb for the other).
// Calls from several host threads are serialised while they enqueue.
gptq_status launch_factor_inverse(int64_t d, const FactorWs& f, hipStream_t st) {
  int64_t s_top = 0;
  for (int64_t s = kNb; s < d; s *= 2) s_top = s;
  std::lock_guard<std::mutex> lock(g_side_mu);
  SideStream* side = nullptr;
  if (s_top > 0) {
    const gptq_status rc = side_stream(st, &side);
    if (rc != GPTQ_OK) return rc;
  }
  if (!side) {
    // one stream: the factor, then every level in order
    const gptq_status rc = launch_cholesky_upper(d, f, st, -1, nullptr);
    if (rc != GPTQ_OK) return rc;
    for (int64_t s = kNb; s < d; s *= 2) {
      const int64_t np = cdiv(d, 2 * s);
      gptq_status r2;
      if ((r2 = launch_trtri_t(d, f, f.T, s, 0, np, kAllWg, st)) != GPTQ_OK) return r2;
      if ((r2 = launch_trtri_r(d, f, f.T, s, 0, np, kAllWg, st)) != GPTQ_OK) return r2;
    }
    return GPTQ_OK;
  }
  bool forked = false;
  auto at_split = [&]() -> gptq_status {
    GPTQ_CHECK_HIP(hipEventRecord(side->ready, st));
    GPTQ_CHECK_HIP(hipStreamWaitEvent(side->st, side->ready, 0));
    forked = true;
    gptq_status rc = GPTQ_OK;
    for (int64_t s = kNb; s < s_top && rc == GPTQ_OK; s *= 2) {
      const int64_t p0 = s_top / (2 * s);
      const int64_t np = int64_t(cdiv(d, 2 * s)) - p0;
      rc = launch_trtri_t(d, f, f.Tb, s, p0, np, kSideWg, side->st);
      if (rc == GPTQ_OK) rc = launch_trtri_r(d, f, f.Tb, s, p0, np, kSideWg, side->st);
    }
    if (rc == GPTQ_OK) rc = launch_trtri_t(d, f, f.Tb, s_top, 0, 1, kSideWg, side->st);
    // recorded even after a failed launch, so the caller's stream can join
    GPTQ_CHECK_HIP(hipEventRecord(side->done, side->st));
    return rc;
  };
  gptq_status rc = launch_cholesky_upper(d, f, st, s_top, at_split);
  for (int64_t s = kNb; s < s_top && rc == GPTQ_OK; s *= 2) {
    const int64_t np = s_top / (2 * s);
    rc = launch_trtri_t(d, f, f.T, s, 0, np, kAllWg, st);
    if (rc == GPTQ_OK) rc = launch_trtri_r(d, f, f.T, s, 0, np, kAllWg, st);
  }
  if (forked) GPTQ_CHECK_HIP(hipStreamWaitEvent(st, side->done, 0));
  if (rc != GPTQ_OK) return rc;
  if (!forked) return GPTQ_ERR_HIP;  // the factor never reached column s_top
  return launch_trtri_r(d, f, f.Tb, s_top, 0, 1, kAllWg, st);
}

gptq_status launch_r_to_f32(int64_t d, const FactorWs& f, float* R,
                            hipStream_t st) {
  r_to_f32_kernel<<<static_cast<unsigned>(d), 256, 0, st>>>(f.R, d, R);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

}  // namespace gptq
