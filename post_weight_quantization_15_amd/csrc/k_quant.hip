// Column-by-column quantization with OBS feedback and lazy block updates.
//
// [teardown] Algorithm 1 and [derivation] section 10: for each block
// [i, i2) of the processing order and each column j in it
//   q = Delta (clip(round(w / Delta) + z, 0, 2^b - 1) - z)      (eq. (36))
//   eta = (w - q) / R_jj,  W[:, j:i2] -= eta R[j, j:i2]           (eq. (42))
// then W[:, i2:] -= E R[i:i2, i2:] with E = [eta_i .. eta_{i2-1}]  (eq. (46)).
// Dynamic groups refit Delta, z at each group start on the current working
// weights ([derivation] 8.3/8.4); the whole-row grid is fitted once on the
// original row ([derivation] section 10 pseudocode).
//
// Layout: the fp32 working copy is kept feature-major, WT[j][r] = W_work[r][j]
// (column j of the processing order is one contiguous vector over the m
// output rows), so reading a column, writing its codes and eta, and the
// lazy update all stream contiguous memory.
//
// Chain kernel: rows are independent given R and their grids ([derivation]
// 2.3); each row is spread over the 16 lanes of one DPP row, lane q holding
// the block columns q, q + 16, ..., q + 112 in registers.  Per column the
// owning lane's residual is broadcast to the row with one DPP row_newbcast
// and every lane updates its own later columns.
// Lazy update: v_mfma_f32_16x16x4_f32 (exact fp32 products, fp32 sums).
#include <algorithm>

#include "chain.h"

namespace gptq {
namespace {

using chain::kB;
using chain::kCols;
using chain::kRowLanes;

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }

// Grids fitted once on the ORIGINAL weights: the whole-row grid (g = d,
// [derivation] section 10) or the static groups (contiguous original
// columns [G g, (G + 1) g), 8.3).  One wave per (row, group); scale / zero
// land at [G][r].
template <class T>
__global__ __launch_bounds__(64) void fit_groups_kernel(
    const T* __restrict__ W, int64_t m, int64_t d, int64_t ldw, int64_t g,
    float maxq, int sym, float* __restrict__ scale, uint8_t* __restrict__ zero) {
  const int64_t r = blockIdx.x, G = blockIdx.y;
  const int64_t c0 = G * g, c1 = min(c0 + g, d);
  float lo = 0.0f, hi = 0.0f;
  for (int64_t c = c0 + threadIdx.x; c < c1; c += 64) {
    const float x = to_f32(W[r * ldw + c]);
    lo = fminf(lo, x);
    hi = fmaxf(hi, x);
  }
  for (int o = 32; o > 0; o >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, o));
    hi = fmaxf(hi, __shfl_xor(hi, o));
  }
  if (threadIdx.x == 0) {
    float s, z;
    chain::fit_grid(lo, hi, maxq, sym != 0, s, z);
    scale[G * m + r] = s;
    zero[G * m + r] = static_cast<uint8_t>(z);
  }
}

// A grid given by the caller ([m, n_g] row-major) into the [n_g][m] layout.
__global__ __launch_bounds__(256) void grid_in_kernel(
    const float* __restrict__ s_in, const uint8_t* __restrict__ z_in, int64_t m,
    int64_t ng, float* __restrict__ scale, uint8_t* __restrict__ zero) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e >= m * ng) return;
  const int64_t r = e / ng, G = e % ng;
  scale[G * m + r] = s_in[e];
  zero[G * m + r] = z_in[e];
}

__global__ void pinv_kernel(const int32_t* __restrict__ perm, int64_t d,
                            int32_t* __restrict__ pinv) {
  const int64_t j = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (j < d) pinv[perm[j]] = static_cast<int32_t>(j);
}

// WT[j][r] = dead[perm[j]] ? 0 : W[r][perm[j]]  via 64x64 LDS tiles.  Thread
// (row y = t / 4, quarter x = t % 4) reads columns 16x..16x+15 of row y (two
// 16-byte loads of bf16 when the order is the identity and the row allows
// it), then writes 16 consecutive rows of one column as four 16-byte stores
// (VEC: m % 4 == 0 and WT 16-byte aligned).
template <class T, bool VEC>
__global__ __launch_bounds__(256) void init_work_kernel(
    const T* __restrict__ W, int64_t m, int64_t d, int64_t ldw,
    const int32_t* __restrict__ perm, const uint8_t* __restrict__ dead,
    int ident, float* __restrict__ WT) {
  __shared__ float tile[64][65];       // [row][column]
  const int64_t r0 = int64_t(blockIdx.x) * 64, j0 = int64_t(blockIdx.y) * 64;
  const int t = threadIdx.x, y = t >> 2, x = t & 3;
  const int64_t r = r0 + y;
  const int64_t jb = j0 + 16 * x;
  bool wide = false;
  if constexpr (sizeof(T) == 2) {
    wide = ident && r < m && jb + 16 <= d &&
           (reinterpret_cast<uintptr_t>(W + r * ldw + jb) & 15) == 0;
  }
  if (wide) {
    const u32x4* p = reinterpret_cast<const u32x4*>(W + r * ldw + jb);
    const u32x4 a = p[0], b = p[1];
    const uint32_t wv[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t j = jb + 2 * u;
      tile[y][16 * x + 2 * u] = dead[j] ? 0.0f : __uint_as_float(wv[u] << 16);
      tile[y][16 * x + 2 * u + 1] = dead[j + 1] ? 0.0f : __uint_as_float(wv[u] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int64_t j = jb + u;
      float v = 0.0f;
      if (r < m && j < d) {
        const int32_t p = ident ? static_cast<int32_t>(j) : perm[j];
        if (!dead[p]) v = to_f32(W[r * ldw + p]);
      }
      tile[y][16 * x + u] = v;
    }
  }
  __syncthreads();
  // column jj = t / 4 of the tile, rows 16x..16x+15
  const int64_t j = j0 + y;
  if (j >= d) return;
  float* dst = WT + j * m + r0 + 16 * x;
  if (VEC && r0 + 16 * x + 16 <= m) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      reinterpret_cast<f32x4*>(dst)[u] = f32x4{tile[16 * x + 4 * u][y], tile[16 * x + 4 * u + 1][y],
                                               tile[16 * x + 4 * u + 2][y], tile[16 * x + 4 * u + 3][y]};
  } else {
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (r0 + 16 * x + u < m) dst[u] = tile[16 * x + u][y];
  }
}

// Diagonal blocks of R in the chain's lane order:
// RL[blk][k][q][t] = R[i + k][i + q + 16 t] for the block starting at
// i = blk * bi, k <= q + 16 t < bw (0 elsewhere, up to 128 x 128).  Row k
// of a block is then one 32-byte run per lane q.
__global__ __launch_bounds__(256) void rl_kernel(const float* __restrict__ R,
                                                 int64_t d, int bi,
                                                 float* __restrict__ RL) {
  const int64_t blk = blockIdx.y;
  const int64_t i = blk * bi;
  const int bw = static_cast<int>(min<int64_t>(bi, d - i));
  for (int e = threadIdx.x + blockIdx.x * 256; e < kB * kB; e += 256 * gridDim.x) {
    const int k = e / kB, q = (e / kCols) % kRowLanes, t = e % kCols;
    const int c = q + kRowLanes * t;
    RL[blk * kB * kB + e] = (k <= c && c < bw) ? R[(i + k) * d + i + c] : 0.0f;
  }
}

__global__ void zero_fill_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// WT[i2 + t][r] -= sum_k R[i0 + k][i2 + t] * E[k][r]   (t < d - i2, r < m).
// 256 threads = 2 x 2 waves, each a (16 NA) (t) x 64 (r) tile of NA x 4
// 16x16x4 MFMA blocks (NA = 4 or 2).  Lane l feeds A[row = l%16][k = l/16]
// and B[k = l/16][col = l%16] and receives D[row = 4(l/16) + v][col = l%16].
// Block a of a wave covers t = tw + a + NA row, block b covers
// r = rw + b + 4 col, so a lane's blocks touch NA consecutive t (or four
// consecutive r): operands arrive as one 8- or 16-byte load per k step and
// the final read-modify-write of W is one 16-byte access per (a, v).
// Operands are prefetched kDepth k steps ahead in a register ring; the W
// values to update are loaded before the product starts.  The narrow form
// (NA = 2) doubles the workgroups of a launch, for launches whose wide
// workgroups would leave part of the chip idle in their last round.
constexpr int kDepth = 8;

// Elements c0..c0+N-1 of a row, the address clamped into [0, lim).  Lanes
// whose columns fall past lim only feed outputs that are never stored, so
// the data needs no masking (a select on loaded data would pin the wait for
// the load next to the load).  Elements N..3 of the result are unused.
template <bool VEC, int N>
__device__ inline f32x4 load4(const float* row, int64_t c0, int64_t lim) {
  if (VEC) {   // lim, c0 multiples of 4 (lim >= 4), row 16-byte aligned
    const float* p = row + (c0 < lim ? c0 : lim - N);
    if (N == 4) return *reinterpret_cast<const f32x4*>(p);
    const float2 v = *reinterpret_cast<const float2*>(p);
    return f32x4{v.x, v.y, 0.f, 0.f};
  }
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < N; ++c) v[c] = row[min(c0 + c, lim - 1)];
  return v;
}

template <bool VEC, int KS, int NA>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void lazy_update_kernel(
    float* __restrict__ WT, int64_t m, int64_t d, const float* __restrict__ R,
    int64_t i0, int bw, const float* __restrict__ E) {
  const int64_t i2 = i0 + bw, nT = d - i2;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lk = lane >> 4;
  const int64_t tw = int64_t(blockIdx.y) * (32 * NA) + (wave >> 1) * (16 * NA);
  const int64_t rw = int64_t(blockIdx.x) * 128 + (wave & 1) * 64;
  const int64_t ta = tw + NA * lr, rb = rw + 4 * lr;
  const float* Rt = R + i0 * d + i2;       // Rt[k d + t]
  auto ldA = [&](int ks) -> f32x4 {
    const int k = 4 * ks + lk;
    return load4<VEC, NA>(Rt + int64_t(min(k, bw - 1)) * d, ta, nT);
  };
  auto ldB = [&](int ks) -> f32x4 {
    const int k = 4 * ks + lk;
    return load4<VEC, 4>(E + int64_t(k) * m, rb, m);     // rows >= bw are zero
  };
  f32x4 Wv[NA][4];
  auto ldW = [&]() {
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t t = tw + a + 4 * NA * lk + NA * v;
        Wv[a][v] = load4<VEC, 4>(WT + (i2 + min(t, nT - 1)) * m, rb, m);
      }
  };
  constexpr int kWAt = KS > 8 ? KS - 8 : 0;   // step after which W is fetched
  f32x4 acc[NA][4];
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  // KS k steps (4 k each) cover bw, fully unrolled; rows bw..4 KS - 1 of E
  // hold zeros, so the steps past bw add nothing.  Each step's MFMAs and the loads kDepth steps ahead are fenced
  // from the scheduler so that the loads stay that far ahead of their use.
  f32x4 A[kDepth], B[kDepth];
#pragma unroll
  for (int s = 0; s < kDepth && s < KS; ++s) {
    A[s] = ldA(s);
    B[s] = ldB(s);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int s = ks % kDepth;
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(A[s][a], B[s][b], acc[a][b], 0, 0, 0);
    if (ks + kDepth < KS) {
      A[s] = ldA(ks + kDepth);
      B[s] = ldB(ks + kDepth);
    }
    if (ks == kWAt) ldW();
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t t = tw + a + 4 * NA * lk + NA * v;
      if (t >= nT) continue;
      f32x4 x = Wv[a][v];
#pragma unroll
      for (int b = 0; b < 4; ++b) x[b] -= acc[a][b][v];
      float* row = WT + (i2 + t) * m;
      if (VEC) {
        if (rb < m) *reinterpret_cast<f32x4*>(row + rb) = x;
      } else {
#pragma unroll
        for (int b = 0; b < 4; ++b)
          if (rb + b < m) row[rb + b] = x[b];
      }
    }
}

unsigned cdiv(int64_t a, int64_t b) { return static_cast<unsigned>((a + b - 1) / b); }

template <bool VEC, int KS>
void lazy_launch(bool narrow, dim3 grid, hipStream_t st, float* WT, int64_t m,
                 int64_t d, const float* R, int64_t i0, int bw, const float* E) {
  if (narrow)
    lazy_update_kernel<VEC, KS, 2><<<grid, 256, 0, st>>>(WT, m, d, R, i0, bw, E);
  else
    lazy_update_kernel<VEC, KS, 4><<<grid, 256, 0, st>>>(WT, m, d, R, i0, bw, E);
}

}  // namespace

gptq_status launch_fit_grids(const void* W, gptq_dtype dt, int64_t m, int64_t d,
                             int64_t ldw, int64_t g, float maxq, int sym,
                             float* scalesP, uint8_t* zerosP, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(m), cdiv(d, g));
  if (dt == GPTQ_F32)
    fit_groups_kernel<float><<<grid, 64, 0, st>>>(
        static_cast<const float*>(W), m, d, ldw, g, maxq, sym, scalesP, zerosP);
  else
    fit_groups_kernel<uint16_t><<<grid, 64, 0, st>>>(
        static_cast<const uint16_t*>(W), m, d, ldw, g, maxq, sym, scalesP, zerosP);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

gptq_status launch_grid_in(const float* s_in, const uint8_t* z_in, int64_t m,
                           int64_t ng, float* scalesP, uint8_t* zerosP,
                           hipStream_t st) {
  grid_in_kernel<<<cdiv(m * ng, 256), 256, 0, st>>>(s_in, z_in, m, ng, scalesP, zerosP);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

gptq_status launch_init_work(const void* W, gptq_dtype dt, int64_t m,
                             int64_t d, int64_t ldw, const int32_t* perm,
                             const uint8_t* dead, bool ident, float* WT,
                             int32_t* pinv, hipStream_t st) {
  pinv_kernel<<<cdiv(d, 256), 256, 0, st>>>(perm, d, pinv);
  GPTQ_CHECK_LAUNCH();
  const dim3 grid(cdiv(m, 64), cdiv(d, 64));
  const bool vec = m % 4 == 0 && reinterpret_cast<uintptr_t>(WT) % 16 == 0;
#define GPTQ_INIT(TY, V) init_work_kernel<TY, V><<<grid, 256, 0, st>>>( \
      static_cast<const TY*>(W), m, d, ldw, perm, dead, ident ? 1 : 0, WT)
  if (dt == GPTQ_F32) {
    if (vec) GPTQ_INIT(float, true); else GPTQ_INIT(float, false);
  } else {
    if (vec) GPTQ_INIT(uint16_t, true); else GPTQ_INIT(uint16_t, false);
  }
#undef GPTQ_INIT
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

gptq_status launch_rbt(const float* R, int64_t d, int bi, float* RL,
                       hipStream_t st) {
  const int64_t nblk = (d + bi - 1) / bi;
  rl_kernel<<<dim3(8, static_cast<unsigned>(nblk)), 256, 0, st>>>(R, d, bi, RL);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

gptq_status launch_chain(const ChainArgs& a, hipStream_t st) {
  if (a.kn % 32 != 0) return GPTQ_ERR_INVALID_ARG;
  if (a.fs == chain::kFsStatic) return launch_chain_static(a, st);
  if (a.fs == chain::kFsRow) return launch_chain_row(a, st);
  // dynamic groups: the largest instantiated granularity that divides g
  if (a.gsize % 128 == 0) return launch_chain_g128(a, st);
  if (a.gsize % 64 == 0) return launch_chain_g64(a, st);
  if (a.gsize % 8 == 0) return launch_chain_g8(a, st);
  return launch_chain_g1(a, st);
}

gptq_status launch_lazy_update(float* WT, int64_t m, int64_t d, const float* R,
                               int64_t i0, int bw, float* E,
                               hipStream_t st) {
  const int64_t nT = d - i0 - bw;
  if (nT <= 0) return GPTQ_OK;
  // Workgroups run one per CU at a time here, each for a time about
  // proportional to its tile; the narrow tile (half the work, a little less
  // efficient per product) is taken when its rounds of kCUs workgroups come
  // out shorter.
  constexpr int64_t kCUs = 256;
  const int64_t wg_wide = int64_t(cdiv(m, 128)) * cdiv(nT, 128);
  const int64_t wg_narrow = int64_t(cdiv(m, 128)) * cdiv(nT, 64);
  const bool narrow = 0.6 * double((wg_narrow + kCUs - 1) / kCUs) <
                      double((wg_wide + kCUs - 1) / kCUs);
  const dim3 grid(cdiv(m, 128), cdiv(nT, narrow ? 64 : 128));
  // 16-byte accesses need every row start and column offset 4-aligned
  const bool vec = m % 4 == 0 && d % 4 == 0 && (i0 + bw) % 4 == 0 &&
                   reinterpret_cast<uintptr_t>(R) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(WT) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(E) % 16 == 0;
  const int ks = (bw + 3) / 4;      // k steps; bw <= 4 kLazyMaxKs
  const int kpad = ks <= 4 ? 16 : ks <= 8 ? 32 : ks <= 16 ? 64 : ks <= 32 ? 128 : ks <= 64 ? 256 : 512;
  if (kpad > bw) {     // rows of E the product reads past bw must be zero
    const int64_t n = int64_t(kpad - bw) * m;
    zero_fill_kernel<<<cdiv(n, 256), 256, 0, st>>>(E + int64_t(bw) * m, n);
  }
#define GPTQ_LAZY(V, K) lazy_launch<V, K>(narrow, grid, st, WT, m, d, R, i0, bw, E)
#define GPTQ_LAZY_KS(V)                        \
  if (ks <= 4) GPTQ_LAZY(V, 4);                 \
  else if (ks <= 8) GPTQ_LAZY(V, 8);            \
  else if (ks <= 16) GPTQ_LAZY(V, 16);          \
  else if (ks <= 32) GPTQ_LAZY(V, 32);          \
  else if (ks <= 64) GPTQ_LAZY(V, 64);          \
  else GPTQ_LAZY(V, 128);
  if (vec) {
    GPTQ_LAZY_KS(true)
  } else {
    GPTQ_LAZY_KS(false)
  }
#undef GPTQ_LAZY_KS
#undef GPTQ_LAZY
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

}  // namespace gptq
