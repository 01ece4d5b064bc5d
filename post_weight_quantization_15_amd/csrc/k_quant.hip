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

#include "common.h"

namespace gptq {
namespace {

constexpr int kB = 128;        // largest block handled by one chain launch
constexpr int kRowLanes = 16;  // lanes per output row (one DPP row)
constexpr int kCols = kB / kRowLanes;   // block columns per lane
constexpr int kChainRows = 16; // output rows per 256-thread workgroup
constexpr int kTp = kChainRows + 1;     // LDS pitch of the row tiles

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }

// Min-max grid widened to contain 0 (so z represents 0 exactly); a flat
// (all-zero) range becomes [-1, 1].  Delta = (hi - lo) / (2^b - 1),
// z = round(-lo / Delta), all in IEEE fp32.
__device__ inline void fit_grid(float lo, float hi, float maxq, float& scale,
                                float& zero) {
  if (hi == lo) {
    lo = -1.0f;
    hi = 1.0f;
  }
  scale = (hi - lo) / maxq;
  zero = fminf(fmaxf(rintf(-lo / scale), 0.0f), maxq);
}

// Whole-row grid on the original weights: one wave per row.
template <class T>
__global__ __launch_bounds__(64) void fit_rows_kernel(
    const T* __restrict__ W, int64_t d, int64_t ldw, float maxq,
    float* __restrict__ scale, uint8_t* __restrict__ zero) {
  const int64_t r = blockIdx.x;
  float lo = 0.0f, hi = 0.0f;
  for (int64_t c = threadIdx.x; c < d; c += 64) {
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
    fit_grid(lo, hi, maxq, s, z);
    scale[r] = s;
    zero[r] = static_cast<uint8_t>(z);
  }
}

__global__ void pinv_kernel(const int32_t* __restrict__ perm, int64_t d,
                            int32_t* __restrict__ pinv) {
  const int64_t j = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (j < d) pinv[perm[j]] = static_cast<int32_t>(j);
}

// WT[j][r] = dead[perm[j]] ? 0 : W[r][perm[j]]  via 64x64 LDS tiles.
template <class T>
__global__ __launch_bounds__(256) void init_work_kernel(
    const T* __restrict__ W, int64_t m, int64_t d, int64_t ldw,
    const int32_t* __restrict__ perm, const uint8_t* __restrict__ dead,
    float* __restrict__ WT) {
  __shared__ float tile[64][65];
  const int64_t r0 = int64_t(blockIdx.x) * 64, j0 = int64_t(blockIdx.y) * 64;
  const int lx = threadIdx.x & 63, ly = threadIdx.x >> 6;
  const int64_t j = j0 + lx;
  int64_t src = -1;
  if (j < d) {
    const int32_t p = perm[j];
    if (!dead[p]) src = p;
  }
  for (int y = ly; y < 64; y += 4) {
    const int64_t r = r0 + y;
    tile[y][lx] = (r < m && src >= 0) ? to_f32(W[r * ldw + src]) : 0.0f;
  }
  __syncthreads();
  for (int y = ly; y < 64; y += 4) {
    const int64_t jj = j0 + y, r = r0 + lx;
    if (jj < d && r < m) WT[jj * m + r] = tile[lx][y];
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

__device__ inline float row_bcast(float x, int src) {
  // DPP row_newbcast: lane src of every 16-lane row to the whole row
  switch (src) {
#define GPTQ_BC(L) case L: return __int_as_float(__builtin_amdgcn_update_dpp( \
      0, __float_as_int(x), 0x150 + L, 0xF, 0xF, false));
    GPTQ_BC(0) GPTQ_BC(1) GPTQ_BC(2) GPTQ_BC(3) GPTQ_BC(4) GPTQ_BC(5)
    GPTQ_BC(6) GPTQ_BC(7) GPTQ_BC(8) GPTQ_BC(9) GPTQ_BC(10) GPTQ_BC(11)
    GPTQ_BC(12) GPTQ_BC(13) GPTQ_BC(14) GPTQ_BC(15)
#undef GPTQ_BC
  }
  return x;
}

// min / max over the 16 lanes of a row
__device__ inline void row_minmax(float& lo, float& hi) {
#pragma unroll
  for (int o = 1; o < kRowLanes; o <<= 1) {
    lo = fminf(lo, __shfl_xor(lo, o));
    hi = fmaxf(hi, __shfl_xor(hi, o));
  }
}

// One block [i0, i0 + bw) of the column loop for 16 output rows per
// workgroup.  Thread (row rr = tid / 16, lane q = tid % 16) holds w[t] =
// W_work[r0 + rr][i0 + q + 16 t].  For each column k (owner lane k % 16, slot
// k / 16): every lane quantizes its slot-k/16 value, the owner's residual
// eta = (w - q) / R_kk is broadcast over the row, and each lane applies
// w[t] -= eta R[k][q + 16 t] for its later slots (R is upper triangular, so
// slots at or before column k receive 0).  This is the in-block step of
// the column loop ([derivation] eq. (42)); the block's R is read from LDS in
// the RL lane order.
// FS: a dynamic group can only start at block offsets that are multiples of
// FS (0 = the whole-row grid, no refits).  A group that starts inside the
// block ends inside it (checked on the host), so every fit sees fully
// compensated columns; a group that starts at the block start and reaches
// past it also reads its later columns from WT (compensated by every
// earlier block).
// VEC: 0 = scalar global accesses, 1 = 16-byte ones, 2 = 16-byte ones and
// a full 128-column block.
// The quotients w / Delta and rho / R_jj are products with fp32
// reciprocals; they differ from the IEEE quotients by at most an ulp, which
// can only matter within 1e-6 of a rounding boundary.
template <int FS, int VEC>
__global__ __launch_bounds__(256) void chain_kernel(
    const float* __restrict__ WT, int64_t m, int64_t d, const float* __restrict__ RL,
    int64_t i0, int bw_arg, int bi, float maxq, int64_t gsize,
    float* __restrict__ scalesP, uint8_t* __restrict__ zerosP,
    uint8_t* __restrict__ codesP, float* __restrict__ E,
    const float* __restrict__ R, int64_t sb0, int kn, const float* __restrict__ Esb) {
  const int bw = VEC == 2 ? kB : bw_arg;
  __shared__ __attribute__((aligned(16))) float rl[kB * kB];
  __shared__ float tile[kB][kTp];
  __shared__ uint8_t ctile[kB][kChainRows];
  const int tid = threadIdx.x;
  const int rr = tid >> 4, q = tid & 15;
  const int64_t r0 = int64_t(blockIdx.x) * kChainRows;
  const int64_t r = r0 + rr;
  const bool act = r < m;
  const int64_t rs = act ? r : m - 1;
  // stage RL of this block (contiguous 64 KiB) and the block's columns of the
  // workgroup's rows (one 64-byte run per column)
  {
    const f32x4* src = reinterpret_cast<const f32x4*>(RL + (i0 / bi) * int64_t(kB) * kB);
    f32x4* dst = reinterpret_cast<f32x4*>(rl);
    f32x4 buf[kB * kB / 4 / 256];
#pragma unroll
    for (int u = 0; u < kB * kB / 4 / 256; ++u) buf[u] = src[tid + 256 * u];
#pragma unroll
    for (int u = 0; u < kB * kB / 4 / 256; ++u) dst[tid + 256 * u] = buf[u];
  }
  {
    const int c = tid >> 1, h = tid & 1;
    float v[8];
    if (c < bw) {
      const float* col = WT + (i0 + c) * m + r0 + 8 * h;
      if (VEC && r0 + 8 * h + 8 <= m) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(col);
        const f32x4 b = *reinterpret_cast<const f32x4*>(col + 4);
        v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
        v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = (r0 + 8 * h + u < m) ? col[u] : 0.0f;
      }
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) tile[c][8 * h + u] = v[u];
  }
  __syncthreads();
  if (kn > 0) {
    // the earlier blocks of this lazy batch, not yet applied to WT:
    // tile[c][rr] -= sum_{k < kn} Esb[k][r0 + rr] R[sb0 + k][i0 + c]
    // (wave wv: columns 32 wv .. 32 wv + 31 as two 16 x 16 MFMA blocks)
    const int wv = tid >> 6, l = tid & 63, lr = l & 15, lk = l >> 4;
    const float* Ea = Esb + min(r0 + lr, m - 1);
    const float* Rb0 = R + sb0 * d + min(i0 + 32 * wv + lr, d - 1);
    const float* Rb1 = R + sb0 * d + min(i0 + 32 * wv + 16 + lr, d - 1);
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    // 32 k per batch (kn is a multiple of 32), the next batch's loads in
    // flight during the current batch's products
    float a[2][8], b0[2][8], b1[2][8];
    auto fetch = [&](int buf, int k0) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t k = k0 + 4 * u + lk;
        a[buf][u] = Ea[k * m];
        b0[buf][u] = Rb0[k * d];
        b1[buf][u] = Rb1[k * d];
      }
    };
    auto mma = [&](int buf) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[buf][u], b0[buf][u], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[buf][u], b1[buf][u], acc1, 0, 0, 0);
      }
    };
    fetch(0, 0);
    for (int k0 = 0; k0 < kn; k0 += 64) {
      if (k0 + 32 < kn) fetch(1, k0 + 32);
      mma(0);
      if (k0 + 32 >= kn) break;
      if (k0 + 64 < kn) fetch(0, k0 + 64);
      mma(1);
    }
    // D[row 4 lk + v][column lr] of each block
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      tile[32 * wv + lr][4 * lk + v] -= acc0[v];
      tile[32 * wv + 16 + lr][4 * lk + v] -= acc1[v];
    }
    __syncthreads();
  }
  float w[kCols], rinv[kCols], eta[kCols], code[kCols];
#pragma unroll
  for (int t = 0; t < kCols; ++t) {
    const int c = q + kRowLanes * t;
    w[t] = tile[c][rr];
    const float rjj = rl[(c * kRowLanes + q) * kCols + t];
    rinv[t] = c < bw ? 1.0f / rjj : 0.0f;
    eta[t] = 0.0f;
    code[t] = 0.0f;
  }
  // grid in force at the block start: the row grid, or the dynamic group
  // that contains column i0 (fitted by this launch if it starts here, by an
  // earlier launch otherwise)
  const int64_t g0 = (FS == 0) ? 0 : i0 / gsize;
  float scale = scalesP[g0 * m + rs];
  float zero = static_cast<float>(zerosP[g0 * m + rs]);
  float inv_scale = 1.0f / scale;
  // R rows of the next kPf columns in registers (the LDS latency stays off
  // the column-to-column dependence)
  constexpr int kPf = 4;
  f32x4 pa[kPf], pb[kPf];
#pragma unroll
  for (int p = 0; p < kPf; ++p) {
    const float* rp = rl + (p * kRowLanes + q) * kCols;
    pa[p] = *reinterpret_cast<const f32x4*>(rp);
    pb[p] = *reinterpret_cast<const f32x4*>(rp + 4);
  }
#pragma clang loop unroll(full)
  for (int tk = 0; tk < kCols; ++tk) {
#pragma clang loop unroll(full)
  for (int qk = 0; qk < kRowLanes; ++qk) {
    const int k = kRowLanes * tk + qk;
    // uniform: columns past a partial block (a full block has none, and
    // its column steps are one straight run the compiler can pipeline)
    if (VEC != 2 && k >= bw) continue;
    if (FS > 0 && k % (FS > 0 ? FS : 1) == 0 && (i0 + k) % gsize == 0) {
      const int64_t col = i0 + k;
      const int64_t gend = min(col + gsize, d);
      float lo = 0.0f, hi = 0.0f;
#pragma unroll
      for (int t = tk; t < kCols; ++t) {
        const int64_t c = i0 + q + kRowLanes * t;
        if (c >= col && c < gend && c < i0 + bw) {
          lo = fminf(lo, w[t]);
          hi = fmaxf(hi, w[t]);
        }
      }
      for (int64_t cc = i0 + bw + q; cc < gend; cc += kRowLanes) {
        const float x = WT[cc * m + rs];
        lo = fminf(lo, x);
        hi = fmaxf(hi, x);
      }
      row_minmax(lo, hi);
      fit_grid(lo, hi, maxq, scale, zero);
      inv_scale = 1.0f / scale;
      if (q == 0 && act) {
        scalesP[(col / gsize) * m + r] = scale;
        zerosP[(col / gsize) * m + r] = static_cast<uint8_t>(zero);
      }
    }
    // c - z = clamp(rint(x / scale), -z, maxq - z) (small integers, exact),
    // and w - q = x - scale (c - z) in one rounding: six dependent
    // operations from the column's value to its residual
    const float x = w[tk];
    const float cz = fminf(fmaxf(rintf(x * inv_scale), -zero), maxq - zero);
    const float e = fmaf(-scale, cz, x) * rinv[tk];
    if (q == qk) {
      code[tk] = cz + zero;
      eta[tk] = e;
    }
    const float eb = row_bcast(e, qk);
    const int sl = k % kPf;
    const f32x4 ra = pa[sl], rb = pb[sl];
    // keep every element of this column's rows live up to here: a row
    // register with a dead element could be reused while its load is in
    // flight, which would make the next load wait
    asm volatile("" :: "v"(ra), "v"(rb));
    if (k + kPf < kB) {
      const float* rp = rl + ((k + kPf) * kRowLanes + q) * kCols;
      if (k + kPf < 4 * kRowLanes) pa[sl] = *reinterpret_cast<const f32x4*>(rp);
      pb[sl] = *reinterpret_cast<const f32x4*>(rp + 4);
    }
    if (tk < 4) {
#pragma unroll
      for (int t = tk; t < 4; ++t) w[t] = fmaf(-eb, ra[t], w[t]);
    }
#pragma unroll
    for (int t = (tk > 4 ? tk : 4); t < kCols; ++t) w[t] = fmaf(-eb, rb[t - 4], w[t]);
  }
  }
  // codes and residuals out through LDS, one coalesced run per column
  __syncthreads();
#pragma unroll
  for (int t = 0; t < kCols; ++t) {
    const int cidx = q + kRowLanes * t;
    tile[cidx][rr] = eta[t];
    ctile[cidx][rr] = static_cast<uint8_t>(code[t]);
  }
  __syncthreads();
  {
    const int c = tid >> 1, h = tid & 1;
    if (c < bw) {
      float* erow = E + int64_t(c) * m + r0 + 8 * h;
      uint8_t* crow = codesP + (i0 + c) * m + r0 + 8 * h;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (r0 + 8 * h + u < m) {
          erow[u] = tile[c][8 * h + u];
          crow[u] = ctile[c][8 * h + u];
        }
    }
  }
}

__global__ void zero_fill_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// WT[i2 + t][r] -= sum_k R[i0 + k][i2 + t] * E[k][r]   (t < d - i2, r < m).
// 256 threads = 2 x 2 waves, each a 64 (t) x 64 (r) tile of 4 x 4
// 16x16x4 MFMA blocks.  Lane l feeds A[row = l%16][k = l/16] and
// B[k = l/16][col = l%16] and receives D[row = 4(l/16) + v][col = l%16].
// Block a of a wave covers t = tw + a + 4 row, block b covers
// r = rw + b + 4 col, so a lane's four blocks touch four consecutive t (or r):
// operands arrive as one 16-byte load per k step and the final
// read-modify-write of W is one 16-byte access per (a, v).  Operands are
// prefetched kDepth k steps ahead in a register ring; the W values to update
// are loaded before the product starts.
constexpr int kDepth = 4;

// Elements c0..c0+3 of a row, the address clamped into [0, lim).  Lanes
// whose columns fall past lim only feed outputs that are never stored, so
// the data needs no masking (a select on loaded data would pin the wait for
// the load next to the load).
template <bool VEC>
__device__ inline f32x4 load4(const float* row, int64_t c0, int64_t lim) {
  if (VEC)     // lim, c0 multiples of 4 (lim >= 4), row 16-byte aligned
    return *reinterpret_cast<const f32x4*>(row + (c0 < lim ? c0 : lim - 4));
  f32x4 v;
#pragma unroll
  for (int c = 0; c < 4; ++c) v[c] = row[min(c0 + c, lim - 1)];
  return v;
}

template <bool VEC, int KS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void lazy_update_kernel(
    float* __restrict__ WT, int64_t m, int64_t d, const float* __restrict__ R,
    int64_t i0, int bw, const float* __restrict__ E) {
  const int64_t i2 = i0 + bw, nT = d - i2;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lk = lane >> 4;
  const int64_t tw = int64_t(blockIdx.y) * 128 + (wave >> 1) * 64;
  const int64_t rw = int64_t(blockIdx.x) * 128 + (wave & 1) * 64;
  const int64_t ta = tw + 4 * lr, rb = rw + 4 * lr;
  const float* Rt = R + i0 * d + i2;       // Rt[k d + t]
  auto ldA = [&](int ks) -> f32x4 {
    const int k = 4 * ks + lk;
    return load4<VEC>(Rt + int64_t(min(k, bw - 1)) * d, ta, nT);
  };
  auto ldB = [&](int ks) -> f32x4 {
    const int k = 4 * ks + lk;
    return load4<VEC>(E + int64_t(k) * m, rb, m);     // rows >= bw are zero
  };
  f32x4 Wv[4][4];
  auto ldW = [&]() {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t t = tw + a + 16 * lk + 4 * v;
        Wv[a][v] = load4<VEC>(WT + (i2 + min(t, nT - 1)) * m, rb, m);
      }
  };
  constexpr int kWAt = KS > 8 ? KS - 8 : 0;   // step after which W is fetched
  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
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
    for (int a = 0; a < 4; ++a)
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
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t t = tw + a + 16 * lk + 4 * v;
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

}  // namespace

gptq_status launch_fit_rows(const void* W, gptq_dtype dt, int64_t m, int64_t d,
                            int64_t ldw, int bits, float* scale, uint8_t* zero,
                            hipStream_t st) {
  const float maxq = static_cast<float>((1 << bits) - 1);
  if (dt == GPTQ_F32)
    fit_rows_kernel<float><<<static_cast<unsigned>(m), 64, 0, st>>>(
        static_cast<const float*>(W), d, ldw, maxq, scale, zero);
  else
    fit_rows_kernel<uint16_t><<<static_cast<unsigned>(m), 64, 0, st>>>(
        static_cast<const uint16_t*>(W), d, ldw, maxq, scale, zero);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

gptq_status launch_init_work(const void* W, gptq_dtype dt, int64_t m,
                             int64_t d, int64_t ldw, const int32_t* perm,
                             const uint8_t* dead, float* WT, int32_t* pinv,
                             hipStream_t st) {
  pinv_kernel<<<cdiv(d, 256), 256, 0, st>>>(perm, d, pinv);
  GPTQ_CHECK_LAUNCH();
  const dim3 grid(cdiv(m, 64), cdiv(d, 64));
  if (dt == GPTQ_F32)
    init_work_kernel<float><<<grid, 256, 0, st>>>(static_cast<const float*>(W), m, d, ldw, perm, dead, WT);
  else
    init_work_kernel<uint16_t><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(W), m, d, ldw, perm, dead, WT);
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

gptq_status launch_chain(float* WT, int64_t m, int64_t d, const float* RL,
                         int64_t i0, int bw, int bi, int bits, int64_t gsize,
                         float* scalesP, uint8_t* zerosP, uint8_t* codesP,
                         float* E, const float* R, int64_t sb0, const float* Esb,
                         hipStream_t st) {
  const int kn = static_cast<int>(i0 - sb0);
  if (kn % 32 != 0) return GPTQ_ERR_INVALID_ARG;
  const float maxq = static_cast<float>((1 << bits) - 1);
  int fs = 0;
  if (gsize > 0) {
    fs = 1;
    while (fs < kB && gsize % (2 * fs) == 0) fs *= 2;
  }
  const bool vec = m % 4 == 0 && reinterpret_cast<uintptr_t>(WT) % 16 == 0;
  const dim3 grid(cdiv(m, kChainRows));
#define GPTQ_CHAIN(FSV, V)                                                     \
  chain_kernel<FSV, V><<<grid, 256, 0, st>>>(WT, m, d, RL, i0, bw, bi, maxq,  \
                                             gsize, scalesP, zerosP, codesP, E, \
                                             R, sb0, kn, Esb)
#define GPTQ_CHAIN_FS(V)                     \
  switch (fs) {                              \
    case 0: GPTQ_CHAIN(0, V); break;         \
    case 1: GPTQ_CHAIN(1, V); break;         \
    case 2: GPTQ_CHAIN(2, V); break;         \
    case 4: GPTQ_CHAIN(4, V); break;         \
    case 8: GPTQ_CHAIN(8, V); break;         \
    case 16: GPTQ_CHAIN(16, V); break;       \
    case 32: GPTQ_CHAIN(32, V); break;       \
    case 64: GPTQ_CHAIN(64, V); break;       \
    default: GPTQ_CHAIN(128, V); break;      \
  }
  if (vec && bw == kB) {
    GPTQ_CHAIN_FS(2)
  } else if (vec) {
    GPTQ_CHAIN_FS(1)
  } else {
    GPTQ_CHAIN_FS(0)
  }
#undef GPTQ_CHAIN_FS
#undef GPTQ_CHAIN
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

gptq_status launch_lazy_update(float* WT, int64_t m, int64_t d, const float* R,
                               int64_t i0, int bw, float* E,
                               hipStream_t st) {
  const int64_t nT = d - i0 - bw;
  if (nT <= 0) return GPTQ_OK;
  const dim3 grid(cdiv(m, 128), cdiv(nT, 128));
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
#define GPTQ_LAZY(V, K) lazy_update_kernel<V, K><<<grid, 256, 0, st>>>(WT, m, d, R, i0, bw, E)
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
