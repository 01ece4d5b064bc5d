// The in-block column chain of the GPTQ loop, shared by the chain_*.hip
// instantiation units (each compiles a few template variants, so the build
// runs them in parallel).
//
// [teardown] Algorithm 1 and [derivation] section 10: for each column j of
// the block [i, i2) of the processing order
//   q = Delta (clip(round(w / Delta) + z, 0, maxq) - z)           (eq. (36))
//   eta = (w - q) / R_jj,  W[:, j:i2] -= eta R[j, j:i2]             (eq. (42))
// with the grid either fitted at a dynamic group start on the current
// working weights ([derivation] 8.3/8.4), fixed for the row, or fixed per
// static group (grid of position j = group floor(pi_j / g), 8.3).
//
// Rows are independent given R and their grids ([derivation] 2.3); each row
// is spread over the 16 lanes of one DPP row, lane q holding the block
// columns q, q + 16, ..., q + 112 in registers.  Per column the owning
// lane's residual is broadcast to the row with one DPP row_newbcast and
// every lane updates its own later columns.
#pragma once

#include "common.h"

namespace gptq {
namespace chain {

constexpr int kB = 128;        // largest block handled by one chain launch
constexpr int kRowLanes = 16;  // lanes per output row (one DPP row)
constexpr int kCols = kB / kRowLanes;   // block columns per lane
constexpr int kChainRows = 16; // output rows per 256-thread workgroup
constexpr int kTp = kChainRows + 1;     // LDS pitch of the row tiles

// FS modes of the chain kernel besides the dynamic-group granularities.
constexpr int kFsRow = 0;      // one grid for the whole row (no refits)
constexpr int kFsStatic = -1;  // a grid per column, fixed in advance

// Min-max grid widened to contain 0 (so z represents 0 exactly); a flat
// (all-zero) range becomes [-1, 1].  Delta = (hi - lo) / maxq,
// z = round(-lo / Delta), all in IEEE fp32.  The symmetric grid first
// widens the range to [-a, a], a = max(-lo, hi), with maxq = 2^b - 2 (2^b - 1
// levels -h..h around an exact 0, z = h; at 2 bits the ternary grid).
__device__ inline void fit_grid(float lo, float hi, float maxq, bool sym,
                                float& scale, float& zero) {
  if (sym) {
    hi = fmaxf(-lo, hi);
    lo = -hi;
  }
  if (hi == lo) {
    lo = -1.0f;
    hi = 1.0f;
  }
  scale = (hi - lo) / maxq;
  zero = fminf(fmaxf(rintf(-lo / scale), 0.0f), maxq);
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

// min / max over the 16 lanes of a row, by DPP inside the row: mirror
// (lane i with 15 - i), half mirror (i with 7 - i in each half of 8), then
// the two swaps inside each quad; after the second step each quad's four
// lanes together hold all sixteen values.  min and max are exact, so the
// order of the combination does not change the result.
template <int CTRL>
__device__ inline float row_dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

__device__ inline void row_minmax(float& lo, float& hi) {
  lo = fminf(lo, row_dpp<0x140>(lo));   // row_mirror
  hi = fmaxf(hi, row_dpp<0x140>(hi));
  lo = fminf(lo, row_dpp<0x141>(lo));   // row_half_mirror
  hi = fmaxf(hi, row_dpp<0x141>(hi));
  lo = fminf(lo, row_dpp<0x4E>(lo));    // quad_perm [2, 3, 0, 1]
  hi = fmaxf(hi, row_dpp<0x4E>(hi));
  lo = fminf(lo, row_dpp<0xB1>(lo));    // quad_perm [1, 0, 3, 2]
  hi = fmaxf(hi, row_dpp<0xB1>(hi));
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
// FS > 0: a dynamic group can only start at block offsets that are
// multiples of FS.  A group that starts inside the block ends inside it
// (checked on the host), so every fit sees fully compensated columns; a
// group that starts at the block start and reaches past it also reads its
// later columns from WT (compensated by every earlier block).  EXACT: the
// groups are FS columns long and the block starts on a group boundary.
// FS == kFsRow: the row's grid (scalesP row 0).  FS == kFsStatic: column
// i0 + c uses static group perm[i0 + c] / gsize of scalesP / zerosP.
// VEC: 0 = scalar global accesses, 1 = 16-byte ones (m % 4 == 0, WT and E
// 16-byte aligned, codes 4-byte aligned), 2 = 16-byte ones and a full
// 128-column block.  The R block is copied into LDS 16 bytes per lane in
// every mode (RL is 16-byte aligned).
// Stored codes: c = cz + z, or for signed grids (sgn: the symmetric grid,
// whose zero point is h = maxq / 2 everywhere) the low bits of c - h (two's
// complement, cmask = 2^b - 1), converted on the way out.
// The quotients w / Delta and rho / R_jj are products with fp32
// reciprocals; they differ from the IEEE quotients by at most an ulp, which
// can only matter within 1e-6 of a rounding boundary.
// nblk > 1 (full blocks of one lazy batch, VEC == 2): the launch runs the
// blocks i0, i0 + bi, ... one after the other for its rows; block u first
// takes the residuals of the blocks before it in the batch (rows are
// independent, so they are this workgroup's own, written by it to E and read
// back after a barrier).
template <int FS, int VEC, bool EXACT>
__global__ __launch_bounds__(256) void chain_kernel(
    const float* __restrict__ WT, int64_t m, int64_t d, const float* __restrict__ RL,
    int64_t i0_arg, int bw_arg, int bi, float maxq, int64_t gsize, int sym, int sgn,
    int cmask, const int32_t* __restrict__ perm,
    float* __restrict__ scalesP, uint8_t* __restrict__ zerosP,
    uint8_t* __restrict__ codesP, float* __restrict__ E_arg,
    const float* __restrict__ R, int64_t sb0, int kn_arg, const float* __restrict__ Esb,
    int nblk) {
  const int bw = VEC == 2 ? kB : bw_arg;
  constexpr int kSg = FS == kFsStatic ? kB : 1;
  __shared__ __attribute__((aligned(16))) float rl[kB * kB];
  __shared__ float tile[kB][kTp];
  __shared__ __attribute__((aligned(16))) uint8_t ctile[kB][kChainRows];
  __shared__ float sgs[kSg][kChainRows], sgz[kSg][kChainRows], sgi[kSg][kChainRows];
  for (int blk = 0; blk < nblk; ++blk) {
  const int64_t i0 = i0_arg + int64_t(blk) * bi;
  const int kn = kn_arg + blk * bi;
  float* __restrict__ E = E_arg + int64_t(blk) * bi * m;
  if (blk > 0) __syncthreads();   // the previous block's reads of rl / tile / ctile
  const int tid = threadIdx.x;
  const int rr = tid >> 4, q = tid & 15;
  const int64_t r0 = int64_t(blockIdx.x) * kChainRows;
  const int64_t r = r0 + rr;
  const bool act = r < m;
  const int64_t rs = act ? r : m - 1;
  // stage RL of this block (contiguous 64 KiB) and the block's columns of the
  // workgroup's rows (one 64-byte run per column)
  {
    // straight into LDS, no registers: each wave instruction copies 1 KiB,
    // lane l taking its bytes 16 l .. 16 l + 15
    typedef const void __attribute__((address_space(1)))* gvoid;
    typedef void __attribute__((address_space(3)))* lvoid;
    const char* src = reinterpret_cast<const char*>(RL + (i0 / bi) * int64_t(kB) * kB);
    char* dst = reinterpret_cast<char*>(rl);
    const int wv = tid >> 6, ln = tid & 63;
#pragma unroll
    for (int u = 0; u < kB * kB / 4 / 256; ++u) {
      const int chunk = u * 256 + wv * 64;
      __builtin_amdgcn_global_load_lds((gvoid)(src + 16 * (chunk + ln)), (lvoid)(dst + 16 * chunk),
                                       16, 0, 0);
    }
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
  if (FS == kFsStatic) {
    // the fixed grid of every block column for the workgroup's rows
#pragma unroll
    for (int u = 0; u < kB * kChainRows / 256; ++u) {
      const int e = tid + 256 * u;
      const int c = e / kChainRows, row = e % kChainRows;
      float s = 1.0f, z = 0.0f;
      if (c < bw) {
        const int64_t g = perm[i0 + c] / gsize;
        const int64_t rr2 = min(r0 + row, m - 1);
        s = scalesP[g * m + rr2];
        z = static_cast<float>(zerosP[g * m + rr2]);
      }
      sgs[c][row] = s;
      sgz[c][row] = z;
      sgi[c][row] = 1.0f / s;
    }
  }
  // the direct copies into LDS are counted by vmcnt, which the barrier does
  // not wait for
  __builtin_amdgcn_s_waitcnt((0 & 15) | ((0 >> 4) << 14) | (7 << 4) | (15 << 8));
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
  // earlier launch otherwise); static grids are read per column below
  float scale = 1.0f, zero = 0.0f, inv_scale = 1.0f;
  if (FS != kFsStatic) {
    const int64_t g0 = (FS == kFsRow) ? 0 : i0 / gsize;
    scale = scalesP[g0 * m + rs];
    zero = static_cast<float>(zerosP[g0 * m + rs]);
    inv_scale = 1.0f / scale;
  }
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
    if (FS == kFsStatic) {
      scale = sgs[k][rr];
      zero = sgz[k][rr];
      inv_scale = sgi[k][rr];
    }
    if (FS > 0 && k % (FS > 0 ? FS : 1) == 0 && (EXACT || (i0 + k) % gsize == 0)) {
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
      // (only a group that starts at the block start can reach past it)
      for (int64_t cc = i0 + bw + q; k == 0 && cc < gend; cc += kRowLanes) {
        const float x = WT[cc * m + rs];
        lo = fminf(lo, x);
        hi = fmaxf(hi, x);
      }
      row_minmax(lo, hi);
      fit_grid(lo, hi, maxq, sym != 0, scale, zero);
      inv_scale = 1.0f / scale;
      if (q == 0 && act) {
        scalesP[(col / gsize) * m + r] = scale;
        zerosP[(col / gsize) * m + r] = static_cast<uint8_t>(zero);
      }
    }
    // c - z = clamp(rint(x / scale), -z, maxq - z) (small integers, exact;
    // the clamp as one median-of-three),
    // and w - q = x - scale (c - z) in one rounding: six dependent
    // operations from the column's value to its residual
    const float x = w[tk];
    const float cz = __builtin_amdgcn_fmed3f(rintf(x * inv_scale), -zero, maxq - zero);
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
  // codes and residuals out through LDS, one coalesced run per column;
  // signed grids (zero point h = maxq / 2 throughout) store c - h
  __syncthreads();
  const int hz = static_cast<int>(maxq) / 2;
#pragma unroll
  for (int t = 0; t < kCols; ++t) {
    const int cidx = q + kRowLanes * t;
    tile[cidx][rr] = eta[t];
    const int c = static_cast<int>(code[t]);
    ctile[cidx][rr] = static_cast<uint8_t>(sgn ? ((c - hz) & cmask) : c);
  }
  __syncthreads();
  if (VEC && r0 + kChainRows <= m) {
    // four lanes per column, consecutive lanes on consecutive addresses:
    // 16-byte runs of E and 4-byte runs of codes (m % 4 == 0 here)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + 256 * u;
      const int c = e >> 2, p4 = 4 * (e & 3);
      if (c < bw) {
        const f32x4 v = {tile[c][p4], tile[c][p4 + 1], tile[c][p4 + 2], tile[c][p4 + 3]};
        *reinterpret_cast<f32x4*>(E + int64_t(c) * m + r0 + p4) = v;
        *reinterpret_cast<uint32_t*>(codesP + (i0 + c) * m + r0 + p4) =
            *reinterpret_cast<const uint32_t*>(&ctile[c][p4]);
      }
    }
  } else {
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
}

// Launches chain_kernel<FS, VEC, EXACT> for the VEC and EXACT the
// arguments allow.
template <int FS>
gptq_status launch_fs(const ChainArgs& a, hipStream_t st) {
  const bool vec = chain_vec(a);
  const dim3 grid(static_cast<unsigned>((a.m + kChainRows - 1) / kChainRows));
  // groups of exactly FS columns starting on an FS boundary: every FS-th
  // block column starts a group, known at compile time (the fits are then
  // straight-line code, which keeps the column loop free of branches)
  const bool exact = FS > 0 && a.gsize == FS && a.i0 % FS == 0;
#define GPTQ_CHAIN(V, X)                                                         \
  chain_kernel<FS, V, X><<<grid, 256, 0, st>>>(                                   \
      a.WT, a.m, a.d, a.RL, a.i0, a.bw, a.bi, a.maxq, a.gsize, a.sym, a.sgn,     \
      a.cmask, a.perm, a.scalesP, a.zerosP, a.codesP, a.E, a.R, a.sb0, a.kn, a.Esb, \
      a.nblk)
  if (a.nblk > 1 && !(vec && a.bw == kB)) return GPTQ_ERR_INVALID_ARG;
  if (vec && a.bw == kB) {
    if constexpr (FS > 0) {
      if (exact)
        GPTQ_CHAIN(2, true);
      else
        GPTQ_CHAIN(2, false);
    } else {
      GPTQ_CHAIN(2, false);
    }
  } else if (vec) {
    GPTQ_CHAIN(1, false);
  } else {
    GPTQ_CHAIN(0, false);
  }
#undef GPTQ_CHAIN
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

}  // namespace chain
}  // namespace gptq
