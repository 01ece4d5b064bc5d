// Hessian statistics S += X^T X for token-major activations X [n_tok, d].
//
// [derivation] eq. (9): H = (2/N) X X^T with X = reshape(A, [N, d])^T
// (eq. (5)); the sum is additive over calibration chunks (section 9.4).
//
// bf16 path (the hot path): one wave64 per (128x128 upper-triangle tile of S,
// token split).  The contraction runs over tokens, the strided dimension of
// the token-major input, so each lane gathers an 8-token x 8-feature block
// with eight 16-byte loads and transposes it in registers into eight
// 8-token fragments, one per feature.  A lane group (lane / 16) owns 8 tokens
// of a 32-token step and lane % 16 selects 8 features, so fragment f of all
// lanes is the A (or B) operand of one v_mfma_f32_16x16x32_bf16 whose
// 16 rows are the features F0 + 8*i + f, i = 0..15.  8 x 8 such MFMAs cover
// the 128 x 128 tile; no LDS is used.  bf16 x bf16 products are exact in
// fp32 and accumulate in fp32.  Token splits write fp32 partial tiles that a
// second kernel adds to S in a fixed order (bitwise reproducible).
//
// fp32 path: plain tiled kernel accumulating in fp64 (small inputs).
#include <algorithm>

#include "common.h"

namespace gptq {
namespace {

constexpr int kTile = 128;
constexpr int kStep = 32;
constexpr int kTargetWaves = 1024;   // 256 CUs x 4 SIMDs, one wave per SIMD

__host__ __device__ inline int64_t upper_tiles(int64_t nt) { return nt * (nt + 1) / 2; }

__device__ inline void tile_of(int64_t L, int nt, int& ti, int& tj) {
  int t = 0;
  int64_t rem = L;
  while (rem >= nt - t) {
    rem -= nt - t;
    ++t;
  }
  ti = t;
  tj = t + static_cast<int>(rem);
}

// XCD-aware work order.  Workgroup w runs on XCD w % 8, in dispatch order
// within its XCD.  The upper tiles are enumerated block-major (blocks of
// kRegB x kRegB tiles, row-major over the upper block triangle, row-major
// inside a block) and cut into 8 consecutive regions, one per XCD; each XCD
// walks its region split by split.  Concurrent waves of one XCD therefore
// read the same token window of a compact set of panels, which its L2 can
// serve, instead of every XCD streaming every panel.
constexpr int kRegB = 8;
constexpr int kXcd = 8;

__device__ inline void blocked_tile(int64_t t, int nt, int& ti, int& tj) {
  const int nb = (nt + kRegB - 1) / kRegB;
  for (int br = 0; br < nb; ++br) {
    const int r0 = br * kRegB, rh = min(kRegB, nt - r0);
    for (int bc = br; bc < nb; ++bc) {
      const int c0 = bc * kRegB, cw = min(kRegB, nt - c0);
      const int64_t size = (bc == br) ? int64_t(rh) * (rh + 1) / 2 : int64_t(rh) * cw;
      if (t >= size) {
        t -= size;
        continue;
      }
      if (bc == br) {
        int i = 0;
        while (t >= rh - i) {
          t -= rh - i;
          ++i;
        }
        ti = r0 + i;
        tj = r0 + i + static_cast<int>(t);
      } else {
        ti = r0 + static_cast<int>(t / cw);
        tj = c0 + static_cast<int>(t % cw);
      }
      return;
    }
  }
  ti = tj = 0;
}

// Row-major index of upper tile (ti, tj) (the partial-sum layout).
__device__ inline int64_t upper_index(int ti, int tj, int nt) {
  return int64_t(ti) * nt - int64_t(ti) * (ti - 1) / 2 + (tj - ti);
}

// Lane (g = lane/16, fi = lane%16) covers tokens t0+8g .. t0+8g+7 and
// features f .. f+7 of a panel (f = F0 + 8*fi); raw[q] holds token t0+8g+q.
//
// Full steps: `base` = X + t0*ldx is wave-uniform and off[q] is the lane's
// 32-bit element offset, so the loads take the scalar-base form and a step
// only advances the base.
__device__ inline void load_full(const uint16_t* __restrict__ base,
                                 const uint32_t off[8], u32x4 raw[8]) {
#pragma unroll
  for (int q = 0; q < 8; ++q)
    raw[q] = *reinterpret_cast<const u32x4*>(base + off[q]);
}

// Ragged steps (token tail, or a panel crossing d; needs d % 8 == 0 so a
// lane's 8 features are all in range or all out): out-of-range rows and
// features read a clamped in-range address and are zeroed.
__device__ inline void load_masked(const uint16_t* __restrict__ X, int64_t ldx,
                                   int64_t t0, int64_t tlim, int64_t F0,
                                   int64_t d, u32x4 raw[8]) {
  const int lane = threadIdx.x;
  const int64_t tb = t0 + 8 * (lane >> 4);
  const int64_t f = F0 + 8 * (lane & 15);
  const bool fv = f < d;
  const int64_t fc = fv ? f : 0;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const bool tv = tb + q < tlim;
    const u32x4 v = *reinterpret_cast<const u32x4*>(X + (tv ? tb + q : t0) * ldx + fc);
    raw[q] = (fv && tv) ? v : u32x4{0u, 0u, 0u, 0u};
  }
}

// raw[q].dword[p] = features (2p, 2p+1) of token q  ->
// frag[f].dword[t] = tokens (2t, 2t+1) of feature f.  One v_perm_b32 per
// output dword: bytes 0-3 of the selector index the second operand (token
// 2t), bytes 4-7 the first (token 2t+1).
__device__ inline void transpose8x8(const u32x4 raw[8], u32x4 frag[8]) {
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const uint32_t sel = (f & 1) ? 0x07060302u : 0x05040100u;
    uint32_t o[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      o[t] = __builtin_amdgcn_perm(raw[2 * t + 1][f >> 1], raw[2 * t][f >> 1], sel);
    frag[f] = u32x4{o[0], o[1], o[2], o[3]};
  }
}

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 8 x 8 MFMAs: acc[a][b] += (features F0+8i+a) x (features G0+8j+b) over
// the 32 tokens held in the fragments.
__device__ inline void mfma_tile(const u32x4 fa[8], const u32x4 fb[8],
                                 f32x4 acc[8][8]) {
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b)
      acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          as_bf16x8(fa[a]), as_bf16x8(fb[b]), acc[a][b], 0, 0, 0);
}

__global__ __launch_bounds__(64) void hessian_bf16_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, int64_t n_tok, int64_t d,
    int nt, int64_t ks, int nsplit, float* __restrict__ S,
    float* __restrict__ part) {
  // work item of this workgroup (see blocked_tile)
  const int64_t ntiles = upper_tiles(nt);
  const int64_t per_xcd = (ntiles + kXcd - 1) / kXcd;
  const int64_t w = blockIdx.x;
  const int64_t pos = w / kXcd;
  const int split = static_cast<int>(pos / per_xcd);
  const int64_t t = (w % kXcd) * per_xcd + pos % per_xcd;
  if (t >= ntiles || split >= nsplit) return;
  const int lane = threadIdx.x;
  int ti, tj;
  blocked_tile(t, nt, ti, tj);
  const int64_t L = upper_index(ti, tj, nt);
  const int64_t F0 = int64_t(ti) * kTile, G0 = int64_t(tj) * kTile;
  const bool diag = ti == tj;
  const int64_t tbeg = int64_t(split) * ks;
  const int64_t tend = min(tbeg + ks, n_tok);
  const bool panels_full = (F0 + kTile <= d) && (G0 + kTile <= d);

  f32x4 acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[8], rb[8], fa[8], fb[8];
  // full 32-token steps with both panels inside [0, d)
  const int64_t nfull = panels_full ? (tend - tbeg) / kStep : 0;
  if (nfull > 0) {
    uint32_t offa[8], offb[8];
    const int g8 = 8 * (lane >> 4), f8 = 8 * (lane & 15);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      offa[q] = static_cast<uint32_t>((g8 + q) * ldx + F0 + f8);
      offb[q] = static_cast<uint32_t>((g8 + q) * ldx + G0 + f8);
    }
    const uint16_t* base = X + tbeg * ldx;
    const int64_t step = kStep * ldx;
    // The fragments are loop-carried; the raw loads of step s+1 are issued
    // before the MFMAs of step s and transposed after them.
    load_full(base, offa, ra);
    load_full(base, offb, rb);
    transpose8x8(ra, fa);
    transpose8x8(rb, fb);
    for (int64_t s = 0; s < nfull; ++s) {
      const bool more = s + 1 < nfull;
      if (more) {
        base += step;
        load_full(base, offa, ra);
        load_full(base, offb, rb);
      }
      mfma_tile(fa, fb, acc);
      if (more) {
        transpose8x8(ra, fa);
        transpose8x8(rb, fb);
      }
    }
  }
  // ragged remainder (token tail of the split, or panels crossing d)
  for (int64_t t0 = tbeg + nfull * kStep; t0 < tend; t0 += kStep) {
    load_masked(X, ldx, t0, tend, F0, d, ra);
    load_masked(X, ldx, t0, tend, G0, d, rb);
    transpose8x8(ra, fa);
    transpose8x8(rb, fb);
    mfma_tile(fa, fb, acc);
  }

  // acc[f][f'][v] = S(F0 + 8*(4g+v) + f, G0 + 8*fi + f')
  const int g = lane >> 4, fi = lane & 15;
  if (nsplit == 1) {
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const int a = 8 * (4 * g + v) + f;
        const int64_t i = F0 + a;
#pragma unroll
        for (int f2 = 0; f2 < 8; ++f2) {
          const int b = 8 * fi + f2;
          const int64_t j = G0 + b;
          if (i < d && j < d && (!diag || a <= b)) {
            const float nv = S[i * d + j] + acc[f][f2][v];
            S[i * d + j] = nv;
            if (i != j) S[j * d + i] = nv;
          }
        }
      }
  } else {
    float* tile = part + ((int64_t(split) * upper_tiles(nt) + L) * kTile) * kTile;
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const int a = 8 * (4 * g + v) + f;
        f32x4 lo{acc[f][0][v], acc[f][1][v], acc[f][2][v], acc[f][3][v]};
        f32x4 hi{acc[f][4][v], acc[f][5][v], acc[f][6][v], acc[f][7][v]};
        *reinterpret_cast<f32x4*>(tile + a * kTile + 8 * fi) = lo;
        *reinterpret_cast<f32x4*>(tile + a * kTile + 8 * fi + 4) = hi;
      }
  }
}

// Adds the split partials of every upper tile to S in split order (fp64
// running sum) and mirrors the result into the lower triangle.
__global__ __launch_bounds__(256) void hessian_reduce_kernel(
    const float* __restrict__ part, int64_t d, int nt, int nsplit,
    float* __restrict__ S) {
  const int64_t L = blockIdx.x;
  int ti, tj;
  tile_of(L, nt, ti, tj);
  const int a = blockIdx.y * 2 + (threadIdx.x >> 7);
  const int b = threadIdx.x & 127;
  const int64_t i = int64_t(ti) * kTile + a, j = int64_t(tj) * kTile + b;
  if (i >= d || j >= d || (ti == tj && a > b)) return;
  const int64_t ntiles = upper_tiles(nt);
  double sum = 0.0;
  for (int s = 0; s < nsplit; ++s)
    sum += part[((int64_t(s) * ntiles + L) * kTile + a) * kTile + b];
  const float nv = static_cast<float>(static_cast<double>(S[i * d + j]) + sum);
  S[i * d + j] = nv;
  if (i != j) S[j * d + i] = nv;
}

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }

// Generic path (fp32 activations, or bf16 rows that are not 16-byte
// aligned): 64x64 upper tiles, 4x4 outputs per thread, fp64 sums.
template <class T>
__global__ __launch_bounds__(256) void hessian_generic_kernel(
    const T* __restrict__ X, int64_t ldx, int64_t n_tok, int64_t d,
    int nt64, float* __restrict__ S) {
  __shared__ float As[16][65];
  __shared__ float Bs[16][65];
  int ti, tj;
  tile_of(blockIdx.x, nt64, ti, tj);
  const int64_t F0 = int64_t(ti) * 64, G0 = int64_t(tj) * 64;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  double acc[4][4] = {};
  for (int64_t t0 = 0; t0 < n_tok; t0 += 16) {
    for (int e = threadIdx.x; e < 16 * 64; e += 256) {
      const int tt = e >> 6, ff = e & 63;
      const int64_t t = t0 + tt;
      As[tt][ff] = (t < n_tok && F0 + ff < d) ? to_f32(X[t * ldx + F0 + ff]) : 0.f;
      Bs[tt][ff] = (t < n_tok && G0 + ff < d) ? to_f32(X[t * ldx + G0 + ff]) : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int k = 0; k < 16; ++k) {
      double av[4], bv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        av[u] = As[k][ty * 4 + u];
        bv[u] = Bs[k][tx * 4 + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[u][w] = fma(av[u], bv[w], acc[u][w]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int a = ty * 4 + u, b = tx * 4 + w;
      const int64_t i = F0 + a, j = G0 + b;
      if (i < d && j < d && (ti != tj || a <= b)) {
        const float nv = static_cast<float>(static_cast<double>(S[i * d + j]) + acc[u][w]);
        S[i * d + j] = nv;
        if (i != j) S[j * d + i] = nv;
      }
    }
}

struct SplitPlan {
  int nsplit;
  int64_t ks;
};

// Chooses the token split so the (tile x split) work items fill whole rounds
// of one wave per SIMD, trading the tail-round loss against the partial-tile
// traffic (written and read once, 64 KiB per tile and split).
SplitPlan plan_splits(int64_t d, int64_t n_tok) {
  const int64_t nt = (d + kTile - 1) / kTile;
  const int64_t ntiles = upper_tiles(nt);
  const double mfma_s = 2.0 * double(n_tok) * double(d) * double(d) / 1.25e15;
  const int max_split = static_cast<int>(std::max<int64_t>(1, (n_tok + 4095) / 4096));
  SplitPlan best{1, n_tok};
  double best_t = 1e30;
  for (int ns = 1; ns <= std::min(max_split, 64); ++ns) {
    const int64_t ks = ((n_tok + ns - 1) / ns + kStep - 1) / kStep * kStep;
    const int nsr = static_cast<int>((n_tok + ks - 1) / ks);
    const int64_t items = ntiles * nsr;
    const double rounds = double((items + kTargetWaves - 1) / kTargetWaves);
    const double eff = double(items) / (rounds * kTargetWaves);
    const double t = mfma_s / eff +
                     (nsr > 1 ? 2.0 * nsr * ntiles * 65536.0 / 4.0e12 : 0.0);
    if (t < best_t * 0.999) {
      best_t = t;
      best = SplitPlan{nsr, ks};
    }
  }
  return best;
}

}  // namespace

size_t hessian_ws_bytes(int64_t d, int64_t n_tok) {
  if (d <= 0 || n_tok <= 0) return 0;
  const SplitPlan p = plan_splits(d, n_tok);
  if (p.nsplit <= 1) return 0;
  const int64_t nt = (d + kTile - 1) / kTile;
  return align_up(size_t(p.nsplit) * size_t(upper_tiles(nt)) * kTile * kTile * sizeof(float));
}

namespace {
bool mfma_path_ok(int64_t d, const void* X, gptq_dtype dt, int64_t ldx) {
  // per-lane element offsets of a 32-token step are kept in 32 bits
  return dt == GPTQ_BF16 && d % 8 == 0 && ldx % 8 == 0 &&
         reinterpret_cast<uintptr_t>(X) % 16 == 0 &&
         int64_t(kStep) * ldx + d < (int64_t(1) << 32);
}
}  // namespace

gptq_status launch_hessian(float* S, int64_t d, const void* X, gptq_dtype dt,
                           int64_t n_tok, int64_t ldx, void* ws,
                           hipStream_t st) {
  if (n_tok == 0) return GPTQ_OK;
  if (!mfma_path_ok(d, X, dt, ldx)) {
    const int nt64 = static_cast<int>((d + 63) / 64);
    const dim3 grid(static_cast<unsigned>(upper_tiles(nt64)));
    if (dt == GPTQ_F32)
      hessian_generic_kernel<float><<<grid, 256, 0, st>>>(
          static_cast<const float*>(X), ldx, n_tok, d, nt64, S);
    else
      hessian_generic_kernel<uint16_t><<<grid, 256, 0, st>>>(
          static_cast<const uint16_t*>(X), ldx, n_tok, d, nt64, S);
    GPTQ_CHECK_LAUNCH();
    return GPTQ_OK;
  }
  const int nt = static_cast<int>((d + kTile - 1) / kTile);
  const SplitPlan p = plan_splits(d, n_tok);
  const int64_t per_xcd = (upper_tiles(nt) + kXcd - 1) / kXcd;
  hessian_bf16_kernel<<<dim3(static_cast<unsigned>(kXcd * per_xcd * p.nsplit)), 64, 0, st>>>(
      static_cast<const uint16_t*>(X), ldx, n_tok, d, nt, p.ks, p.nsplit, S,
      static_cast<float*>(ws));
  GPTQ_CHECK_LAUNCH();
  if (p.nsplit > 1) {
    hessian_reduce_kernel<<<dim3(static_cast<unsigned>(upper_tiles(nt)), kTile / 2), 256, 0, st>>>(
        static_cast<const float*>(ws), d, nt, p.nsplit, S);
    GPTQ_CHECK_LAUNCH();
  }
  return GPTQ_OK;
}

}  // namespace gptq
