// Inference on the stored GPTQ format: Y = X W_hat^T with the packed low-bit
// weights dequantized inside the product ([wiki] "inference": W4A16, the
// int4 -> 16-bit expansion happens inside a fused matmul kernel; the stored
// format is that of [derivation] 3.1 / 8.3: b-bit codes per (row, column),
// a scale and zero per (row, group), a group id per column).
//
//   W_hat[r][c] = Delta[r][g(c)] * (code[r][c] - z[r][g(c)]),  g(c) = g_idx[c]
//   (signed codes of the symmetric grid: sign-extended, z = 0).
//
// The weight stream is the HBM cost (b/8 bytes per weight); activations are
// bf16 token rows (the "A16" of W4A16), products and sums fp32.
//
// Layout of the work: a workgroup owns 32 output rows (eight per wave) for
// one activation row, or 16 rows (four per wave) for a tile of 4 or 8
// activation rows; it walks the input dimension in chunks of 2048 columns.
// Per chunk the activations and the group ids are staged in LDS with
// 16-byte loads (each 8-column sub-block also gets its group id when its 8
// columns share one group -- always, for contiguous groups of a multiple of
// 8 -- else -1), and lane l of every wave takes the 32-column segment l of
// the chunk: the segment's codes are bits words of every row (column c of a
// row starts at bit c * bits, so a 32-column segment is exactly `bits` whole
// words), one wide load per row, coalesced across the wave.  A sub-block
// with one group factors the group's grid out: sum_i x_i Delta (c_i - z) =
// Delta (sum_i x_i c_i - z sum_i x_i), the grid loaded once per run of
// sub-blocks in that group; a mixed sub-block (act-order with dynamic
// groups) dequantizes column by column.  The wave's 64 partial sums per
// (row, token) are reduced with lane shuffles at the end.
#include "common.h"

namespace gptq {
namespace {

constexpr int kChunk = 2048;           // columns per LDS chunk
constexpr int kSub = kChunk / 8;       // 8-column sub-blocks per chunk

// Rows per wave: eight for one activation row (the chunk's staging is then
// shared by 32 rows per workgroup), four for the tiles of 4 or 8.
constexpr int rows_per_wave(int nx) { return nx == 1 ? 8 : 4; }

// 16-byte (or 8-byte) accesses allowed: bit 0 activations (ldx % 8 == 0,
// 16-byte aligned), bit 1 group ids (16-byte aligned), bit 2 code words
// (row stride and base aligned to the segment's load size).
constexpr int kVecX = 1, kVecG = 2, kVecW = 4;

__device__ inline float bf16_to_f32(uint32_t u) { return __uint_as_float(u << 16); }

// Code i (0..7) of sub-block sb (0..3) of a segment held in w[0..BITS).
template <int BITS>
__device__ inline uint32_t code_at(const uint32_t* w, int sb, int i) {
  const int p = (8 * sb + i) * BITS;
  const int wi = p >> 5, off = p & 31;
  uint32_t v = w[wi] >> off;
  if (off + BITS > 32) v |= w[wi + 1] << (32 - off);
  return v & ((1u << BITS) - 1u);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// sum a.lo b.lo + a.hi b.hi + c of two bf16 pairs, accumulated in fp32
// (the bf16 products are exact in fp32)
__device__ inline float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// bf16 round to nearest even (NaN stays a quiet NaN).
__device__ inline uint16_t f32_to_bf16(float v) {
  const uint32_t u = __float_as_uint(v);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
    return static_cast<uint16_t>((u >> 16) | 0x40u);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// The elementwise activation applied to a layer's output before it feeds
// the next layer (0 none, 1 ReLU, 2 SiLU).
__device__ inline float activate(float v, int act) {
  if (act == 1) return v > 0.0f ? v : 0.0f;
  if (act == 2) return v / (1.0f + expf(-v));
  return v;
}

// out_bf16 = 0: Y fp32; 1: Y bf16 after the activation `act`.
// Step Delta of (row, group) index i: fp32, or fp16 widened exactly.
template <bool SF16>
__device__ inline float load_scale(const void* __restrict__ p, int64_t i) {
  if (SF16) return static_cast<float>(static_cast<const _Float16*>(p)[i]);
  return static_cast<const float*>(p)[i];
}

template <int BITS, int NX, bool SF16>
__global__ __launch_bounds__(256) void dequant_matmul_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, int64_t n,
    const uint32_t* __restrict__ qw, int64_t words,
    const void* __restrict__ scales, const uint8_t* __restrict__ zeros,
    int64_t ng, const int32_t* __restrict__ g_idx, int64_t m, int64_t d,
    int sgn, void* __restrict__ Y, int64_t ldy, int out_bf16, int act, int vec) {
  constexpr int kRowsPerWave = rows_per_wave(NX);
  constexpr int kRowsPerWg = 4 * kRowsPerWave;
  __shared__ __attribute__((aligned(16))) uint16_t xs[NX][kChunk];
  __shared__ __attribute__((aligned(16))) int32_t gs[kChunk];
  __shared__ int32_t ug[kSub];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t r0 = int64_t(blockIdx.x) * kRowsPerWg + kRowsPerWave * wv;
  const int64_t k0 = int64_t(blockIdx.y) * NX;          // first activation row
  const int nk = static_cast<int>(min<int64_t>(NX, n - k0));
  // rows of this wave, clamped into range (their sums are not stored)
  int64_t rows[kRowsPerWave];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) rows[i] = min<int64_t>(r0 + i, m - 1);
  float acc[kRowsPerWave][NX];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i)
#pragma unroll
    for (int k = 0; k < NX; ++k) acc[i][k] = 0.0f;
  const uint32_t hb = 1u << (BITS - 1);

  for (int64_t c0 = 0; c0 < d; c0 += kChunk) {
    // ---- stage the chunk's activations and group ids (thread t: columns
    //      8t .. 8t + 7 of the chunk)
    {
      const int64_t cb = c0 + 8 * tid;
      const bool full = cb + 8 <= d;
#pragma unroll
      for (int k = 0; k < NX; ++k) {
        const bool krow = k < nk;
        const uint16_t* src = X + (k0 + (krow ? k : 0)) * ldx;
        if ((vec & kVecX) && full) {
          const uint4 v = *reinterpret_cast<const uint4*>(src + cb);
          *reinterpret_cast<uint4*>(&xs[k][8 * tid]) = krow ? v : uint4{0u, 0u, 0u, 0u};
        } else {
          uint16_t v[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = (krow && cb + i < d) ? src[cb + i] : uint16_t(0);
#pragma unroll
          for (int i = 0; i < 8; ++i) xs[k][8 * tid + i] = v[i];
        }
      }
      int32_t g[8];
      if ((vec & kVecG) && full) {
        const int4 a = *reinterpret_cast<const int4*>(g_idx + cb);
        const int4 b = *reinterpret_cast<const int4*>(g_idx + cb + 4);
        g[0] = a.x; g[1] = a.y; g[2] = a.z; g[3] = a.w;
        g[4] = b.x; g[5] = b.y; g[6] = b.z; g[7] = b.w;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) g[i] = g_idx[min<int64_t>(cb + i, d - 1)];
      }
      bool same = true;
#pragma unroll
      for (int i = 1; i < 8; ++i) same = same && (g[i] == g[0] || cb + i >= d);
#pragma unroll
      for (int i = 0; i < 8; ++i) gs[8 * tid + i] = g[i];
      ug[tid] = same ? g[0] : -1;
    }
    __syncthreads();
    // ---- this lane's 32-column segment of every row of the wave
    const int64_t seg = c0 / 32 + lane;
    if (seg * 32 < d) {
      uint32_t w[kRowsPerWave][BITS];
      if ((vec & kVecW) && BITS != 3 && (seg + 1) * BITS <= words) {
        // the segment's BITS words in one (two at 8 bits) wide load per row
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) {
          const uint32_t* p = qw + rows[i] * words + seg * BITS;
          if (BITS == 2) {
            const uint2 v = *reinterpret_cast<const uint2*>(p);
            w[i][0] = v.x; w[i][1 % BITS] = v.y;
          } else {
#pragma unroll
            for (int h = 0; h < BITS / 4; ++h) {
              const uint4 v = *reinterpret_cast<const uint4*>(p + 4 * h);
              w[i][(4 * h) % BITS] = v.x; w[i][(4 * h + 1) % BITS] = v.y;
              w[i][(4 * h + 2) % BITS] = v.z; w[i][(4 * h + 3) % BITS] = v.w;
            }
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i)
#pragma unroll
          for (int j = 0; j < BITS; ++j) {
            const int64_t wi = seg * BITS + j;
            w[i][j] = wi < words ? qw[rows[i] * words + wi] : 0u;
          }
      }
      // the grid of the previous uniform sub-block, reused while the group
      // stays the same (a 32-column segment usually lies in one group)
      int Gp = -1;
      float sc[kRowsPerWave], zc[kRowsPerWave];
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) {
        const int cl = 32 * lane + 8 * sb;          // column within the chunk
        if (c0 + cl >= d) break;
        float xv[NX][8];
        uint32_t xp[NX][4];     // bf16 pairs (x0, x2), (x4, x6), (x1, x3), (x5, x7)
#pragma unroll
        for (int k = 0; k < NX; ++k) {
          const uint4 raw = *reinterpret_cast<const uint4*>(&xs[k][cl]);
          const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
          if (BITS == 4) {
            xp[k][0] = __builtin_amdgcn_perm(raw.y, raw.x, 0x05040100u);
            xp[k][1] = __builtin_amdgcn_perm(raw.w, raw.z, 0x05040100u);
            xp[k][2] = __builtin_amdgcn_perm(raw.y, raw.x, 0x07060302u);
            xp[k][3] = __builtin_amdgcn_perm(raw.w, raw.z, 0x07060302u);
          } else if (BITS == 2) {   // (x0, x4), (x1, x5), (x2, x6), (x3, x7)
            xp[k][0] = __builtin_amdgcn_perm(raw.z, raw.x, 0x05040100u);
            xp[k][1] = __builtin_amdgcn_perm(raw.z, raw.x, 0x07060302u);
            xp[k][2] = __builtin_amdgcn_perm(raw.w, raw.y, 0x05040100u);
            xp[k][3] = __builtin_amdgcn_perm(raw.w, raw.y, 0x07060302u);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            xv[k][2 * i] = bf16_to_f32(u[i] & 0xFFFFu);
            xv[k][2 * i + 1] = bf16_to_f32(u[i] >> 16);
          }
        }
        const int G = ug[cl / 8];
        if (G >= 0) {
          float xsum[NX];
#pragma unroll
          for (int k = 0; k < NX; ++k) {
            float t = 0.0f;
            if (BITS == 4 || BITS == 2) {
              // the activation pairs against bf16 ones (0x3F80 = 1.0)
#pragma unroll
              for (int i = 0; i < 4; ++i) t = dot2_bf16(xp[k][i], 0x3F803F80u, t);
            } else {
#pragma unroll
              for (int i = 0; i < 8; ++i) t += xv[k][i];
            }
            xsum[k] = t;
          }
          if (G != Gp) {
#pragma unroll
            for (int r = 0; r < kRowsPerWave; ++r) {
              sc[r] = load_scale<SF16>(scales, rows[r] * ng + G);
              // 4- and 2-bit: the zero term 16 + z of the expansion below
              // (signed codes: z = 8 or 2); other widths: z itself
              const float z = static_cast<float>(zeros[rows[r] * ng + G]);
              zc[r] = BITS == 4 ? 16.0f + (sgn ? 8.0f : z)
                    : BITS == 2 ? 16.0f + (sgn ? 2.0f : z) : z;
            }
            Gp = G;
          }
          if (BITS == 4) {
            // the sub-block's 8 codes are word sb of the segment; each code
            // k becomes the bf16 value 16 + k (exponent of 16: 0x4180, k in
            // mantissa bits 3..6), two per register, and meets the matching
            // activation pair in one fp32-accumulating dot product:
            // t = sum x (16 + k), so sum x (k - z) = t - (16 + z) sum x.
            // Signed codes: k = c ^ 8 = c_s + 8, i.e. the same with z = 8.
#pragma unroll
            for (int r = 0; r < kRowsPerWave; ++r) {
              const uint32_t wr = w[r][sb % BITS] ^ (sgn ? 0x88888888u : 0u);
              const uint32_t lo = ((wr << 3) & 0x78787878u) | 0x80808080u;   // codes 0, 2, 4, 6
              const uint32_t hi = ((wr >> 1) & 0x78787878u) | 0x80808080u;   // codes 1, 3, 5, 7
              const uint32_t p02 = __builtin_amdgcn_perm(0x41414141u, lo, 0x04010400u);
              const uint32_t p46 = __builtin_amdgcn_perm(0x41414141u, lo, 0x04030402u);
              const uint32_t p13 = __builtin_amdgcn_perm(0x41414141u, hi, 0x04010400u);
              const uint32_t p57 = __builtin_amdgcn_perm(0x41414141u, hi, 0x04030402u);
#pragma unroll
              for (int k = 0; k < NX; ++k) {
                float t = dot2_bf16(p02, xp[k][0], 0.0f);
                t = dot2_bf16(p46, xp[k][1], t);
                t = dot2_bf16(p13, xp[k][2], t);
                t = dot2_bf16(p57, xp[k][3], t);
                acc[r][k] = fmaf(sc[r], fmaf(-zc[r], xsum[k], t), acc[r][k]);
              }
            }
          } else if (BITS == 2) {
            // the sub-block's 8 codes are half sb % 2 of word sb / 2; code j
            // (bits 2j) goes to mantissa bits 3..4 of a bf16 16 + k as
            // above, pairs (c0, c4), (c1, c5), (c2, c6), (c3, c7).  Signed
            // codes: k = c ^ 2 = c_s + 2.
#pragma unroll
            for (int r = 0; r < kRowsPerWave; ++r) {
              const uint32_t v = ((w[r][(sb / 2) % BITS] >> (16 * (sb % 2))) & 0xFFFFu) ^
                                 (sgn ? 0xAAAAu : 0u);
              const uint32_t t04 = ((v << 3) & 0x1818u) | 0x8080u;
              const uint32_t t15 = ((v << 1) & 0x1818u) | 0x8080u;
              const uint32_t t26 = ((v >> 1) & 0x1818u) | 0x8080u;
              const uint32_t t37 = ((v >> 3) & 0x1818u) | 0x8080u;
              const uint32_t p04 = __builtin_amdgcn_perm(0x41414141u, t04, 0x04010400u);
              const uint32_t p15 = __builtin_amdgcn_perm(0x41414141u, t15, 0x04010400u);
              const uint32_t p26 = __builtin_amdgcn_perm(0x41414141u, t26, 0x04010400u);
              const uint32_t p37 = __builtin_amdgcn_perm(0x41414141u, t37, 0x04010400u);
#pragma unroll
              for (int k = 0; k < NX; ++k) {
                float t = dot2_bf16(p04, xp[k][0], 0.0f);
                t = dot2_bf16(p15, xp[k][1], t);
                t = dot2_bf16(p26, xp[k][2], t);
                t = dot2_bf16(p37, xp[k][3], t);
                acc[r][k] = fmaf(sc[r], fmaf(-zc[r], xsum[k], t), acc[r][k]);
              }
            }
          } else {
#pragma unroll
          for (int r = 0; r < kRowsPerWave; ++r) {
            const float s = sc[r];
            const float z = zc[r];
            float cv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const uint32_t c = code_at<BITS>(w[r], sb, i);
              cv[i] = sgn ? static_cast<float>(static_cast<int>(c ^ hb) - static_cast<int>(hb))
                          : static_cast<float>(c);
            }
#pragma unroll
            for (int k = 0; k < NX; ++k) {
              float t = 0.0f;
#pragma unroll
              for (int i = 0; i < 8; ++i) t = fmaf(xv[k][i], cv[i], t);
              acc[r][k] = fmaf(s, fmaf(-z, xsum[k], t), acc[r][k]);
            }
          }
          }
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int Gi = gs[cl + i];
#pragma unroll
            for (int r = 0; r < kRowsPerWave; ++r) {
              const float s = load_scale<SF16>(scales, rows[r] * ng + Gi);
              const float z = static_cast<float>(zeros[rows[r] * ng + Gi]);
              const uint32_t c = code_at<BITS>(w[r], sb, i);
              const float cv = sgn ? static_cast<float>(static_cast<int>(c ^ hb) - static_cast<int>(hb))
                                   : static_cast<float>(c);
              const float wq = s * (cv - z);
#pragma unroll
              for (int k = 0; k < NX; ++k) acc[r][k] = fmaf(xv[k][i], wq, acc[r][k]);
            }
          }
        }
      }
    }
    __syncthreads();
  }
  // ---- reduce the 64 lanes' partial sums; lane 0 writes
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
    for (int k = 0; k < NX; ++k) {
      float v = acc[r][k];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
      acc[r][k] = v;
    }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
      for (int k = 0; k < NX; ++k)
        if (r0 + r < m && k < nk) {
          const int64_t e = (k0 + k) * ldy + r0 + r;
          if (out_bf16)
            static_cast<uint16_t*>(Y)[e] = f32_to_bf16(activate(acc[r][k], act));
          else
            static_cast<float*>(Y)[e] = acc[r][k];
        }
  }
}

// ---------------------------------------------------------------------------
// Many activation rows (n > 16; up to 16 the vector kernel's passes of 8 rows
// take less time than a mostly empty tile): the same product on the matrix
// cores.
//
// A workgroup of eight waves (two per SIMD, so that one wave's waits and
// VALU work overlap the other's MFMAs) owns a tile of 256 activation rows x
// 128 weight rows; wave w holds activation rows 64 (w % 4) .. + 63 and weight
// rows 64 (w / 4) .. + 63 as 4 x 4 fragments of v_mfma_f32_16x16x32_bf16.
// The input dimension goes by in blocks of 64 columns (two 32-column steps),
// double buffered in LDS with one barrier per block:
//  * activations: global_load_lds_dwordx4 straight into LDS (no registers),
//    a block ahead; blocks at the edges of the input (rows past n, columns
//    past d, unaligned rows) go through registers, zero-filled;
//  * codes: loaded into registers a block ahead, expanded by the whole
//    workgroup into bf16 B operands in LDS (each code once per workgroup).
// Both are stored as 16-byte units (8 columns) of a row, unit c of row r at
// c ^ ((r / 2) % 8): the MFMA fragment reads (16 consecutive rows, one unit
// each) then touch all 16 bank groups once, and each 8-row direct load
// still fills every row with its 8 units (128 contiguous bytes).
//
// Exactness: a weight is never rounded to bf16.  B holds an exact small
// number per code -- 16 + k for 2-, 3- and 4-bit codes (the code in mantissa
// bits 3..6 under the exponent of 16), k itself for 8-bit codes -- with k the
// unsigned code, or the signed code plus 2^(b-1).  Per group G the matrix
// cores form P = sum x B over the group's columns and (one more product with
// B = 1) Xs = sum x; the group is folded into the fp32 result when it ends:
//   sum x Delta (c - z) = Delta (P - (16 + z) Xs)    (2-, 3-, 4-bit)
//                       = Delta (P - z Xs)            (8-bit)
// with z = 2^(b-1) for signed codes.  A step whose 32 columns share one group
// (contiguous groups of a multiple of 32 columns, the whole-row grid) just
// accumulates; a step that mixes groups (act-order with dynamic groups,
// groups of 8) runs once per group present, its A operand masked to that
// group's columns, and folds each at once.
constexpr int kTm = 256;               // activation rows per workgroup
constexpr int kTn = 128;               // weight rows per workgroup
constexpr int kBk = 64;                // columns per LDS block
constexpr int kGemmThreads = 512;      // eight waves
constexpr int kUnitsA = kTm * kBk / 8; // 16-byte units of a block's activations
constexpr int kUnitsB = kTn * kBk / 8; // and of its expanded codes

// LDS byte offset of unit c (8 columns) of row r of a block.
__device__ inline uint32_t unit_off(int r, int c) {
  return static_cast<uint32_t>((r * (kBk / 8) + (c ^ ((r >> 1) & 7))) * 16);
}

// Eight codes in nibbles (code i at bits 4i) as four bf16 pairs 16 + k in
// natural order (codes 2p, 2p + 1 in pair p).
__device__ inline u32x4 expand_nibbles(uint32_t w) {
  const uint32_t lo = ((w << 3) & 0x78787878u) | 0x80808080u;   // codes 0, 2, 4, 6
  const uint32_t hi = ((w >> 1) & 0x78787878u) | 0x80808080u;   // codes 1, 3, 5, 7
  return u32x4{__builtin_amdgcn_perm(hi, lo, 0x0C040C00u) | 0x41004100u,
               __builtin_amdgcn_perm(hi, lo, 0x0C050C01u) | 0x41004100u,
               __builtin_amdgcn_perm(hi, lo, 0x0C060C02u) | 0x41004100u,
               __builtin_amdgcn_perm(hi, lo, 0x0C070C03u) | 0x41004100u};
}

// The B operand of one 8-column run: its codes (w0; w1 holds codes 4..7 of
// 8-bit codes) as exact bf16 numbers, natural order.
template <int BITS>
__device__ inline u32x4 expand_run(uint32_t w0, uint32_t w1, int sgn) {
  if (BITS == 4) return expand_nibbles(w0 ^ (sgn ? 0x88888888u : 0u));
  if (BITS == 3) {
    // spread the 3-bit fields to nibbles
    uint32_t u = (w0 & 0xFFFu) | ((w0 & 0xFFF000u) << 4);
    u = (u & 0x003F003Fu) | ((u & 0x0FC00FC0u) << 2);
    u = (u & 0x07070707u) | ((u & 0x38383838u) << 1);
    return expand_nibbles(u ^ (sgn ? 0x44444444u : 0u));
  }
  if (BITS == 2) {
    // spread the 2-bit fields to nibbles
    uint32_t u = (w0 & 0xFFu) | ((w0 & 0xFF00u) << 8);
    u = (u & 0x000F000Fu) | ((u & 0x00F000F0u) << 4);
    u = (u & 0x03030303u) | ((u & 0x0C0C0C0Cu) << 2);
    return expand_nibbles(u ^ (sgn ? 0x22222222u : 0u));
  }
  // 8-bit: each code converted exactly to fp32, its upper half is the bf16
  const uint32_t a = w0 ^ (sgn ? 0x80808080u : 0u), b = w1 ^ (sgn ? 0x80808080u : 0u);
  const float f[8] = {float(a & 0xFFu), float((a >> 8) & 0xFFu), float((a >> 16) & 0xFFu),
                      float(a >> 24), float(b & 0xFFu), float((b >> 8) & 0xFFu),
                      float((b >> 16) & 0xFFu), float(b >> 24)};
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = __builtin_amdgcn_perm(__float_as_uint(f[2 * i + 1]), __float_as_uint(f[2 * i]),
                                 0x07060302u);
  return r;
}

// The code bits of 8-column run `ch` of a weight row (row pointer p,
// `words` words), masked to the run: w0 (and w1 for 8-bit codes).  Runs past
// the end read the last word (their activations are zero).
template <int BITS>
__device__ inline void load_run(const uint32_t* __restrict__ p, int64_t words, int64_t ch,
                                uint32_t& w0, uint32_t& w1) {
  if (BITS == 4) {
    w0 = p[min<int64_t>(ch, words - 1)];
    w1 = 0u;
  } else if (BITS == 2) {
    w0 = (p[min<int64_t>(ch >> 1, words - 1)] >> (16 * (ch & 1))) & 0xFFFFu;
    w1 = 0u;
  } else if (BITS == 8) {
    w0 = p[min<int64_t>(2 * ch, words - 1)];
    w1 = p[min<int64_t>(2 * ch + 1, words - 1)];
  } else {
    const int64_t bit = 24 * ch;
    const int64_t i = min<int64_t>(bit >> 5, words - 1);
    const uint32_t lo = p[i], hi = p[min<int64_t>(i + 1, words - 1)];
    w0 = __builtin_amdgcn_alignbit(hi, lo, static_cast<uint32_t>(bit & 31)) & 0xFFFFFFu;
    w1 = 0u;
  }
}

// P += A B on v_mfma_f32_16x16x32_bf16 (the compiler's builtin, so that the
// wait states between an MFMA and the instructions reading its result are
// the compiler's to insert).
__device__ inline void mfma_acc(f32x4& P, const u32x4& a, const u32x4& b) {
  P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                              __builtin_bit_cast(bf16x8, b), P, 0, 0, 0);
}

typedef const void __attribute__((address_space(1)))* gvoid;
typedef void __attribute__((address_space(3)))* lvoid;

template <int BITS, bool SF16>
__global__ __launch_bounds__(kGemmThreads) void dequant_gemm_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, int64_t n,
    const uint32_t* __restrict__ qw, int64_t words,
    const void* __restrict__ scales, const uint8_t* __restrict__ zeros,
    int64_t ng, const int32_t* __restrict__ g_idx, int64_t m, int64_t d,
    int sgn, void* __restrict__ Y, int64_t ldy, int out_bf16, int act, int vec,
    unsigned tiles_m, unsigned tiles) {
  constexpr int kSteps = kBk / 32;
  __shared__ __attribute__((aligned(16))) char lA[2][kUnitsA * 16];
  __shared__ __attribute__((aligned(16))) char lB[2][kUnitsB * 16];
  __shared__ int32_t gsh[2][kBk];
  __shared__ int32_t desc[2][kSteps];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int q = lane >> 4, c16 = lane & 15;
  // consecutive tiles share activation rows; spread them so that each
  // XCD (blocks b, b + 8, ...) walks a contiguous range of tiles
  unsigned tile = blockIdx.x;
  const unsigned per = tiles / 8;
  if (tile < 8 * per) tile = (tile % 8) * per + tile / 8;
  const int64_t rb = int64_t(tile % tiles_m) * kTn;     // first weight row
  const int64_t tb = int64_t(tile / tiles_m) * kTm;     // first activation row
  const int wm = (wv & 3) * 64, wn = (wv >> 2) * 64;     // wave's offsets
  // blocks whose activation rows all exist and lie 16-byte aligned go
  // straight to LDS (the last, partial column block never does)
  const bool direct_rows = (vec & kVecX) && tb + kTm <= n;

  // weight rows of the lane's B fragments (clamped; not stored past m)
  int64_t rowj[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) rowj[j] = min<int64_t>(rb + wn + 16 * j + c16, m - 1);
  constexpr bool kMagic = BITS != 8;
  const float zsgn = static_cast<float>(1 << (BITS - 1));

  f32x4 acc[4][4], P[4][4], Xs[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    Xs[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = P[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // the grid of the open group: Delta and the zero term (16 + z, or z)
  float gs_s[4], gs_z[4];
  int cur = -1;        // open group (uniform over the workgroup), -1: none

  auto open_grid = [&](int G, float* s, float* z) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s[j] = load_scale<SF16>(scales, rowj[j] * ng + G);
      const float zz = sgn ? zsgn : static_cast<float>(zeros[rowj[j] * ng + G]);
      z[j] = kMagic ? 16.0f + zz : zz;
    }
  };
  // fold the group's products into the result, and clear them
  auto fold = [&](const float* s, const float* z) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          acc[i][j][v] = fmaf(s[j], fmaf(-z[j], Xs[i][v], P[i][j][v]), acc[i][j][v]);
        P[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      Xs[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };

  // ---- activations of a block.  Direct: wave w's instruction i fills the
  //      64 units of rows 8 (4 w + i) .. + 7, lane l writing slot l % 8 of
  //      row l / 8, i.e. reading that row's unit (l % 8) ^ ((row / 2) % 8).
  auto fetch_a_direct = [&](int64_t c0, int buf) {
#pragma unroll
    for (int i = 0; i < kUnitsA / 64 / 8; ++i) {
      const int r = 8 * (4 * wv + i) + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      const uint16_t* src = X + (tb + r) * ldx + c0 + 8 * c;
      __builtin_amdgcn_global_load_lds((gvoid)src,
                                       (lvoid)(lA[buf] + (8 * (4 * wv + i)) * (kBk / 8) * 16),
                                       16, 0, 0);
    }
  };
  // through registers: thread t stages units t + 512 h (row u / 8, unit u % 8)
  auto fetch_a_regs = [&](int64_t c0, int buf) {
#pragma unroll
    for (int h = 0; h < kUnitsA / kGemmThreads; ++h) {
      const int u = tid + kGemmThreads * h;
      const int r = u >> 3, c = u & 7;
      const int64_t tok = tb + r, cb = c0 + 8 * c;
      uint4 v = uint4{0u, 0u, 0u, 0u};
      if (tok < n) {
        const uint16_t* src = X + tok * ldx + cb;
        if ((vec & kVecX) && cb + 8 <= d) {
          v = *reinterpret_cast<const uint4*>(src);
        } else {
          uint32_t e[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) e[k] = cb + k < d ? src[k] : 0u;
          v = uint4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                    e[6] | (e[7] << 16)};
        }
      }
      *reinterpret_cast<uint4*>(lA[buf] + unit_off(r, c)) = v;
    }
  };
  // ---- codes and group ids of a block (registers): thread t takes runs
  //      2 (t % 4), + 1 of weight row t / 4
  const int brow = tid >> 2, bc = 2 * (tid & 3);
  const uint32_t* bsrc = qw + min<int64_t>(rb + brow, m - 1) * words;
  uint32_t cw[2][2];
  int32_t gx = 0;
  auto fetch_codes = [&](int64_t c0) {
#pragma unroll
    for (int e = 0; e < 2; ++e) load_run<BITS>(bsrc, words, c0 / 8 + bc + e, cw[e][0], cw[e][1]);
    if (tid < kBk) gx = g_idx[min<int64_t>(c0 + tid, d - 1)];
  };
  // expanded codes to LDS; the lanes holding group ids also write one
  // descriptor per 32-column step: its group when all its columns share
  // one, else -1
  auto store_codes = [&](int buf) {
#pragma unroll
    for (int e = 0; e < 2; ++e)
      *reinterpret_cast<u32x4*>(lB[buf] + unit_off(brow, bc + e)) =
          expand_run<BITS>(cw[e][0], cw[e][1], sgn);
    if (tid < kBk) {
      gsh[buf][tid] = gx;
      const int half = lane & 32;
      const int G0 = __shfl(gx, half);
      const uint64_t same = __ballot(gx == G0);
      if ((lane & 31) == 0)
        desc[buf][tid >> 5] = ((same >> half) & 0xFFFFFFFFull) == 0xFFFFFFFFull ? G0 : -1;
    }
  };
  auto fetch_a = [&](int64_t c0, int buf) {
    if (direct_rows && c0 + kBk <= d) fetch_a_direct(c0, buf);
    else fetch_a_regs(c0, buf);
  };

  const int64_t nblk = (d + kBk - 1) / kBk;
  fetch_a(0, 0);
  fetch_codes(0);
  store_codes(0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const u32x4 ones = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  for (int64_t blk = 0; blk < nblk; ++blk) {
    const int buf = static_cast<int>(blk & 1);
    const int64_t c0 = blk * kBk;
    const bool more = blk + 1 < nblk;
    if (more) {
      fetch_a(c0 + kBk, buf ^ 1);
      fetch_codes(c0 + kBk);
    }
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      if (c0 + 32 * s >= d) break;       // steps past the end of the input
      const int cs = 4 * s + q;          // the lane's unit within the block
      u32x4 A[4], B[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        A[i] = *reinterpret_cast<const u32x4*>(lA[buf] + unit_off(wm + 16 * i + c16, cs));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        B[j] = *reinterpret_cast<const u32x4*>(lB[buf] + unit_off(wn + 16 * j + c16, cs));
      // the groups present among the step's 32 columns, one pass each in
      // the order of their first column (one pass when the descriptor names
      // the step's single group); a pass masks the activations of the other
      // groups' columns (lane l of the group-id read: column l % 32)
      const int Gs = __builtin_amdgcn_readfirstlane(desc[buf][s]);
      int gl = Gs;
      if (Gs < 0) gl = gsh[buf][32 * s + (lane & 31)];
      uint64_t left = 0xFFFFFFFFull;
      do {
        const int G = Gs >= 0 ? Gs
                              : __builtin_amdgcn_readfirstlane(__shfl(gl, __builtin_ctzll(left)));
        const uint64_t in = Gs >= 0 ? 0xFFFFFFFFull : (__ballot(gl == G) & 0xFFFFFFFFull);
        left &= ~in;
        if (G != cur) {
          if (cur >= 0) fold(gs_s, gs_z);
          open_grid(G, gs_s, gs_z);
          cur = G;
        }
        uint32_t mk[4] = {~0u, ~0u, ~0u, ~0u};
        if (in != 0xFFFFFFFFull) {
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int e0 = 32 * s + 8 * q + 2 * p;
            mk[p] = (gsh[buf][e0] == G ? 0x0000FFFFu : 0u) |
                    (gsh[buf][e0 + 1] == G ? 0xFFFF0000u : 0u);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x4 Am = A[i];
#pragma unroll
          for (int p = 0; p < 4; ++p) Am[p] &= mk[p];
          mfma_acc(Xs[i], Am, ones);
#pragma unroll
          for (int j = 0; j < 4; ++j) mfma_acc(P[i][j], Am, B[j]);
        }
      } while (left);
    }
    if (more) store_codes(buf ^ 1);
    // the next block's direct loads have landed before anyone reads them
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (cur >= 0) fold(gs_s, gs_z);

  // ---- results: lane holds activation rows 4q + v of each 16-row fragment,
  //      weight row c16 of each 16-column fragment
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t tok = tb + wm + 16 * i + 4 * q + v;
      if (tok >= n) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t r = rb + wn + 16 * j + c16;
        if (r >= m) continue;
        const int64_t e = tok * ldy + r;
        if (out_bf16)
          static_cast<uint16_t*>(Y)[e] = f32_to_bf16(activate(acc[i][j][v], act));
        else
          static_cast<float*>(Y)[e] = acc[i][j][v];
      }
    }
}

unsigned cdiv(int64_t a, int64_t b) { return static_cast<unsigned>((a + b - 1) / b); }

template <int BITS, bool SF16>
gptq_status launch_bits(const uint16_t* X, int64_t ldx, int64_t n, const uint32_t* qw,
                        int64_t words, const void* scales, const uint8_t* zeros,
                        int64_t ng, const int32_t* g_idx, int64_t m, int64_t d,
                        int sgn, void* Y, int64_t ldy, int out_bf16, int act,
                        hipStream_t st) {
  const int vecx = (ldx % 8 == 0 && reinterpret_cast<uintptr_t>(X) % 16 == 0) ? kVecX : 0;
  if (n > 16) {
    const unsigned tiles_m = cdiv(m, kTn);
    const unsigned tiles = tiles_m * cdiv(n, kTm);
    dequant_gemm_kernel<BITS, SF16><<<tiles, kGemmThreads, 0, st>>>(
        X, ldx, n, qw, words, scales, zeros, ng, g_idx, m, d, sgn, Y, ldy, out_bf16, act, vecx,
        tiles_m, tiles);
    GPTQ_CHECK_LAUNCH();
    return GPTQ_OK;
  }
  const int nx = n <= 1 ? 1 : n <= 4 ? 4 : 8;
  const int64_t rows_wg = 4 * rows_per_wave(nx);
  const dim3 grid(cdiv(m, rows_wg), cdiv(n, nx));
  const int wbytes = BITS == 2 ? 8 : 16;       // wide code load of one segment
  const int vec = vecx |
                  (reinterpret_cast<uintptr_t>(g_idx) % 16 == 0 ? kVecG : 0) |
                  ((words * 4 % wbytes == 0 && reinterpret_cast<uintptr_t>(qw) % wbytes == 0)
                       ? kVecW : 0);
#define GPTQ_DQ(NXV)                                                                 \
  dequant_matmul_kernel<BITS, NXV, SF16><<<grid, 256, 0, st>>>(X, ldx, n, qw, words, scales, \
                                                         zeros, ng, g_idx, m, d, sgn, Y, ldy, \
                                                         out_bf16, act, vec)
  if (nx == 1)
    GPTQ_DQ(1);
  else if (nx == 4)
    GPTQ_DQ(4);
  else
    GPTQ_DQ(8);
#undef GPTQ_DQ
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

}  // namespace

gptq_status launch_dequant_matmul(const uint16_t* X, int64_t ldx, int64_t n,
                                  const uint32_t* qweight, int64_t m, int64_t d,
                                  int bits, const void* scales, int scale_f16,
                                  const uint8_t* zeros, int64_t ng,
                                  const int32_t* g_idx, int sgn, void* Y,
                                  int64_t ldy, int out_bf16, int act,
                                  hipStream_t st) {
  if (n == 0) return GPTQ_OK;
  if (n > int64_t(65535) * 8) return GPTQ_ERR_INVALID_ARG;   // grid.y
  const int64_t words = (d * bits + 31) / 32;
#define GPTQ_DQB(B)                                                                       \
  (scale_f16 ? launch_bits<B, true>(X, ldx, n, qweight, words, scales, zeros, ng, g_idx, m, d, \
                                    sgn, Y, ldy, out_bf16, act, st)                           \
             : launch_bits<B, false>(X, ldx, n, qweight, words, scales, zeros, ng, g_idx, m, d, \
                                     sgn, Y, ldy, out_bf16, act, st))
  switch (bits) {
    case 2: return GPTQ_DQB(2);
    case 3: return GPTQ_DQB(3);
    case 4: return GPTQ_DQB(4);
    case 8: return GPTQ_DQB(8);
  }
#undef GPTQ_DQB
  return GPTQ_ERR_INVALID_ARG;
}

}  // namespace gptq
