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
// Layout of the work: a workgroup owns 16 output rows (four per wave) and
// one tile of up to NX activation rows; it walks the input dimension in
// chunks of 2048 columns.  Per chunk the activations and the group ids are
// staged in LDS (each 8-column sub-block also gets its group id when its 8
// columns share one group -- always, for contiguous groups of a multiple of
// 8 -- else -1), and lane l of every wave takes the 32-column segment l of
// the chunk: the segment's codes are bits words of every row (column c of a
// row starts at bit c * bits, so a 32-column segment is exactly `bits` whole
// words), read coalesced across the wave.  A sub-block with one group
// factors the group's grid out: sum_i x_i Delta (c_i - z) = Delta (sum_i x_i
// c_i - z sum_i x_i); a mixed sub-block (act-order with dynamic groups)
// dequantizes column by column.  The wave's 64 partial sums per (row,
// token) are reduced with lane shuffles at the end.
#include "common.h"

namespace gptq {
namespace {

constexpr int kChunk = 2048;           // columns per LDS chunk
constexpr int kSub = kChunk / 8;       // 8-column sub-blocks per chunk
constexpr int kRowsPerWave = 4;
constexpr int kRowsPerWg = 4 * kRowsPerWave;

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
    int sgn, void* __restrict__ Y, int64_t ldy, int out_bf16, int act) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[NX][kChunk];
  __shared__ int32_t gs[kChunk];
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
#pragma unroll
      for (int k = 0; k < NX; ++k) {
        uint16_t v[8];
        const bool krow = k < nk;
        const uint16_t* src = X + (k0 + (krow ? k : 0)) * ldx;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (krow && cb + i < d) ? src[cb + i] : uint16_t(0);
#pragma unroll
        for (int i = 0; i < 8; ++i) xs[k][8 * tid + i] = v[i];
      }
      int32_t g[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) g[i] = g_idx[min<int64_t>(cb + i, d - 1)];
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
#pragma unroll
      for (int i = 0; i < kRowsPerWave; ++i)
#pragma unroll
        for (int j = 0; j < BITS; ++j) {
          const int64_t wi = seg * BITS + j;
          w[i][j] = wi < words ? qw[rows[i] * words + wi] : 0u;
        }
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) {
        const int cl = 32 * lane + 8 * sb;          // column within the chunk
        if (c0 + cl >= d) break;
        float xv[NX][8];
#pragma unroll
        for (int k = 0; k < NX; ++k) {
          const uint4 raw = *reinterpret_cast<const uint4*>(&xs[k][cl]);
          const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
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
#pragma unroll
            for (int i = 0; i < 8; ++i) t += xv[k][i];
            xsum[k] = t;
          }
#pragma unroll
          for (int r = 0; r < kRowsPerWave; ++r) {
            const float s = load_scale<SF16>(scales, rows[r] * ng + G);
            const float z = static_cast<float>(zeros[rows[r] * ng + G]);
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

unsigned cdiv(int64_t a, int64_t b) { return static_cast<unsigned>((a + b - 1) / b); }

template <int BITS, bool SF16>
gptq_status launch_bits(const uint16_t* X, int64_t ldx, int64_t n, const uint32_t* qw,
                        int64_t words, const void* scales, const uint8_t* zeros,
                        int64_t ng, const int32_t* g_idx, int64_t m, int64_t d,
                        int sgn, void* Y, int64_t ldy, int out_bf16, int act,
                        hipStream_t st) {
  const int nx = n <= 1 ? 1 : n <= 4 ? 4 : 8;
  const dim3 grid(cdiv(m, kRowsPerWg), cdiv(n, nx));
#define GPTQ_DQ(NXV)                                                                 \
  dequant_matmul_kernel<BITS, NXV, SF16><<<grid, 256, 0, st>>>(X, ldx, n, qw, words, scales, \
                                                         zeros, ng, g_idx, m, d, sgn, Y, ldy, \
                                                         out_bf16, act)
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
