// Final outputs in the original column order ([derivation] section 10: undo
// the column permutation; 3.1: codes are stored packed, scale/zero per row
// and group, group_id per column when dynamic groups meet act-order, 8.3).
//
// Packing layout (the pages leave it to the kernel): per row an LSB-first bit
// stream of b-bit codes in little-endian uint32 words; column c occupies
// stream bits [c*b, (c+1)*b), stream bit p is bit p%32 of word p/32, and a
// 3-bit code may straddle two words.
#include "common.h"

namespace gptq {
namespace {

// codesO[r][c] = codesP[pinv[c]][r] through 64x64 LDS tiles.
__global__ __launch_bounds__(256) void unpermute_codes_kernel(
    const uint8_t* __restrict__ codesP, int64_t m, int64_t d,
    const int32_t* __restrict__ pinv, uint8_t* __restrict__ codesO) {
  __shared__ uint8_t tile[64][65];
  const int64_t r0 = int64_t(blockIdx.x) * 64, c0 = int64_t(blockIdx.y) * 64;
  const int lx = threadIdx.x & 63, ly = threadIdx.x >> 6;
  for (int y = ly; y < 64; y += 4) {
    const int64_t c = c0 + y, r = r0 + lx;
    tile[y][lx] = (c < d && r < m) ? codesP[int64_t(pinv[c]) * m + r] : 0;
  }
  __syncthreads();
  for (int y = ly; y < 64; y += 4) {
    const int64_t r = r0 + y, c = c0 + lx;
    if (r < m && c < d) codesO[r * d + c] = tile[lx][y];
  }
}

__global__ __launch_bounds__(256) void pack_kernel(
    const uint8_t* __restrict__ codesO, int64_t m, int64_t d, int bits,
    int64_t words, uint32_t* __restrict__ qweight) {
  const int64_t w = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t r = blockIdx.y;
  if (w >= words) return;
  const int64_t bit0 = 32 * w;
  const int64_t cfirst = bit0 / bits;
  const int64_t clast = min((bit0 + 31) / bits, d - 1);
  const uint8_t* row = codesO + r * d;
  uint32_t word = 0;
  for (int64_t c = cfirst; c <= clast; ++c) {
    const int64_t sh = c * bits - bit0;
    const uint32_t code = row[c];
    word |= (sh >= 0) ? (code << sh) : (code >> (-sh));
  }
  qweight[r * words + w] = word;
}

// scales[r][g] = scalesP[g][r], zeros likewise.
__global__ __launch_bounds__(256) void meta_kernel(
    const float* __restrict__ scalesP, const uint8_t* __restrict__ zerosP,
    int64_t m, int64_t ng, float* __restrict__ scales,
    uint8_t* __restrict__ zeros) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e >= m * ng) return;
  const int64_t r = e / ng, g = e % ng;
  scales[e] = scalesP[g * m + r];
  zeros[e] = zerosP[g * m + r];
}

__global__ void gidx_kernel(const int32_t* __restrict__ pinv, int64_t d,
                            int64_t gsize, int32_t* __restrict__ g_idx) {
  const int64_t c = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (c < d) g_idx[c] = gsize > 0 ? static_cast<int32_t>(pinv[c] / gsize) : 0;
}

// w_hat[r][c] = Delta * (code - z) of the processing group holding column c.
__global__ __launch_bounds__(256) void w_hat_kernel(
    const uint8_t* __restrict__ codesO, const float* __restrict__ scales,
    const uint8_t* __restrict__ zeros, const int32_t* __restrict__ g_idx,
    int64_t m, int64_t d, int64_t ng, float* __restrict__ w_hat) {
  const int64_t c = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t r = blockIdx.y;
  if (c >= d) return;
  const int64_t g = g_idx[c];
  const float s = scales[r * ng + g];
  const float z = static_cast<float>(zeros[r * ng + g]);
  w_hat[r * d + c] = s * (static_cast<float>(codesO[r * d + c]) - z);
}

unsigned cdiv(int64_t a, int64_t b) { return static_cast<unsigned>((a + b - 1) / b); }

}  // namespace

gptq_status launch_outputs(int64_t m, int64_t d, int bits, int gsize,
                           const uint8_t* codesP, const float* scalesP,
                           const uint8_t* zerosP, const int32_t* pinv,
                           uint8_t* codesO, uint32_t* qweight, float* scales,
                           uint8_t* zeros, int32_t* g_idx, float* w_hat,
                           hipStream_t st) {
  const int64_t ng = gsize > 0 ? (d + gsize - 1) / gsize : 1;
  const int64_t words = (d * bits + 31) / 32;
  unpermute_codes_kernel<<<dim3(cdiv(m, 64), cdiv(d, 64)), 256, 0, st>>>(codesP, m, d, pinv, codesO);
  GPTQ_CHECK_LAUNCH();
  pack_kernel<<<dim3(cdiv(words, 256), static_cast<unsigned>(m)), 256, 0, st>>>(codesO, m, d, bits, words, qweight);
  GPTQ_CHECK_LAUNCH();
  meta_kernel<<<cdiv(m * ng, 256), 256, 0, st>>>(scalesP, zerosP, m, ng, scales, zeros);
  GPTQ_CHECK_LAUNCH();
  gidx_kernel<<<cdiv(d, 256), 256, 0, st>>>(pinv, d, gsize, g_idx);
  GPTQ_CHECK_LAUNCH();
  if (w_hat) {
    w_hat_kernel<<<dim3(cdiv(d, 256), static_cast<unsigned>(m)), 256, 0, st>>>(codesO, scales, zeros, g_idx, m, d, ng, w_hat);
    GPTQ_CHECK_LAUNCH();
  }
  return GPTQ_OK;
}

}  // namespace gptq
