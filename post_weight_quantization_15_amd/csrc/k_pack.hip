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

// One 64-row x 64-column tile of the outputs: the codes of original columns
// c0..c0+63 (processing positions pinv[c]) gathered through LDS, then
// packed: a row's 64 b-bit codes are exactly 2b words of its bit stream
// (the tile starts on bit 64 b c0 / 64, a word boundary).  codesO[r][c]
// (the unpacked codes in original order) is written as well when given.
// VEC: m % 4 == 0 and codesP 4-byte aligned, four rows per load.
template <bool VEC>
__global__ __launch_bounds__(256) void unpermute_pack_kernel(
    const uint8_t* __restrict__ codesP, int64_t m, int64_t d,
    const int32_t* __restrict__ pinv, int bits, int64_t words,
    uint32_t* __restrict__ qweight, uint8_t* __restrict__ codesO) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[64][68];   // [column][row]
  const int64_t r0 = int64_t(blockIdx.x) * 64, c0 = int64_t(blockIdx.y) * 64;
  const int t = threadIdx.x;
  if (VEC) {
    const int q = t & 15;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int y = (t >> 4) + 16 * k;
      const int64_t c = c0 + y, r = r0 + 4 * q;
      uint32_t v = 0;
      if (c < d && r < m) v = *reinterpret_cast<const uint32_t*>(codesP + int64_t(pinv[c]) * m + r);
      *reinterpret_cast<uint32_t*>(&tile[y][4 * q]) = v;
    }
  } else {
    const int lx = t & 63, ly = t >> 6;
    for (int y = ly; y < 64; y += 4) {
      const int64_t c = c0 + y, r = r0 + lx;
      tile[y][lx] = (c < d && r < m) ? codesP[int64_t(pinv[c]) * m + r] : 0;
    }
  }
  __syncthreads();
  // thread (row rr, word slot ws): words ws, ws + 4, ... of the row's 2b
  const int rr = t >> 2, ws = t & 3;
  const int64_t r = r0 + rr;
  if (r < m) {
    const int64_t w0 = c0 * bits / 32;
    for (int w = ws; w < 2 * bits; w += 4) {
      if (w0 + w >= words) break;
      const int bit0 = 32 * w;
      const int cfirst = bit0 / bits, clast = min((bit0 + 31) / bits, 63);
      uint32_t word = 0;
      for (int c = cfirst; c <= clast; ++c) {
        const int sh = c * bits - bit0;
        const uint32_t code = tile[c][rr];
        word |= (sh >= 0) ? (code << sh) : (code >> (-sh));
      }
      qweight[r * words + w0 + w] = word;
    }
  }
  if (codesO) {
    const int lx = t & 63, ly = t >> 6;
    for (int y = ly; y < 64; y += 4) {
      const int64_t rrow = r0 + y, c = c0 + lx;
      if (rrow < m && c < d) codesO[rrow * d + c] = tile[lx][y];
    }
  }
}

// scales[r][g] = scalesP[g][r], zeros likewise (0 for signed codes: their
// zero point is implicit).
__global__ __launch_bounds__(256) void meta_kernel(
    const float* __restrict__ scalesP, const uint8_t* __restrict__ zerosP,
    int64_t m, int64_t ng, int sgn, float* __restrict__ scales,
    uint8_t* __restrict__ zeros) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e >= m * ng) return;
  const int64_t r = e / ng, g = e % ng;
  scales[e] = scalesP[g * m + r];
  zeros[e] = sgn ? 0 : zerosP[g * m + r];
}

// Group of original column c: its processing group (dynamic groups,
// [derivation] 8.3 group_id[pi_j] = floor(j / g)), its own contiguous group
// (static groups, floor(c / g)), or 0 (whole-row grid).
__global__ void gidx_kernel(const int32_t* __restrict__ pinv, int64_t d,
                            int64_t gsize, int stat, int32_t* __restrict__ g_idx) {
  const int64_t c = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (c >= d) return;
  g_idx[c] = gsize <= 0 ? 0 : static_cast<int32_t>((stat ? c : int64_t(pinv[c])) / gsize);
}

// w_hat[r][c] = Delta * (code - z) of the group holding column c; signed
// codes (the low `bits` bits of c - z) are sign-extended, z = 0.
__global__ __launch_bounds__(256) void w_hat_kernel(
    const uint8_t* __restrict__ codesO, const float* __restrict__ scales,
    const uint8_t* __restrict__ zeros, const int32_t* __restrict__ g_idx,
    int64_t m, int64_t d, int64_t ng, int sgn, int bits,
    float* __restrict__ w_hat) {
  const int64_t c = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t r = blockIdx.y;
  if (c >= d) return;
  const int64_t g = g_idx[c];
  const float s = scales[r * ng + g];
  const int code = codesO[r * d + c];
  const float v = sgn ? static_cast<float>(code >= (1 << (bits - 1)) ? code - (1 << bits) : code)
                      : static_cast<float>(code) - static_cast<float>(zeros[r * ng + g]);
  w_hat[r * d + c] = s * v;
}

unsigned cdiv(int64_t a, int64_t b) { return static_cast<unsigned>((a + b - 1) / b); }

}  // namespace

gptq_status launch_outputs(int64_t m, int64_t d, int bits, int gsize, int sgn,
                           int stat, const uint8_t* codesP,
                           const float* scalesP, const uint8_t* zerosP,
                           const int32_t* pinv, uint8_t* codesO,
                           uint32_t* qweight, float* scales, uint8_t* zeros,
                           int32_t* g_idx, float* w_hat, hipStream_t st) {
  const int64_t ng = gsize > 0 ? (d + gsize - 1) / gsize : 1;
  const int64_t words = (d * bits + 31) / 32;
  // the unpacked codes in original order are kept only for w_hat
  uint8_t* co = w_hat ? codesO : nullptr;
  const dim3 grid(cdiv(m, 64), cdiv(d, 64));
  if (m % 4 == 0 && reinterpret_cast<uintptr_t>(codesP) % 4 == 0)
    unpermute_pack_kernel<true><<<grid, 256, 0, st>>>(codesP, m, d, pinv, bits, words, qweight, co);
  else
    unpermute_pack_kernel<false><<<grid, 256, 0, st>>>(codesP, m, d, pinv, bits, words, qweight, co);
  GPTQ_CHECK_LAUNCH();
  meta_kernel<<<cdiv(m * ng, 256), 256, 0, st>>>(scalesP, zerosP, m, ng, sgn, scales, zeros);
  GPTQ_CHECK_LAUNCH();
  gidx_kernel<<<cdiv(d, 256), 256, 0, st>>>(pinv, d, gsize, stat, g_idx);
  GPTQ_CHECK_LAUNCH();
  if (w_hat) {
    w_hat_kernel<<<dim3(cdiv(d, 256), static_cast<unsigned>(m)), 256, 0, st>>>(codesO, scales, zeros, g_idx, m, d, ng, sgn, bits, w_hat);
    GPTQ_CHECK_LAUNCH();
  }
  return GPTQ_OK;
}

}  // namespace gptq
