// Kernels of the layer-by-layer driver ([derivation] 3.2 steps 1-2 and 10:
// capture each layer's inputs, quantize it, verify its reconstruction error,
// then go on to the next layer).
//
// Layer error ([derivation] eq. (6)):
//   (1/N) ||(W - W_hat) X||_F^2 = (1/N) sum_r dw_r^T S dw_r,   S = X X^T,
// computed from S instead of the N-token outputs: T = dW S is a d x d
// contraction per row block (64 rows x 64 columns of T per workgroup, fp32
// products and sums, 4 x 4 per thread through LDS tiles of 16 k), and each
// workgroup's sum_j T[r][j] dW[r][j] goes out in fp64; a second kernel adds
// the partials in a fixed order.
#include "common.h"

namespace gptq {
namespace {

constexpr int kT = 64;      // output tile edge
constexpr int kK = 16;      // k per LDS stage

__device__ inline float load_w(const void* W, gptq_dtype dt, int64_t idx) {
  if (dt == GPTQ_F32) return static_cast<const float*>(W)[idx];
  return __uint_as_float(uint32_t(static_cast<const uint16_t*>(W)[idx]) << 16);
}

__global__ __launch_bounds__(256) void quadform_kernel(
    const void* __restrict__ W, gptq_dtype wdt, int64_t ldw,
    const float* __restrict__ W_hat, const float* __restrict__ S, int64_t m,
    int64_t d, double* __restrict__ part) {
  __shared__ float As[kK][kT + 1];   // dW[r0 + r][k0 + k] as As[k][r]
  __shared__ float Bs[kK][kT + 1];   // S[k0 + k][j0 + j]
  __shared__ double red[kT][17];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int64_t r0 = int64_t(blockIdx.x) * kT, j0 = int64_t(blockIdx.y) * kT;
  float acc[4][4] = {};
  for (int64_t k0 = 0; k0 < d; k0 += kK) {
    for (int e = tid; e < kK * kT; e += 256) {
      const int kk = e / kT, rr = e % kT;
      const int64_t r = r0 + rr, k = k0 + kk;
      float a = 0.0f, b = 0.0f;
      if (r < m && k < d) a = load_w(W, wdt, r * ldw + k) - W_hat[r * d + k];
      if (k < d && j0 + rr < d) b = S[k * d + j0 + rr];
      As[kk][rr] = a;
      Bs[kk][rr] = b;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = As[kk][4 * ty + u];
        b[u] = Bs[kk][4 * tx + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(a[u], b[v], acc[u][v]);
    }
    __syncthreads();
  }
  // sum_j T[r][j] dW[r][j] over this tile's columns
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t r = r0 + 4 * ty + u;
    double sr = 0.0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t j = j0 + 4 * tx + v;
      if (r < m && j < d)
        sr += double(acc[u][v]) * double(load_w(W, wdt, r * ldw + j) - W_hat[r * d + j]);
    }
    red[4 * ty + u][tx] = sr;
  }
  __syncthreads();
  if (tid < kT) {
    double t = 0.0;
    for (int x = 0; x < 16; ++x) t += red[tid][x];
    part[int64_t(blockIdx.y) * (int64_t(gridDim.x) * kT) + r0 + tid] = t;
  }
}

// out[0] = (sum of all partials, fixed order) / n
__global__ __launch_bounds__(256) void sum_parts_kernel(const double* __restrict__ part,
                                                        int64_t count, double inv_n,
                                                        double* __restrict__ out) {
  __shared__ double red[256];
  double t = 0.0;
  for (int64_t i = threadIdx.x; i < count; i += 256) t += part[i];
  red[threadIdx.x] = t;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = red[0] * inv_n;
}

__global__ void fill_f32_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

unsigned cdiv(int64_t a, int64_t b) { return static_cast<unsigned>((a + b - 1) / b); }

}  // namespace

size_t layer_error_part_count(int64_t m, int64_t d) {
  return size_t(cdiv(m, kT)) * kT * size_t(cdiv(d, kT));
}

gptq_status launch_layer_error(const void* W, gptq_dtype wdt, int64_t ldw,
                               const float* W_hat, const float* S, int64_t m,
                               int64_t d, int64_t n, double* part, double* out,
                               hipStream_t st) {
  const dim3 grid(cdiv(m, kT), cdiv(d, kT));
  quadform_kernel<<<grid, 256, 0, st>>>(W, wdt, ldw, W_hat, S, m, d, part);
  GPTQ_CHECK_LAUNCH();
  sum_parts_kernel<<<1, 256, 0, st>>>(part, int64_t(layer_error_part_count(m, d)),
                                      1.0 / double(n), out);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

gptq_status launch_zero_f32(float* p, int64_t n, hipStream_t st) {
  if (n <= 0) return GPTQ_OK;
  fill_f32_kernel<<<cdiv(n, 256), 256, 0, st>>>(p, n);
  GPTQ_CHECK_LAUNCH();
  return GPTQ_OK;
}

}  // namespace gptq
