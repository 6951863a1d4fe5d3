// fp32 projection GEMM used by the fp32 workload: Y[rows, out] = X[rows, in] . W[out, in]^T.
// 64 x 64 output tile per 256-thread workgroup, 16-deep K slices staged in
// LDS, 4 x 4 outputs per thread, fp32 FMA accumulation in K order.
#include "common.h"
#include "kernels.h"

namespace hymba {

namespace {

__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ X, int64_t ldx,
                                                       const float* __restrict__ W, int64_t ldw,
                                                       float* __restrict__ Y, int64_t ldy, int64_t rows,
                                                       int out, int in) {
  __shared__ float xs[16][64 + 4];
  __shared__ float ws[16][64 + 4];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t r0 = (int64_t)blockIdx.y * 64;
  const int c0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < in; k0 += 16) {
    for (int i = threadIdx.x; i < 1024; i += 256) {
      const int r = i >> 4, k = i & 15;
      const bool kin = k0 + k < in;
      xs[k][r] = (kin && r0 + r < rows) ? X[(r0 + r) * ldx + k0 + k] : 0.f;
      ws[k][r] = (kin && c0 + r < out) ? W[(int64_t)(c0 + r) * ldw + k0 + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(xs[k][ty * 4 + i], ws[k][tx * 4 + j], acc[i][j]);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = r0 + ty * 4 + i;
    if (r >= rows) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = c0 + tx * 4 + j;
      if (c < out) Y[r * ldy + c] = acc[i][j];
    }
  }
}

}  // namespace

hipError_t launch_gemm_f32(const float* X, int64_t ldx, const float* W, int64_t ldw, float* Y,
                           int64_t ldy, int64_t rows, int out, int in, hipStream_t s) {
  if (rows <= 0 || out <= 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>(ceil_div(out, 64)), static_cast<unsigned>(ceil_div(rows, 64)));
  hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, s, X, ldx, W, ldw, Y, ldy, rows, out, in);
  return hipGetLastError();
}

}  // namespace hymba
