// Element-type conversion of strided [rows, cols] blocks (cols % 4 == 0, rows
// and blocks 4-element aligned): bf16 inputs and weights to the fp16
// activation type, fp16 B/C columns to the fp32 side buffer the scan reads
// through the scalar unit, and fp32/fp16 results to the bf16 output.
#include "common.h"
#include "kernels.h"

namespace hymba {

namespace {

template <typename S> struct Quad;
template <> struct Quad<float> {
  __device__ static __forceinline__ void load(const float* p, float (&v)[4]) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  }
  __device__ static __forceinline__ void store(float* p, const float (&v)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <typename T> struct Quad16 {
  __device__ static __forceinline__ void load(const T* p, float (&v)[4]) {
    const uint2 x = *reinterpret_cast<const uint2*>(p);
    v[0] = Pair<T>::lo(x.x); v[1] = Pair<T>::hi(x.x); v[2] = Pair<T>::lo(x.y); v[3] = Pair<T>::hi(x.y);
  }
  __device__ static __forceinline__ void store(T* p, const float (&v)[4]) {
    uint2 x;
    x.x = Pair<T>::pack(v[0], v[1]);
    x.y = Pair<T>::pack(v[2], v[3]);
    *reinterpret_cast<uint2*>(p) = x;
  }
};
template <> struct Quad<bf16_t> : Quad16<bf16_t> {};
template <> struct Quad<half_t> : Quad16<half_t> {};

template <typename S, typename D>
__global__ __launch_bounds__(256) void convert_kernel(const S* __restrict__ src, int64_t ld_src, D* __restrict__ dst,
                                                      int64_t ld_dst, int64_t rows, int64_t quads_per_row) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * quads_per_row) return;
  const int64_t r = i / quads_per_row, c = (i % quads_per_row) * 4;
  float v[4];
  Quad<S>::load(src + r * ld_src + c, v);
  Quad<D>::store(dst + r * ld_dst + c, v);
}

template <typename S, typename D>
hipError_t conv(const S* src, int64_t ld_src, D* dst, int64_t ld_dst, int64_t rows, int64_t cols, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  if (cols % 4) return hipErrorInvalidValue;
  const int64_t n = rows * (cols / 4);
  hipLaunchKernelGGL((convert_kernel<S, D>), dim3(static_cast<unsigned>(ceil_div(n, 256))), dim3(256), 0, s, src,
                     ld_src, dst, ld_dst, rows, cols / 4);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_convert(const bf16_t* src, int64_t ld_src, half_t* dst, int64_t ld_dst, int64_t rows,
                          int64_t cols, hipStream_t s) { return conv(src, ld_src, dst, ld_dst, rows, cols, s); }
hipError_t launch_convert(const half_t* src, int64_t ld_src, float* dst, int64_t ld_dst, int64_t rows,
                          int64_t cols, hipStream_t s) { return conv(src, ld_src, dst, ld_dst, rows, cols, s); }
hipError_t launch_convert(const float* src, int64_t ld_src, bf16_t* dst, int64_t ld_dst, int64_t rows,
                          int64_t cols, hipStream_t s) { return conv(src, ld_src, dst, ld_dst, rows, cols, s); }
hipError_t launch_convert(const half_t* src, int64_t ld_src, bf16_t* dst, int64_t ld_dst, int64_t rows,
                          int64_t cols, hipStream_t s) { return conv(src, ld_src, dst, ld_dst, rows, cols, s); }

}  // namespace hymba
