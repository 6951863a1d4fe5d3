// Element-type conversion of strided [rows, cols] blocks (cols % 4 == 0, rows
// and blocks 4-element aligned): bf16 inputs and weights to the fp16
// activation type and fp32/fp16 results to the bf16 output; and the input
// conversion fused with the fp32 B/C columns of the shared projection.
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

// The input conversion of a bf16 layer fused with the B/C columns of the shared projection in
// fp32: x16 = fp16(x) and bc = x . W_bc^T with fp32 accumulation (v_mfma_f32_16x16x32_f16; bf16
// values convert to fp16 exactly, so the products are exact and only the fp32 sums round).  The B/C
// columns are shared by every channel of a token, and every channel's normalised SSM output
// depends on sum_n C[n] B[n]; a 16-bit copy of them would carry its rounding into every channel of
// the row.  One wave = RG groups of 16 rows; in each 32-column step a lane holds row l % 16 of
// every group and the 8 input columns [8 (l/16), +8) -- its fp16 A fragments, which it also
// stores to x16.  The weight rows W_bc (fp16, <= 32 x d, L2-resident) are the B fragments, loaded
// once per step for the RG groups; the next step's loads are issued before this step's work.  The
// C fragment gives lane l column l % 16 of rows 4 (l/16) + 0..3.
template <int NCB, int RG>   // NCB: 16-column blocks of B/C (1: N = 8, 2: N = 16); RG: row groups
__global__ __launch_bounds__(256) void convert_bc_kernel(ConvBcArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t r0 = ((int64_t)blockIdx.x * 4 + wave) * (16 * RG);
  const int i = lane & 15, kq = lane >> 4;
  const bf16_t* xr[RG];
  half_t* xo[RG];
  bool row_ok[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    const int64_t row = r0 + 16 * g + i;
    row_ok[g] = row < a.rows;
    xr[g] = a.x + (row_ok[g] ? row : a.rows - 1) * a.ldx + 8 * kq;
    xo[g] = a.x16 + row * a.ldx16 + 8 * kq;
  }
  const half_t* wr[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) wr[cb] = a.wbc + (int64_t)(16 * cb + i) * a.ldw + 8 * kq;
  f32x4_t acc[RG][NCB];
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[g][cb] = f32x4_t{};
  // d % 8 == 0: a lane's 8 columns of a step are all in or all out
  auto load = [&](int k0, uint4 (&xv)[RG], uint4 (&wv)[NCB]) {
    const bool k_ok = k0 + 8 * kq < a.d;
#pragma unroll
    for (int g = 0; g < RG; ++g)
      xv[g] = k_ok ? *reinterpret_cast<const uint4*>(xr[g] + k0) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      wv[cb] = k_ok ? *reinterpret_cast<const uint4*>(wr[cb] + k0) : make_uint4(0u, 0u, 0u, 0u);
  };
  uint4 xv[RG], wv[NCB];
  load(0, xv, wv);
  for (int k0 = 0; k0 < a.d; k0 += 32) {
    uint4 xn[RG], wn[NCB];
    if (k0 + 32 < a.d) load(k0 + 32, xn, wn);
    const bool k_ok = k0 + 8 * kq < a.d;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      uint4 hv;
      hv.x = pack_f16x2(bf16lo(xv[g].x), bf16hi(xv[g].x));
      hv.y = pack_f16x2(bf16lo(xv[g].y), bf16hi(xv[g].y));
      hv.z = pack_f16x2(bf16lo(xv[g].z), bf16hi(xv[g].z));
      hv.w = pack_f16x2(bf16lo(xv[g].w), bf16hi(xv[g].w));
      if (k_ok && row_ok[g]) *reinterpret_cast<uint4*>(xo[g] + k0) = hv;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        acc[g][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, hv),
                                                            __builtin_bit_cast(f16x8_t, wv[cb]), acc[g][cb], 0, 0, 0);
    }
#pragma unroll
    for (int g = 0; g < RG; ++g) xv[g] = xn[g];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) wv[cb] = wn[cb];
  }
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t orow = r0 + 16 * g + 4 * kq + r;
        if (orow < a.rows) a.bc[orow * a.ldbc + 16 * cb + i] = acc[g][cb][r];
      }
}

constexpr int kConvRowGroups = 2;

}  // namespace

hipError_t launch_convert_bc(const ConvBcArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (a.d % 8 || (a.nbc != 16 && a.nbc != 32) || a.ldx % 8 || a.ldx16 % 8 || a.ldw % 8) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(ceil_div(a.rows, 4 * 16 * kConvRowGroups))), block(256);
  if (a.nbc == 32) hipLaunchKernelGGL((convert_bc_kernel<2, kConvRowGroups>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((convert_bc_kernel<1, kConvRowGroups>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_convert(const bf16_t* src, int64_t ld_src, half_t* dst, int64_t ld_dst, int64_t rows,
                          int64_t cols, hipStream_t s) { return conv(src, ld_src, dst, ld_dst, rows, cols, s); }
hipError_t launch_convert(const half_t* src, int64_t ld_src, float* dst, int64_t ld_dst, int64_t rows,
                          int64_t cols, hipStream_t s) { return conv(src, ld_src, dst, ld_dst, rows, cols, s); }
hipError_t launch_convert(const float* src, int64_t ld_src, bf16_t* dst, int64_t ld_dst, int64_t rows,
                          int64_t cols, hipStream_t s) { return conv(src, ld_src, dst, ld_dst, rows, cols, s); }
hipError_t launch_convert(const half_t* src, int64_t ld_src, bf16_t* dst, int64_t ld_dst, int64_t rows,
                          int64_t cols, hipStream_t s) { return conv(src, ld_src, dst, ld_dst, rows, cols, s); }

}  // namespace hymba
