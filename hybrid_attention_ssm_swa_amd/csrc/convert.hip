// Element-type conversion of strided [rows, cols] blocks (cols % 4 == 0, rows
// and blocks 4-element aligned): bf16 inputs and weights to the fp16
// activation type and fp32/fp16 results to the bf16 output; and the input
// conversion fused with the fp32 B/C columns of the shared projection.
#include <algorithm>

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
// once per step for the RG groups.  Steps go in pairs (each row's whole 128-byte line), the next
// pair's loads issued before this pair's work.  The
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
  // a pair of 32-column steps: each row's whole 128-byte line.  d % 8 == 0: a lane's 8 columns of
  // a step are all in or all out.
  struct Pair2 { uint4 x[2][RG]; uint4 w[2][NCB]; };
  auto load = [&](int k0, Pair2& p) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = k0 + 32 * h;
      const bool k_ok = k + 8 * kq < a.d;
#pragma unroll
      for (int g = 0; g < RG; ++g)
        p.x[h][g] = k_ok ? *reinterpret_cast<const uint4*>(xr[g] + k) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        p.w[h][cb] = k_ok ? *reinterpret_cast<const uint4*>(wr[cb] + k) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  Pair2 cur;
  load(0, cur);
  for (int k0 = 0; k0 < a.d; k0 += 64) {
    Pair2 nxt;
    if (k0 + 64 < a.d) load(k0 + 64, nxt);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = k0 + 32 * h;
      const bool k_ok = k + 8 * kq < a.d;
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        const uint4 xv = cur.x[h][g];
        uint4 hv;
        hv.x = pack_f16x2(bf16lo(xv.x), bf16hi(xv.x));
        hv.y = pack_f16x2(bf16lo(xv.y), bf16hi(xv.y));
        hv.z = pack_f16x2(bf16lo(xv.z), bf16hi(xv.z));
        hv.w = pack_f16x2(bf16lo(xv.w), bf16hi(xv.w));
        if (k_ok && row_ok[g]) *reinterpret_cast<uint4*>(xo[g] + k) = hv;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          acc[g][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, hv),
                                                              __builtin_bit_cast(f16x8_t, cur.w[h][cb]), acc[g][cb],
                                                              0, 0, 0);
      }
    }
    cur = nxt;
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

// 16-row groups per wave: every wave reads the whole of W_bc once (from L2), so more rows per wave
// cut those reads; with 4 groups the 1.5B layer's 131,072-row conversion takes 0.215 ms, with 2
// groups 0.241 and with 1 group 0.296.
#ifndef HYMBA_CONV_ROW_GROUPS
#define HYMBA_CONV_ROW_GROUPS 4
#endif
constexpr int kConvRowGroups = HYMBA_CONV_ROW_GROUPS;

// Few rows (a decode step, the meta prefix): the same products and conversion, with one workgroup
// of kRowsWaves waves per 16 rows and 16-column block of B/C, and the 32-column steps of K split
// over its waves.  Each wave issues the loads of kRowsBatch steps before it uses any, and the
// waves' partial sums meet in LDS, added in wave order; the workgroups of column block 0 also
// store x16.  With whole rows per wave a 128-row call would run on a single CU, bound by the
// rate at which one CU can load (measured ~46 us for the 1.5B layer's 128 x 1600 inputs).
constexpr int kRowsWaves = 8;
constexpr int kRowsBatch = 8;
constexpr int64_t kFewRows = 2048;   // up to this many rows take the split-K kernel

__global__ __launch_bounds__(64 * kRowsWaves) void convert_bc_rows_kernel(ConvBcArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = lane & 15, kq = lane >> 4;
  const int cb = blockIdx.y;   // 16-column block of B/C
  const bool store_x = cb == 0;
  const int64_t row = (int64_t)blockIdx.x * 16 + i;
  const bool row_ok = row < a.rows;
  const bf16_t* xr = a.x + (row_ok ? row : a.rows - 1) * a.ldx + 8 * kq;
  half_t* xo = a.x16 + row * a.ldx16 + 8 * kq;
  const half_t* wr = a.wbc + (int64_t)(16 * cb + i) * a.ldw + 8 * kq;
  const int nsteps = (a.d + 31) / 32;
  const int s0 = wave * nsteps / kRowsWaves, s1 = (wave + 1) * nsteps / kRowsWaves;
  f32x4_t acc = f32x4_t{};
  for (int sb = s0; sb < s1; sb += kRowsBatch) {
    uint4 xv[kRowsBatch], wv[kRowsBatch];
#pragma unroll
    for (int j = 0; j < kRowsBatch; ++j) {
      const int k = (sb + j) * 32;   // xr, wr, xo already point at the lane's 8 columns
      const bool ok = sb + j < s1 && k + 8 * kq < a.d;   // d % 8 == 0: the 8 columns are all in or out
      xv[j] = ok ? *reinterpret_cast<const uint4*>(xr + k) : make_uint4(0u, 0u, 0u, 0u);
      wv[j] = ok ? *reinterpret_cast<const uint4*>(wr + k) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int j = 0; j < kRowsBatch; ++j) {
      const int k = (sb + j) * 32;
      const bool ok = sb + j < s1 && k + 8 * kq < a.d;
      uint4 hv;
      hv.x = pack_f16x2(bf16lo(xv[j].x), bf16hi(xv[j].x));
      hv.y = pack_f16x2(bf16lo(xv[j].y), bf16hi(xv[j].y));
      hv.z = pack_f16x2(bf16lo(xv[j].z), bf16hi(xv[j].z));
      hv.w = pack_f16x2(bf16lo(xv[j].w), bf16hi(xv[j].w));
      if (store_x && ok && row_ok) *reinterpret_cast<uint4*>(xo + k) = hv;
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, hv),
                                                   __builtin_bit_cast(f16x8_t, wv[j]), acc, 0, 0, 0);
    }
  }
  __shared__ f32x4_t part[kRowsWaves][64];
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {   // the waves' sums in order
    f32x4_t sum = part[0][lane];
#pragma unroll
    for (int w = 1; w < kRowsWaves; ++w) {
      const f32x4_t v = part[w][lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) sum[r] += v[r];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t orow = (int64_t)blockIdx.x * 16 + 4 * kq + r;
      if (orow < a.rows) a.bc[orow * a.ldbc + 16 * cb + i] = sum[r];
    }
  }
}

// Records in *flag whether any of the n fp16 values at p is inf or NaN (all exponent bits set):
// a bf16 weight beyond fp16's range became inf in the layer's fp16 copy.  Lane 0 of a wave that
// saw one stores 1 (every writer stores the same value).
__global__ __launch_bounds__(256) void nonfinite16_kernel(const uint16_t* __restrict__ p, int64_t n,
                                                          uint32_t* __restrict__ flag) {
  const int64_t n8 = n / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
    const uint4 v = reinterpret_cast<const uint4*>(p)[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) bad |= ((w[j] & 0x7c00u) == 0x7c00u) | ((w[j] & 0x7c000000u) == 0x7c000000u);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0)
    for (int64_t i = 8 * n8; i < n; ++i) bad |= (p[i] & 0x7c00u) == 0x7c00u;
  if (__builtin_amdgcn_ballot_w64(bad) != 0 && (threadIdx.x & 63) == 0) *flag = 1u;
}

}  // namespace

hipError_t launch_nonfinite16_check(const half_t* p, int64_t n, uint32_t* flag, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (reinterpret_cast<uintptr_t>(p) % 16) return hipErrorInvalidValue;
  const unsigned blocks = static_cast<unsigned>(std::min<int64_t>(1024, std::max<int64_t>(1, ceil_div(n / 8, 256))));
  hipLaunchKernelGGL(nonfinite16_kernel, dim3(blocks), dim3(256), 0, s, reinterpret_cast<const uint16_t*>(p), n,
                     flag);
  return hipGetLastError();
}

hipError_t launch_convert_bc(const ConvBcArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (a.d % 8 || (a.nbc != 16 && a.nbc != 32) || a.ldx % 8 || a.ldx16 % 8 || a.ldw % 8) return hipErrorInvalidValue;
  if (a.rows <= kFewRows) {
    const dim3 grid(static_cast<unsigned>(ceil_div(a.rows, 16)), static_cast<unsigned>(a.nbc / 16)),
        block(64 * kRowsWaves);
    hipLaunchKernelGGL(convert_bc_rows_kernel, grid, block, 0, s, a);
    return hipGetLastError();
  }
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
