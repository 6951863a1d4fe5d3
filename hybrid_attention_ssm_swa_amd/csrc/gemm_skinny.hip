// Weight-streaming GEMM for few rows (decode): Y[M, N] = X[M, K] . W[N, K]^T with
// 16-bit operands and fp32 accumulation on v_mfma_f32_32x32x16_{f16,bf16}.
//
// At M ~ 128 the product is bound by reading W once from HBM (K*N 16-bit words
// against 2*M*K*N flops), and the whole difficulty is keeping enough of W in
// flight on enough CUs:
//  * a workgroup of 4 waves owns 64 output features for up to 128 rows (wave w
//    takes rows [32w, 32w + 32)) and at most kC (8, 4 or 2) chunks of 64 k;
//    K is split over workgroups so that there are ~256 of them;
//  * each workgroup issues all its loads at once (straight-line code, no loop
//    that would wait for one batch before issuing the next), stages its W
//    chunks in LDS (row stride 144 B) behind one barrier, and runs the MFMAs;
//  * X fragments (16 bytes per lane) go straight to registers (X is small and
//    stays in L2) and are converted to W's type there when X is bf16 and W fp16
//    (exact in range);
//  * the product is computed transposed, C = W_chunk . X^T, so each lane ends
//    with 4 consecutive features of one row per register group;
//  * with more than one split the workgroups write fp32 partial sums and a
//    second kernel adds them in split order (deterministic) and writes y.
// An optional fp32 copy of the output columns [c0, c1) goes to y32 (the decode
// path's B/C columns, which the scan reads in fp32).
#include "common.h"
#include "kernels.h"

namespace hymba {

namespace {

constexpr int kSkF = 64;          // features per workgroup
constexpr int kSkM = 128;         // rows per workgroup (4 waves x 32)
constexpr int kSkK = 64;          // k per chunk
constexpr int kSkStr = kSkK + 8;  // LDS row stride in 16-bit words (144 bytes)

struct __align__(16) Q4 { uint32_t x, y, z, w; };

// v if keep, else zeros: per 32-bit word (a select of the whole struct is lowered through
// scratch memory)
__device__ __forceinline__ Q4 keep_or_zero(bool keep, Q4 v) {
  Q4 r;
  r.x = keep ? v.x : 0u;
  r.y = keep ? v.y : 0u;
  r.z = keep ? v.z : 0u;
  r.w = keep ? v.w : 0u;
  return r;
}

template <typename WT> struct Mfma;
template <> struct Mfma<half_t> {
  __device__ static __forceinline__ f32x16_t run(Q4 a, Q4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
  }
};
template <> struct Mfma<bf16_t> {
  __device__ static __forceinline__ f32x16_t run(Q4 a, Q4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  }
};

// 8 elements of X's type -> 8 elements of W's type
template <typename XT, typename WT> struct ToW {
  __device__ static __forceinline__ Q4 run(Q4 v) { return v; }
};
template <> struct ToW<bf16_t, half_t> {
  __device__ static __forceinline__ Q4 run(Q4 v) {
    Q4 r;
    r.x = pack_f16x2(bf16lo(v.x), bf16hi(v.x));
    r.y = pack_f16x2(bf16lo(v.y), bf16hi(v.y));
    r.z = pack_f16x2(bf16lo(v.z), bf16hi(v.z));
    r.w = pack_f16x2(bf16lo(v.w), bf16hi(v.w));
    return r;
  }
};

template <typename OT> struct Out4;
template <> struct Out4<half_t> {
  __device__ static __forceinline__ void store(half_t* p, float a, float b, float c, float d) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_f16x2(a, b), pack_f16x2(c, d));
  }
};
template <> struct Out4<bf16_t> {
  __device__ static __forceinline__ void store(bf16_t* p, float a, float b, float c, float d) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
  }
};
template <> struct Out4<float> {
  __device__ static __forceinline__ void store(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  }
};

// Buffer resource (gfx9: stride 0, byte range; reads whose vector offset is past the range
// return 0) built from wave-uniform values, so that its loads need no per-lane loop.
// readfirstlane returns a signed int: each half goes through uint32_t before widening, or a low
// word with bit 31 set would sign-extend into the high word and wreck the base address.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* p, int64_t bytes) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32)));
  const uint64_t u = static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32);
  const int n = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes < INT32_MAX ? bytes : INT32_MAX));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), 0, n, 0x00020000);
}

// One workgroup: 64 features x up to 128 rows x at most kC chunks of K (split s of S).  All of
// its loads are issued first (straight-line code: every chunk of W and X in flight at once), the
// W chunks are staged in LDS behind a single barrier, then the MFMAs run.  With S == 1 the
// workgroup writes y (and y32) itself, else its fp32 partial sums go to part[s][m][n].
template <typename WT, typename XT, typename OT, int kC>
__global__ __launch_bounds__(256) void skinny_gemm_kernel(SkinnyArgs<WT, XT, OT> a, float* part, int S) {
  __shared__ __align__(16) uint16_t wl[kC][kSkF * kSkStr];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int f0 = blockIdx.x * kSkF;
  const int split = blockIdx.y;
  const int m0 = blockIdx.z * kSkM + w * 32;
  const int nch = static_cast<int>(ceil_div(a.K, kSkK));
  const int cbeg = split * kC;
  const int k_hi = min((cbeg + kC) * kSkK, a.K);   // this split's k range [cbeg*64, k_hi)
  // Operands are read through buffer resources with the whole byte offset in the per-lane
  // offset: the hardware range check covers that offset (not the scalar one), so reads past the
  // end of a matrix return zeros instead of touching memory.
  const auto rs_w = uniform_rsrc(a.w, int64_t(a.N) * a.ldw * 2);
  const auto rs_x = uniform_rsrc(a.x, int64_t(a.M) * a.ldx * 2);
  // W chunk: 512 segments of 16 bytes, two per thread; rows past N load row N-1 (never stored)
  int wrow[2], wseg[2];
  uint32_t wvo[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int idx = tid + q * 256;
    wrow[q] = idx >> 3;
    wseg[q] = idx & 7;
    wvo[q] = static_cast<uint32_t>(((int64_t)min(f0 + wrow[q], a.N - 1) * a.ldw + wseg[q] * 8) * 2);
  }
  // X fragment: row m0 + lane % 32 (rows past M load row M-1), k offset 8 * (lane / 32)
  const uint32_t xvo = static_cast<uint32_t>(((int64_t)min(m0 + (lane & 31), a.M - 1) * a.ldx + 8 * (lane >> 5)) * 2);
  auto ld = [](__amdgpu_buffer_rsrc_t rs, uint32_t vo) {
    return __builtin_bit_cast(Q4, __builtin_amdgcn_raw_buffer_load_b128(rs, vo, 0, 0));
  };

  Q4 wr[kC][2], xr[kC][4];
#pragma unroll
  for (int c = 0; c < kC; ++c) {   // chunks past the split or past K: zeros, or masked below
    const uint32_t kb = static_cast<uint32_t>(cbeg + c) * kSkK * 2;
    wr[c][0] = ld(rs_w, wvo[0] + kb);
    wr[c][1] = ld(rs_w, wvo[1] + kb);
#pragma unroll
    for (int s = 0; s < 4; ++s) xr[c][s] = ld(rs_x, xvo + s * 32 + kb);
  }
#pragma unroll
  for (int c = 0; c < kC; ++c) {
    const int kc = (cbeg + c) * kSkK;
#pragma unroll
    for (int q = 0; q < 2; ++q)
      *reinterpret_cast<Q4*>(&wl[c][wrow[q] * kSkStr + wseg[q] * 8]) = keep_or_zero(kc + wseg[q] * 8 < k_hi, wr[c][q]);
  }
  __syncthreads();

  f32x16_t acc[2] = {f32x16_t{}, f32x16_t{}};
  const int nc = min(kC, nch - cbeg);
#pragma unroll
  for (int c = 0; c < kC; ++c) {
    if (c < nc) {   // uniform
      const int kc = (cbeg + c) * kSkK;
      const uint16_t* base = &wl[c][(lane & 31) * kSkStr + 8 * (lane >> 5)];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const Q4 a0 = *reinterpret_cast<const Q4*>(base + s * 16);
        const Q4 a1 = *reinterpret_cast<const Q4*>(base + 32 * kSkStr + s * 16);
        const Q4 xb = keep_or_zero(kc + s * 16 + 8 * (lane >> 5) < k_hi, ToW<XT, WT>::run(xr[c][s]));
        acc[0] = Mfma<WT>::run(a0, xb, acc[0]);
        acc[1] = Mfma<WT>::run(a1, xb, acc[1]);
      }
    }
  }

  // lane: row m0 + lane % 32; register group g of block fb: features f0 + 32 fb + 8 g + 4 (lane / 32) + 0..3
  const int m = m0 + (lane & 31);
  if (m >= a.M) return;
#pragma unroll
  for (int fb = 0; fb < 2; ++fb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int f = f0 + 32 * fb + 8 * g + 4 * (lane >> 5);
      if (f >= a.N) continue;   // N % 4 == 0: a group is wholly in or out
      const float v0 = acc[fb][4 * g], v1 = acc[fb][4 * g + 1], v2 = acc[fb][4 * g + 2], v3 = acc[fb][4 * g + 3];
      if (S == 1) {
        Out4<OT>::store(a.y + (int64_t)m * a.ldy + f, v0, v1, v2, v3);
        if (a.y32 && f >= a.c0 && f < a.c1)   // c0, c1 multiples of 4
          Out4<float>::store(a.y32 + (int64_t)m * a.ldy32 + (f - a.c0), v0, v1, v2, v3);
      } else {
        Out4<float>::store(part + ((int64_t)split * a.M + m) * a.N + f, v0, v1, v2, v3);
      }
    }
}

// y[m, n..n+3] = sum over the S splits of part[s][m][n..n+3], in split order
template <typename WT, typename XT, typename OT>
__global__ __launch_bounds__(256) void skinny_reduce_kernel(SkinnyArgs<WT, XT, OT> a, const float* part, int S) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int n4 = a.N / 4;
  if (i >= (int64_t)a.M * n4) return;
  const int m = static_cast<int>(i / n4), f = static_cast<int>(i % n4) * 4;
  float4 s4 = *reinterpret_cast<const float4*>(part + (int64_t)m * a.N + f);
  for (int s = 1; s < S; ++s) {
    const float4 p = *reinterpret_cast<const float4*>(part + ((int64_t)s * a.M + m) * a.N + f);
    s4.x += p.x; s4.y += p.y; s4.z += p.z; s4.w += p.w;
  }
  Out4<OT>::store(a.y + (int64_t)m * a.ldy + f, s4.x, s4.y, s4.z, s4.w);
  if (a.y32 && f >= a.c0 && f < a.c1) Out4<float>::store(a.y32 + (int64_t)m * a.ldy32 + (f - a.c0), s4.x, s4.y, s4.z, s4.w);
}

template <typename WT, typename XT, typename OT>
hipError_t skinny_dispatch(const SkinnyArgs<WT, XT, OT>& a, float* part, size_t part_bytes, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.N % 4 || a.K % 8 || a.K <= 0 || a.ldw % 8 || a.ldx % 8 || a.ldy % 4 || a.c0 % 4 || a.c1 % 4 ||
      (a.y32 && a.ldy32 % 4))
    return hipErrorInvalidValue;
  if (reinterpret_cast<uintptr_t>(a.w) % 16 || reinterpret_cast<uintptr_t>(a.x) % 16 ||
      reinterpret_cast<uintptr_t>(a.y) % 16 || reinterpret_cast<uintptr_t>(a.y32) % 16 ||
      reinterpret_cast<uintptr_t>(part) % 16)
    return hipErrorInvalidValue;
  const SkinnyPlan pl = skinny_plan(a.M, a.N, a.K);
  // buffer offsets are 32-bit: each matrix plus the reach of a split's last chunk stays below 2 GiB
  const int64_t reach = int64_t(pl.S) * pl.kC * kSkK * 2;
  if ((int64_t)a.N * a.ldw * 2 + reach >= INT32_MAX || (int64_t)a.M * a.ldx * 2 + reach >= INT32_MAX)
    return hipErrorInvalidValue;
  if (pl.S > 1 && (!part || part_bytes < pl.part_bytes)) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(ceil_div(a.N, kSkF)), static_cast<unsigned>(pl.S),
                  static_cast<unsigned>(ceil_div(a.M, kSkM)));
  if (pl.kC == 8) hipLaunchKernelGGL((skinny_gemm_kernel<WT, XT, OT, 8>), grid, dim3(256), 0, s, a, part, pl.S);
  else if (pl.kC == 4) hipLaunchKernelGGL((skinny_gemm_kernel<WT, XT, OT, 4>), grid, dim3(256), 0, s, a, part, pl.S);
  else hipLaunchKernelGGL((skinny_gemm_kernel<WT, XT, OT, 2>), grid, dim3(256), 0, s, a, part, pl.S);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.S == 1) return e;
  const int64_t n = (int64_t)a.M * (a.N / 4);
  hipLaunchKernelGGL((skinny_reduce_kernel<WT, XT, OT>), dim3(static_cast<unsigned>(ceil_div(n, 256))), dim3(256), 0,
                     s, a, part, pl.S);
  return hipGetLastError();
}

}  // namespace

// Split of K: at most kC chunks of 64 per workgroup, the largest kC (fewest partial sums) that
// still gives ~256 workgroups, i.e. one per CU.
SkinnyPlan skinny_plan(int M, int N, int K) {
  SkinnyPlan p;
  const int64_t tiles = ceil_div(N, kSkF) * ceil_div(M, kSkM);
  const int64_t nch = ceil_div(K, kSkK);
  for (int kc : {8, 4, 2}) {
    p.kC = kc;
    p.S = static_cast<int>(ceil_div(nch, kc));
    if (tiles * p.S >= 256) break;
  }
  p.part_bytes = p.S > 1 ? static_cast<size_t>(p.S) * M * N * sizeof(float) : 0;
  return p;
}

hipError_t launch_skinny_gemm(const SkinnyArgs<half_t, half_t, half_t>& a, float* part, size_t bytes, hipStream_t s) {
  return skinny_dispatch(a, part, bytes, s);
}
hipError_t launch_skinny_gemm(const SkinnyArgs<half_t, bf16_t, half_t>& a, float* part, size_t bytes, hipStream_t s) {
  return skinny_dispatch(a, part, bytes, s);
}
hipError_t launch_skinny_gemm(const SkinnyArgs<half_t, half_t, bf16_t>& a, float* part, size_t bytes, hipStream_t s) {
  return skinny_dispatch(a, part, bytes, s);
}
hipError_t launch_skinny_gemm(const SkinnyArgs<bf16_t, bf16_t, bf16_t>& a, float* part, size_t bytes, hipStream_t s) {
  return skinny_dispatch(a, part, bytes, s);
}

}  // namespace hymba
