// Kernels of the Griffin recurrent block (Griffin summary, hyeon-jae.tistory.com,
// sections 2.3 and 2.4, appendix A): the causal separable Conv1D of width 4 and
// the RG-LRU recurrence merged with the GeLU branch.
//
// The RG-LRU state is one number per channel, so channels alone (B * R) give
// few independent lanes; the recurrence h_t = a_t h_(t-1) + b_t therefore
// also runs in parallel over time inside a workgroup (the waves take
// consecutive steps of a tile and combine their (decay product, state)
// summaries), each coefficient computed once.  A lane takes two adjacent
// channels: a wave's loads of one time step cover 128 consecutive channels of
// a row (256 bytes of fp16 activations).
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace hymba {

namespace {

constexpr int kConvTaps = 4;
constexpr int kConvSteps = 16;  // time steps per conv thread (the taps stay in registers)
constexpr int kStepChunk = 8;   // time steps whose loads are issued together

// 16 loaded bytes -> floats
template <typename T> struct Unpack;
template <> struct Unpack<float> {
  static constexpr int n = 4;
  __device__ static __forceinline__ void run(const uint4 x, float (&v)[4]) {
    v[0] = __uint_as_float(x.x); v[1] = __uint_as_float(x.y); v[2] = __uint_as_float(x.z); v[3] = __uint_as_float(x.w);
  }
};
template <> struct Unpack<half_t> {
  static constexpr int n = 8;
  __device__ static __forceinline__ void run(const uint4 x, float (&v)[8]) {
    v[0] = f16lo(x.x); v[1] = f16hi(x.x); v[2] = f16lo(x.y); v[3] = f16hi(x.y);
    v[4] = f16lo(x.z); v[5] = f16hi(x.z); v[6] = f16lo(x.w); v[7] = f16hi(x.w);
  }
};

template <int V>
__device__ __forceinline__ void load_f32(const float* p, float (&v)[V]) {
#pragma unroll
  for (int e = 0; e < V; e += 4) {
    const float4 q = *reinterpret_cast<const float4*>(p + e);
    v[e] = q.x; v[e + 1] = q.y; v[e + 2] = q.z; v[e + 3] = q.w;
  }
}
template <int V>
__device__ __forceinline__ void store_f32(float* p, const float (&v)[V]) {
#pragma unroll
  for (int e = 0; e < V; e += 4) *reinterpret_cast<float4*>(p + e) = make_float4(v[e], v[e + 1], v[e + 2], v[e + 3]);
}

// Thread per (sequence, kConvSteps time steps, 16-byte chunk of R); consecutive threads take
// consecutive chunks of a row, so a wave's loads cover 1 KB of one row.  Each input row is read
// once per thread and slides through a three-row register window.
template <typename T>
__global__ __launch_bounds__(256) void griffin_conv_kernel(GriffinConvArgs<T> a) {
  constexpr int V = Unpack<T>::n;
  constexpr int H = kConvTaps - 1;
  const int cpr = a.R / V;
  const int tiles = static_cast<int>(ceil_div(a.seq, kConvSteps));
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)a.B * tiles * cpr) return;
  const int r0 = static_cast<int>(i % cpr) * V;
  const int64_t rest = i / cpr;
  const int t0 = static_cast<int>(rest % tiles) * kConvSteps;
  const int64_t b = rest / tiles;
  const int t1 = min(a.seq, t0 + kConvSteps);
  const T* __restrict__ u = a.u + b * a.seq * a.ld_u + r0;
  T* __restrict__ xc = a.xc + b * a.seq * a.ld_xc + r0;
  float w[kConvTaps][V];
#pragma unroll
  for (int k = 0; k < kConvTaps; ++k) load_f32<V>(a.w + k * a.R + r0, w[k]);
  float win[H][V];   // inputs at t-3, t-2, t-1
#pragma unroll
  for (int j = 0; j < H; ++j) {
    const int tt = t0 - H + j;
    if (tt >= 0) {
      Unpack<T>::run(*reinterpret_cast<const uint4*>(u + (int64_t)tt * a.ld_u), win[j]);
    } else if (a.hist) {
      load_f32<V>(a.hist + (b * H + (H + tt)) * a.R + r0, win[j]);
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e) win[j][e] = 0.f;
    }
  }
  auto step = [&](const uint4 raw, int t) {
    float x[V];
    Unpack<T>::run(raw, x);
    float acc[V];
#pragma unroll
    for (int e = 0; e < V; ++e)
      acc[e] = fmaf(w[0][e], x[e], fmaf(w[1][e], win[2][e], fmaf(w[2][e], win[1][e], w[3][e] * win[0][e])));
    Vec16<T>::store(xc + (int64_t)t * a.ld_xc, acc);
#pragma unroll
    for (int e = 0; e < V; ++e) {
      win[0][e] = win[1][e];
      win[1][e] = win[2][e];
      win[2][e] = x[e];
    }
  };
  if (t1 - t0 == kConvSteps) {
    uint4 raw[kConvSteps];
#pragma unroll
    for (int j = 0; j < kConvSteps; ++j) raw[j] = *reinterpret_cast<const uint4*>(u + (int64_t)(t0 + j) * a.ld_u);
#pragma unroll
    for (int j = 0; j < kConvSteps; ++j) step(raw[j], t0 + j);
  } else {
    for (int t = t0; t < t1; ++t) step(*reinterpret_cast<const uint4*>(u + (int64_t)t * a.ld_u), t);
  }
  // the last tile leaves the last H inputs in the window (read before anything is written: the
  // state may alias hist only when seq == 1, a single tile)
  if (a.state_out && t1 == a.seq) {
#pragma unroll
    for (int j = 0; j < H; ++j) store_f32<V>(a.state_out + (b * H + j) * a.R + r0, win[j]);
  }
}

// Fast transcendental pieces on the hardware exp2 / reciprocal / square root, accurate to a few
// 1e-7 (well inside the fp32 parity bar):
__device__ __forceinline__ float rcp_f(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float exp_f(float x) { return fast_exp2(x * kLog2e); }
__device__ __forceinline__ float sigmoid_f(float x) { return rcp_f(1.f + exp_f(-x)); }

// 1 - a^2 for a = e^la (la <= 0) without cancellation near a = 1: with z = 2 la, the Taylor
// series of -expm1(z) to z^6 for |z| < 1/4 (relative truncation error below |z|^6 / 5040 < 5e-8),
// else 1 - a a (then 1 - a^2 > 0.22 and the rounding of a costs at most a few 1e-7 relative).
__device__ __forceinline__ float one_minus_sq(float a, float la) {
  const float z = 2.f * la;
  float p = fmaf(z, 1.f / 720.f, 1.f / 120.f);
  p = fmaf(z, p, 1.f / 24.f);
  p = fmaf(z, p, 1.f / 6.f);
  p = fmaf(z, p, 0.5f);
  p = fmaf(z, p, 1.f);
  return z > -0.25f ? -z * p : fmaf(-a, a, 1.f);
}

// GeLU(v) = v Phi(v) = v (1 + erf(v / sqrt 2)) / 2, erf by the rational approximation of
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26 (|error| <= 1.5e-7).
__device__ __forceinline__ float gelu_f(float v) {
  const float x = fabsf(v) * 0.70710678118654752f;
  const float t = rcp_f(fmaf(0.3275911f, x, 1.f));
  float p = fmaf(t, 1.061405429f, -1.453152027f);
  p = fmaf(t, p, 1.421413741f);
  p = fmaf(t, p, -0.284496736f);
  p = fmaf(t, p, 0.254829592f);
  const float erf_abs = fmaf(-p * t, exp_f(-x * x), 1.f);
  return 0.5f * v * (1.f + copysignf(erf_abs, v));
}

// c softplus(-Lambda) = -c log sigmoid(Lambda)
__device__ __forceinline__ float decay_scale(float lam, float c) {
  return c * (fmaxf(-lam, 0.f) + log1pf(__expf(-fabsf(lam))));
}

// Raw buffer access (gfx9 buffer resource: base, stride 0, byte range).  The row offset goes in a
// scalar register, the lane's column offset in a vector register, so an access costs no vector
// address arithmetic.  The hardware range check covers only the vector offset, so the callers
// keep every row offset inside the buffer themselves.
constexpr int kBufferFlags = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kBufferFlags);
}

// Two consecutive elements: one 4-byte load for fp16, 8 bytes for fp32, kept packed until used.
template <typename T> struct Pair2;
template <> struct Pair2<half_t> {
  using Raw = uint32_t;
  __device__ static __forceinline__ Raw load(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0);
  }
  __device__ static __forceinline__ void unpack(Raw w, float (&v)[2]) { v[0] = f16lo(w); v[1] = f16hi(w); }
  __device__ static __forceinline__ void store(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff,
                                               const float (&v)[2]) {
    __builtin_amdgcn_raw_buffer_store_b32(pack_f16x2(v[0], v[1]), rs, voff, soff, 0);
  }
};
template <> struct Pair2<float> {
  using Raw = uint2;
  __device__ static __forceinline__ Raw load(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff) {
    const auto w = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, 0);
    return make_uint2(w[0], w[1]);
  }
  __device__ static __forceinline__ void unpack(Raw w, float (&v)[2]) {
    v[0] = __uint_as_float(w.x); v[1] = __uint_as_float(w.y);
  }
  __device__ static __forceinline__ void store(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff,
                                               const float (&v)[2]) {
    using U2 = unsigned __attribute__((ext_vector_type(2)));
    U2 w;
    w[0] = __float_as_uint(v[0]);
    w[1] = __float_as_uint(v[1]);
    __builtin_amdgcn_raw_buffer_store_b64(w, rs, voff, soff, 0);
  }
};

constexpr int kVpl = 2;        // channels per lane
constexpr int kWaveSteps = 8;  // time steps per wave and tile
constexpr int kMaxWaves = 8;

// RG-LRU + GeLU branch in one pass.  Workgroup = kW waves on 128 channels of one sequence, for
// the whole sequence; time runs in tiles of kW * 8 steps, wave w taking steps [8w, 8w + 8) of a
// tile.  A wave loads its steps (the next tile's loads are issued before the current tile is
// processed), computes a_t and b_t = sqrt(1 - a_t^2) i_t xc_t once, keeps them in registers and
// folds them into its summary (prod a_t, h from zero).  After one barrier every wave folds the
// summaries of the waves before it into the tile's carry-in (its start state) and all of them
// into the next tile's carry, reruns its steps from registers and writes y_t = h_t GeLU(v_t).
// The summaries are double-buffered in LDS by tile parity: a buffer is rewritten two tiles later,
// after a barrier every wave passes only once it has read it.
template <typename T, int kW>
__global__ __launch_bounds__(64 * kW) void rglru_kernel(RglruArgs<T> a) {
  using P = Pair2<T>;
  using Raw = typename P::Raw;
  __shared__ float2 sm[2][kW][64][kVpl];
  // the wave index is wave-uniform: readfirstlane tells the compiler (scalar buffer offsets)
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = (blockIdx.x * 64 + lane) * kVpl;
  const int64_t b = blockIdx.y;
  const bool on = r < a.R;
  const int rr = on ? r : 0;   // inactive lanes of a partial last group stay in the barriers
  float c_sp[kVpl], carry[kVpl];
#pragma unroll
  for (int e = 0; e < kVpl; ++e) {
    c_sp[e] = decay_scale(a.lam[rr + e], a.c);
    carry[e] = (on && a.h0) ? a.h0[b * a.R + r + e] : 0.f;
  }
  // one buffer resource per tensor and sequence; byte offsets: row in a scalar, column per lane
  const int64_t row0 = b * a.seq;
  constexpr uint32_t es = sizeof(T);
  const auto rs_g = buffer_rsrc(a.g + row0 * a.ld_g, static_cast<uint32_t>(a.seq * a.ld_g * es));
  const auto rs_x = buffer_rsrc(a.xc + row0 * a.ld_xc, static_cast<uint32_t>(a.seq * a.ld_xc * es));
  const auto rs_v = buffer_rsrc(a.v + row0 * a.ld_v, static_cast<uint32_t>(a.seq * a.ld_v * es));
  const auto rs_y = buffer_rsrc(a.y + row0 * a.ldy, static_cast<uint32_t>(a.seq * a.ldy * es));
  const uint32_t col = static_cast<uint32_t>(rr) * es, col_i = static_cast<uint32_t>(rr + a.R) * es;
  constexpr int kTile = kW * kWaveSteps;
  const int tiles = static_cast<int>(ceil_div(a.seq, kTile));
  struct Raws { Raw rho[kWaveSteps], iota[kWaveSteps], x[kWaveSteps], v[kWaveSteps]; };
  // steps past the sequence re-read its last row (a scalar clamp) and are masked below
  auto fetch = [&](int tile, Raws& q) {
    const int t0 = tile * kTile + w * kWaveSteps;
#pragma unroll
    for (int j = 0; j < kWaveSteps; ++j) {
      const uint32_t t = static_cast<uint32_t>(min(t0 + j, a.seq - 1));
      q.rho[j] = P::load(rs_g, col, t * static_cast<uint32_t>(a.ld_g) * es);
      q.iota[j] = P::load(rs_g, col_i, t * static_cast<uint32_t>(a.ld_g) * es);
      q.x[j] = P::load(rs_x, col, t * static_cast<uint32_t>(a.ld_xc) * es);
      q.v[j] = P::load(rs_v, col, t * static_cast<uint32_t>(a.ld_v) * es);
    }
  };
  auto is_full = [&](int tile) { return on && tile * kTile + (w + 1) * kWaveSteps <= a.seq; };
  float at[kWaveSteps][kVpl], bt[kWaveSteps][kVpl];
  // a_t, b_t of the slice and its summary (prod a_t, h from zero)
  auto coeffs = [&](auto full, const Raws& cur, int t0, float (&A)[kVpl], float (&H)[kVpl]) {
#pragma unroll
    for (int e = 0; e < kVpl; ++e) { A[e] = 1.f; H[e] = 0.f; }
#pragma unroll
    for (int j = 0; j < kWaveSteps; ++j) {
      float rho[kVpl], iota[kVpl], x[kVpl];
      P::unpack(cur.rho[j], rho);
      P::unpack(cur.iota[j], iota);
      P::unpack(cur.x[j], x);
      const bool valid = decltype(full)::value || (on && t0 + j < a.seq);
#pragma unroll
      for (int e = 0; e < kVpl; ++e) {
        const float la = -c_sp[e] * sigmoid_f(rho[e]);   // log a_t = c r_t log sigmoid(Lambda)
        const float ae = exp_f(la);
        const float be = __builtin_amdgcn_sqrtf(one_minus_sq(ae, la)) * sigmoid_f(iota[e]) * x[e];
        at[j][e] = valid ? ae : 1.f;
        bt[j][e] = valid ? be : 0.f;
        H[e] = fmaf(at[j][e], H[e], bt[j][e]);
        A[e] *= at[j][e];
      }
    }
  };
  // rerun of the slice from its start state h, writing y_t = h_t GeLU(v_t)
  auto outputs = [&](auto full, const Raws& cur, int t0, float (&h)[kVpl]) {
#pragma unroll
    for (int j = 0; j < kWaveSteps; ++j) {
      float vv[kVpl], out[kVpl];
      P::unpack(cur.v[j], vv);
#pragma unroll
      for (int e = 0; e < kVpl; ++e) {
        h[e] = fmaf(at[j][e], h[e], bt[j][e]);
        out[e] = h[e] * gelu_f(vv[e]);
      }
      if (decltype(full)::value || (on && t0 + j < a.seq))
        P::store(rs_y, col, static_cast<uint32_t>(t0 + j) * static_cast<uint32_t>(a.ldy) * es, out);
    }
  };
  using Full = std::true_type;
  using Part = std::false_type;
  Raws nxt;
  fetch(0, nxt);
  for (int tile = 0; tile < tiles; ++tile) {
    const Raws cur = nxt;
    if (tile + 1 < tiles) fetch(tile + 1, nxt);
    const int t0 = tile * kTile + w * kWaveSteps;
    const bool full = is_full(tile);
    float A[kVpl], H[kVpl];
    if (full) coeffs(Full{}, cur, t0, A, H);
    else coeffs(Part{}, cur, t0, A, H);
    const int p = tile & 1;
#pragma unroll
    for (int e = 0; e < kVpl; ++e) sm[p][w][lane][e] = make_float2(A[e], H[e]);
    __syncthreads();
    float h[kVpl];
#pragma unroll
    for (int e = 0; e < kVpl; ++e) h[e] = carry[e];
#pragma unroll
    for (int u = 0; u < kW; ++u) {
      float2 q[kVpl];
#pragma unroll
      for (int e = 0; e < kVpl; ++e) q[e] = sm[p][u][lane][e];
      if (u == w) {
#pragma unroll
        for (int e = 0; e < kVpl; ++e) h[e] = carry[e];   // the start state of this wave's steps
      }
#pragma unroll
      for (int e = 0; e < kVpl; ++e) carry[e] = fmaf(q[e].x, carry[e], q[e].y);
    }
    if (full) outputs(Full{}, cur, t0, h);
    else outputs(Part{}, cur, t0, h);
  }
  if (on && w == 0 && a.h_out) {
#pragma unroll
    for (int e = 0; e < kVpl; ++e) a.h_out[b * a.R + r + e] = carry[e];
  }
}

template <typename T>
hipError_t conv_dispatch(const GriffinConvArgs<T>& a, hipStream_t s) {
  constexpr int V = Unpack<T>::n;
  if (a.R % V) return hipErrorInvalidValue;
  const int64_t n = (int64_t)a.B * ceil_div(a.seq, kConvSteps) * (a.R / V);
  if (n <= 0) return hipSuccess;
  if (ceil_div(n, 256) > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((griffin_conv_kernel<T>), dim3(static_cast<unsigned>(ceil_div(n, 256))), dim3(256), 0, s, a);
  return hipGetLastError();
}

// waves per workgroup: enough for the sequence, at most kMaxWaves
template <typename T>
hipError_t rglru_dispatch(const RglruArgs<T>& a, hipStream_t s) {
  if (a.B <= 0 || a.seq <= 0) return hipSuccess;
  if (a.R % kVpl || a.B > 65535) return hipErrorInvalidValue;
  // one sequence of each tensor must fit a buffer's 31-bit byte range
  const int64_t ld = std::max(std::max(a.ld_g, a.ld_xc), std::max(a.ld_v, a.ldy));
  if ((int64_t)a.seq * ld * (int64_t)sizeof(T) >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(ceil_div(a.R, 64 * kVpl)), a.B);
  const int64_t need = ceil_div(a.seq, kWaveSteps);
  if (need >= 8) hipLaunchKernelGGL((rglru_kernel<T, 8>), grid, dim3(64 * 8), 0, s, a);
  else if (need >= 4) hipLaunchKernelGGL((rglru_kernel<T, 4>), grid, dim3(64 * 4), 0, s, a);
  else if (need >= 2) hipLaunchKernelGGL((rglru_kernel<T, 2>), grid, dim3(64 * 2), 0, s, a);
  else hipLaunchKernelGGL((rglru_kernel<T, 1>), grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_griffin_conv(const GriffinConvArgs<float>& a, hipStream_t s) { return conv_dispatch(a, s); }
hipError_t launch_griffin_conv(const GriffinConvArgs<half_t>& a, hipStream_t s) { return conv_dispatch(a, s); }
hipError_t launch_rglru(const RglruArgs<float>& a, hipStream_t s) { return rglru_dispatch(a, s); }
hipError_t launch_rglru(const RglruArgs<half_t>& a, hipStream_t s) { return rglru_dispatch(a, s); }

}  // namespace hymba
