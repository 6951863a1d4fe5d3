// SSM branch of the hybrid-head mixer: a diagonal selective scan.
//
// Method: Hymba summary (greeksharifa.github.io) section 2.1 (SSM heads fed by
// the shared input projection, recurrent summary in a fixed-size state) and
// section 2.3 (the state after the meta-token prefix acts as a learned initial
// state).  The recurrence itself is not printed on the pages; the reading used
// (Mamba-style, one decay per channel and state):
//   dt_t = softplus(dt_raw_t + dt_bias)
//   h_t[c, n] = exp(dt_t[c] * A[c, n]) * h_{t-1}[c, n] + dt_t[c] * u_t[c] * B_t[n]
//   y_t[c]    = sum_n C_t[n] * h_t[c, n] + D[c] * u_t[c]
// The gate (y * SiLU(z)) is applied in the fused epilogue.
//
// Prefill mapping: one lane per (sequence, channel) with all N fp32 states in
// VGPRs, walking the sequence in order; B_t and C_t are the same for every
// channel of a token, so a wave reads them through the scalar unit (uniform
// address) and every multiply takes them as SGPR operands.  exp uses
// A2 = A * log2(e), precomputed once per layer, so each (t, c, n) costs one
// v_exp_f32, two multiplies and two FMAs.  The diagonal recurrence is bound by
// this VALU work rather than by memory (the Griffin summary, hyeon-jae.tistory.com
// section 1, notes diagonal RNN layers are memory bound on TPU; here the
// per-state exp dominates).
#include "common.h"
#include "kernels.h"

namespace hymba {

namespace {

// Raw (unconverted) inputs of one time step.  Loads of the next step are
// issued into a second StepIn before the current step is computed and only
// converted when that step runs, so their latency hides behind a step's VALU
// work.  B/C are fp32 and wave-uniform: they land in SGPRs (scalar loads).
template <typename CT, int N>
struct StepIn {
  CT u, dt;
  float bc[2 * N];
  __device__ __forceinline__ void load(const CT* up, const CT* dp, const float* bcp) {
    u = *up;
    dt = *dp;
#pragma unroll
    for (int i = 0; i < 2 * N; ++i) bc[i] = bcp[i];
  }
  __device__ __forceinline__ float uf() const { return static_cast<float>(u); }
  __device__ __forceinline__ float dtf() const { return static_cast<float>(dt); }
  __device__ __forceinline__ float b(int n) const { return bc[n]; }
  __device__ __forceinline__ float c(int n) const { return bc[N + n]; }
};

template <typename T, int N>
__device__ __forceinline__ float scan_step(const StepIn<T, N>& in, const float (&a2)[N], float (&h)[N],
                                           float Dc, float bias) {
  const float uv = in.uf();
  const float delta = softplus_f(in.dtf() + bias);
  const float du = delta * uv;
  float acc = Dc * uv;
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const float dA = fast_exp2(delta * a2[n]);
    h[n] = fmaf(dA, h[n], du * in.b(n));
    acc = fmaf(in.c(n), h[n], acc);
  }
  return acc;
}

template <typename T, int N>
__global__ __launch_bounds__(64) void selective_scan_kernel(
    const T* __restrict__ u, const T* __restrict__ dt, int64_t ld, const float* __restrict__ bc, int64_t ld_bc,
    const float* __restrict__ A2, const float* __restrict__ Dp, const float* __restrict__ dt_bias,
    const float* __restrict__ h0, int64_t h0_bstride, T* __restrict__ y, int64_t ldy,
    float* __restrict__ h_out, int T_len, int E) {
  const int b = blockIdx.y;
  const int c = blockIdx.x * 64 + threadIdx.x;
  const bool active = c < E;
  const int cc = active ? c : E - 1;
  float a2[N], h[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    a2[n] = A2[(int64_t)cc * N + n];
    h[n] = h0 ? h0[b * h0_bstride + (int64_t)cc * N + n] : 0.f;
  }
  const float Dc = Dp[cc], bias = dt_bias[cc];
  const int64_t row0 = (int64_t)b * T_len;
  const T* up = u + row0 * ld + cc;
  const T* dp = dt + row0 * ld + cc;
  const float* bcp = bc + row0 * ld_bc;
  T* yp = y + row0 * ldy + cc;

  // Prefetches are unconditional (the row index is clamped to the last row) so
  // the number of loads in flight is the same on every path and the wait before
  // a step only covers that step's own inputs.
  StepIn<T, N> s0, s1;
  s0.load(up, dp, bcp);
  const int last = T_len - 1;
  for (int t = 0; t < T_len; t += 2) {
    const int64_t r1 = min(t + 1, last);
    s1.load(up + r1 * ld, dp + r1 * ld, bcp + r1 * ld_bc);
    const float y0 = scan_step<T, N>(s0, a2, h, Dc, bias);
    if (active) Elem<T>::store(yp + (int64_t)t * ldy, y0);
    if (t + 1 >= T_len) break;
    const int64_t r2 = min(t + 2, last);
    s0.load(up + r2 * ld, dp + r2 * ld, bcp + r2 * ld_bc);
    const float y1 = scan_step<T, N>(s1, a2, h, Dc, bias);
    if (active) Elem<T>::store(yp + (int64_t)(t + 1) * ldy, y1);
  }
  if (active && h_out) {
    float* ho = h_out + ((int64_t)b * E + c) * N;
#pragma unroll
    for (int n = 0; n < N; ++n) ho[n] = h[n];
  }
}

// Decode: one token per sequence.  N/4 consecutive lanes share a channel, each
// owning 4 states (one 16-byte state load and store); y is reduced across them.
template <typename T, int N>
__global__ __launch_bounds__(256) void ssm_step_kernel(StepArgs<T> a) {
  constexpr int LPC = N / 4;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.B * a.E * LPC;
  const bool active = gid < total;
  const int64_t g2 = active ? gid : total - 1;
  const int q = static_cast<int>(g2 % LPC);
  const int64_t ch = g2 / LPC;
  const int c = static_cast<int>(ch % a.E);
  const int64_t b = ch / a.E;
  const T* row = a.bc + b * a.ld;
  const float uv = Elem<T>::load(a.u + b * a.ld + c);
  const float dv = Elem<T>::load(a.dt + b * a.ld + c);
  const float delta = softplus_f(dv + a.dt_bias[c]);
  const float du = delta * uv;
  float4* hp = reinterpret_cast<float4*>(a.h + ch * N + 4 * q);
  float4 hv = *hp;
  const float4 a2 = *reinterpret_cast<const float4*>(a.A2 + (int64_t)c * N + 4 * q);
  float hs[4] = {hv.x, hv.y, hv.z, hv.w};
  const float a2s[4] = {a2.x, a2.y, a2.z, a2.w};
  float part = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = 4 * q + j;
    const float bn = Elem<T>::load(row + n), cn = Elem<T>::load(row + N + n);
    hs[j] = fmaf(fast_exp2(delta * a2s[j]), hs[j], du * bn);
    part = fmaf(cn, hs[j], part);
  }
#pragma unroll
  for (int off = 1; off < LPC; off <<= 1) part += __shfl_xor(part, off);
  if (active) {
    *hp = make_float4(hs[0], hs[1], hs[2], hs[3]);
    if (q == 0) Elem<T>::store(a.y + b * a.ldy + c, part + a.D[c] * uv);
  }
}

template <typename T>
hipError_t scan_dispatch(const ScanArgs<T>& a, hipStream_t s) {
  dim3 grid(static_cast<unsigned>(ceil_div(a.E, 64)), a.B), block(64);
  switch (a.N) {
    case 8:
      hipLaunchKernelGGL((selective_scan_kernel<T, 8>), grid, block, 0, s, a.u, a.dt, a.ld, a.bc, a.ld_bc, a.A2,
                         a.D, a.dt_bias, a.h0, a.h0_bstride, a.y, a.ldy, a.h_out, a.T, a.E);
      break;
    case 16:
      hipLaunchKernelGGL((selective_scan_kernel<T, 16>), grid, block, 0, s, a.u, a.dt, a.ld, a.bc, a.ld_bc, a.A2,
                         a.D, a.dt_bias, a.h0, a.h0_bstride, a.y, a.ldy, a.h_out, a.T, a.E);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t step_dispatch(const StepArgs<T>& a, hipStream_t s) {
  const int64_t lanes = (int64_t)a.B * a.E * (a.N / 4);
  dim3 grid(static_cast<unsigned>(ceil_div(lanes, 256))), block(256);
  switch (a.N) {
    case 8: hipLaunchKernelGGL((ssm_step_kernel<T, 8>), grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL((ssm_step_kernel<T, 16>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

__global__ void scale_copy_kernel(const float* __restrict__ src, float* __restrict__ dst, int64_t n,
                                  float scale) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i] * scale;
}

__global__ void fill_kernel(float* __restrict__ dst, int64_t n, float value) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = value;
}

}  // namespace

hipError_t launch_selective_scan(const ScanArgs<float>& a, hipStream_t s) { return scan_dispatch(a, s); }
hipError_t launch_selective_scan(const ScanArgs<half_t>& a, hipStream_t s) { return scan_dispatch(a, s); }
hipError_t launch_ssm_step(const StepArgs<float>& a, hipStream_t s) { return step_dispatch(a, s); }
hipError_t launch_ssm_step(const StepArgs<half_t>& a, hipStream_t s) { return step_dispatch(a, s); }

hipError_t launch_scale_copy(const float* src, float* dst, int64_t n, float scale, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(scale_copy_kernel, dim3(static_cast<unsigned>(ceil_div(n, 256))), dim3(256), 0, s,
                     src, dst, n, scale);
  return hipGetLastError();
}

hipError_t launch_fill(float* dst, int64_t n, float value, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3(static_cast<unsigned>(ceil_div(n, 256))), dim3(256), 0, s, dst, n, value);
  return hipGetLastError();
}

}  // namespace hymba
