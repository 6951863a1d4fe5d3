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
// exp uses A2 = A * log2(e), precomputed once per layer, so each (t, c, n)
// costs one v_exp_f32, two multiplies and two FMAs.  The diagonal recurrence is bound by
// this VALU work rather than by memory (the Griffin summary, hyeon-jae.tistory.com
// section 1, notes diagonal RNN layers are memory bound on TPU; here the
// per-state exp dominates).
#include "common.h"
#include "kernels.h"

namespace hymba {

namespace {

// Prefill mapping.  A channel's N states are split over WPC = N / NS waves of
// one workgroup (wave w owns states [w*NS, (w+1)*NS) of 64 consecutive
// channels, one channel per lane), which gives WPC times more waves than
// channels/64 and so fills every SIMD even at batch 16.  Time runs in chunks
// of TC steps, and everything a chunk needs is fetched one chunk ahead so HBM
// and L2 latency hide behind a chunk of arithmetic: u/dt into registers, the
// wave's B/C columns (uniform across its lanes) into registers and then into
// the wave's LDS slice, read back per step as broadcast LDS reads.  The
// per-wave partial outputs of a chunk are summed across the WPC waves through
// LDS once per chunk (double-buffered, one barrier per chunk).
constexpr int kTC = 16;

template <typename T, int N, int NS>
__global__ __launch_bounds__(64 * (N / NS)) void selective_scan_kernel(
    const T* __restrict__ u, const T* __restrict__ dt, int64_t ld, const float* __restrict__ bc, int64_t ld_bc,
    const float* __restrict__ A2, const float* __restrict__ Dp, const float* __restrict__ dt_bias,
    const float* __restrict__ h0, int64_t h0_bstride, T* __restrict__ y, int64_t ldy,
    float* __restrict__ h_out, int T_len, int E) {
  constexpr int WPC = N / NS;
  constexpr int Q = NS / 4;                 // float4 per step of B (and of C)
  constexpr int ITEMS = kTC * 2 * Q;        // float4 per chunk of this wave's B/C
  constexpr int PER_LANE = (ITEMS + 63) / 64;
  __shared__ float ys[2][WPC][kTC][64];
  __shared__ float4 bcs[2][WPC][kTC][2 * Q];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.y;
  const int c = blockIdx.x * 64 + lane;
  const bool active = c < E;
  const int cc = active ? c : E - 1;
  const int n0 = wave * NS;
  float a2[NS], h[NS];
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    a2[n] = A2[(int64_t)cc * N + n0 + n];
    h[n] = h0 ? h0[b * h0_bstride + (int64_t)cc * N + n0 + n] : 0.f;
  }
  const float Dc = wave == 0 ? Dp[cc] : 0.f;   // the skip term enters one partial sum only
  const float bias = dt_bias[cc];
  const int64_t row0 = (int64_t)b * T_len;
  const T* up = u + row0 * ld + cc;
  const T* dp = dt + row0 * ld + cc;
  const float* bcrow = bc + row0 * ld_bc;
  T* yrow = y + row0 * ldy + c;
  const int last = T_len - 1;

  // B/C item i of a chunk starting at t: step i / (2Q); j = i % (2Q) < Q -> B[n0 + 4j..],
  // else C[n0 + 4(j - Q)..]
  auto fetch_bc = [&](float4 (&r)[PER_LANE], int t) {
#pragma unroll
    for (int k = 0; k < PER_LANE; ++k) {
      const int i = lane + 64 * k;
      if (i < ITEMS) {
        const int st = i / (2 * Q), j = i % (2 * Q);
        const int64_t row = min(t + st, last);
        const int col = j < Q ? n0 + 4 * j : N + n0 + 4 * (j - Q);
        r[k] = *reinterpret_cast<const float4*>(bcrow + row * ld_bc + col);
      }
    }
  };
  auto stash_bc = [&](const float4 (&r)[PER_LANE], int bb) {
#pragma unroll
    for (int k = 0; k < PER_LANE; ++k) {
      const int i = lane + 64 * k;
      if (i < ITEMS) bcs[bb][wave][i / (2 * Q)][i % (2 * Q)] = r[k];
    }
  };

  T un[kTC], dn[kTC];
  float4 bcr[PER_LANE];
#pragma unroll
  for (int s = 0; s < kTC; ++s) {
    const int64_t r = min(s, last);
    un[s] = up[r * ld];
    dn[s] = dp[r * ld];
  }
  fetch_bc(bcr, 0);
  int buf = 0;
  stash_bc(bcr, buf);
  for (int t0 = 0; t0 < T_len; t0 += kTC) {
    T uc[kTC], dc[kTC];
#pragma unroll
    for (int s = 0; s < kTC; ++s) { uc[s] = un[s]; dc[s] = dn[s]; }
    // everything for the next chunk (rows clamped, always in bounds)
#pragma unroll
    for (int s = 0; s < kTC; ++s) {
      const int64_t r = min(t0 + kTC + s, last);
      un[s] = up[r * ld];
      dn[s] = dp[r * ld];
    }
    fetch_bc(bcr, t0 + kTC);
    const int len = min(kTC, T_len - t0);
    float part[kTC];
#pragma unroll
    for (int s = 0; s < kTC; ++s) {
      part[s] = 0.f;
      if (s < len) {
        float bb[NS], cb[NS];
#pragma unroll
        for (int q = 0; q < Q; ++q) {
          const float4 vb = bcs[buf][wave][s][q], vc = bcs[buf][wave][s][Q + q];
          bb[4 * q] = vb.x; bb[4 * q + 1] = vb.y; bb[4 * q + 2] = vb.z; bb[4 * q + 3] = vb.w;
          cb[4 * q] = vc.x; cb[4 * q + 1] = vc.y; cb[4 * q + 2] = vc.z; cb[4 * q + 3] = vc.w;
        }
        const float uv = static_cast<float>(uc[s]);
        const float delta = softplus_f(static_cast<float>(dc[s]) + bias);
        const float du = delta * uv;
        float acc = Dc * uv;
#pragma unroll
        for (int n = 0; n < NS; ++n) {
          const float dA = fast_exp2(delta * a2[n]);
          h[n] = fmaf(dA, h[n], du * bb[n]);
          acc = fmaf(cb[n], h[n], acc);
        }
        part[s] = acc;
      }
    }
    if constexpr (WPC == 1) {
#pragma unroll
      for (int s = 0; s < kTC; ++s)
        if (s < len && active) Elem<T>::store(yrow + (int64_t)(t0 + s) * ldy, part[s]);
    } else {
#pragma unroll
      for (int s = 0; s < kTC; ++s) ys[buf][wave][s][lane] = part[s];
      __syncthreads();
      for (int s = wave; s < len; s += WPC) {
        float yv = 0.f;
#pragma unroll
        for (int w = 0; w < WPC; ++w) yv += ys[buf][w][s][lane];
        if (active) Elem<T>::store(yrow + (int64_t)(t0 + s) * ldy, yv);
      }
    }
    buf ^= 1;
    stash_bc(bcr, buf);   // this wave's own slice: ordered by the wave's LDS queue
  }
  if (active && h_out) {
    float* ho = h_out + ((int64_t)b * E + c) * N + n0;
#pragma unroll
    for (int n = 0; n < NS; ++n) ho[n] = h[n];
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

// States per wave: the fewest waves per channel group (largest NS, least
// per-step overhead) that still gives ~1.5 waves per SIMD of the 1024.
inline int scan_states_per_wave(int B, int E, int N) {
  const int64_t groups = (int64_t)B * ceil_div(E, 64);
  int ns = N;
  while (ns > 4 && groups * (N / ns) < 1536) ns >>= 1;
  return ns;
}

template <typename T, int N, int NS>
void scan_launch(const ScanArgs<T>& a, hipStream_t s) {
  dim3 grid(static_cast<unsigned>(ceil_div(a.E, 64)), a.B), block(64 * (N / NS));
  hipLaunchKernelGGL((selective_scan_kernel<T, N, NS>), grid, block, 0, s, a.u, a.dt, a.ld, a.bc, a.ld_bc, a.A2,
                     a.D, a.dt_bias, a.h0, a.h0_bstride, a.y, a.ldy, a.h_out, a.T, a.E);
}

template <typename T>
hipError_t scan_dispatch(const ScanArgs<T>& a, hipStream_t s) {
  const int ns = scan_states_per_wave(a.B, a.E, a.N);
  if (a.N == 8) {
    if (ns == 8) scan_launch<T, 8, 8>(a, s);
    else scan_launch<T, 8, 4>(a, s);
  } else if (a.N == 16) {
    if (ns == 16) scan_launch<T, 16, 16>(a, s);
    else if (ns == 8) scan_launch<T, 16, 8>(a, s);
    else scan_launch<T, 16, 4>(a, s);
  } else {
    return hipErrorInvalidValue;
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
