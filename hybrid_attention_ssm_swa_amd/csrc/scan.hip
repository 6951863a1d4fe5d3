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
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace hymba {

namespace {

// Prefill mapping.  A channel's N states are split over WPC = N / NS waves of
// one workgroup (wave w owns states [w*NS, (w+1)*NS) of 64 consecutive
// channels, one channel per lane), which gives WPC times more waves than
// channels/64 and so keeps several waves on every SIMD even at batch 16.
// Time runs in chunks of kTC steps with everything a chunk needs fetched one
// chunk ahead, so HBM/L2 latency hides behind a chunk of arithmetic.  Work
// shared by the WPC waves of a channel is done once per workgroup and passed
// through LDS: wave w turns the raw dt/u of steps s = w (mod WPC) of the next
// chunk into (delta, delta*u) pairs, the workgroup loads the chunk's B/C rows
// (uniform over the 64 channels) once, and every wave reads both back per
// step (B/C as broadcast reads).  Each wave's partial sums over its states
// meet in LDS once per chunk; the wave that prepared step s also adds the skip
// term D*u and stores y.
//
// Time segments.  When B * E / 64 channel groups give too few waves to fill the SIMDs (few
// long sequences), time is cut into S segments of seg_len steps (a multiple of the chunk) and
// the scan runs in two launches.  The summary launch runs every segment but the last from a zero
// state and keeps only its end state h_end[j] and its total step sum_t delta_t per channel.  The
// scan launch then runs every segment at once: segment j starts from the true state at its
// beginning, which the recurrence being linear in h gives in closed form from the summaries,
//   H_0 = h0,  H_{i+1} = exp2(A2 * sum_delta_i) * H_i + h_end[i]
// (the product of a segment's decays exp2(delta_t A2) is exp2(A2 sum_t delta_t)), and writes y.
// That is about 1.6 times the arithmetic of one pass, for S times the waves.
constexpr int kTC = 16;

template <int NS> struct BcVec { typedef float4 type; };
template <> struct BcVec<2> { typedef float2 type; };

// kSummary: the summary launch (no y; end state and step sum of segment blockIdx.z into seg_h,
// seg_d).  Otherwise segment blockIdx.z of seg_len steps, started from the summaries of the
// segments before it; the last segment writes h_out.  One segment of T_len steps is the plain scan.
// seg_h: [S - 1][B][E][N], seg_d: [S - 1][B][E] (fp32).
template <typename T, int N, int NS, bool kSummary>
__global__ __launch_bounds__(64 * (N / NS)) void selective_scan_kernel(
    const T* __restrict__ u, const T* __restrict__ dt, int64_t ld, const float* __restrict__ bc, int64_t ld_bc,
    const float* __restrict__ A2, const float* __restrict__ Dp, const float* __restrict__ dt_bias,
    const float* __restrict__ h0, int64_t h0_bstride, T* __restrict__ y, int64_t ldy,
    float* __restrict__ h_out, int T_len, int E, int seg_len, float* __restrict__ seg_h,
    float* __restrict__ seg_d) {
  constexpr int WPC = N / NS;
  constexpr int SPW = kTC / WPC;                   // steps each wave prepares per chunk
  constexpr int ROW4 = 2 * N / 4;                  // float4 per B/C row
  constexpr int ITEMS = kTC * ROW4;                // float4 per chunk of B/C rows
  constexpr int PER_T = (ITEMS + 64 * WPC - 1) / (64 * WPC);
  typedef typename BcVec<NS>::type BV;
  constexpr int VW = sizeof(BV) / sizeof(float);
  static_assert(kTC % WPC == 0 && NS % VW == 0, "scan tiling");
  __shared__ float2 dd[2][kTC][64];                // (delta, delta * u) per step and channel
  __shared__ float4 bcs[2][kTC][ROW4];             // B row then C row per step
  __shared__ float ys[WPC > 1 ? WPC : 1][kTC][64]; // per-wave partial y of a chunk
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.y;
  const int nb = gridDim.y;
  const int seg = blockIdx.z;
  const int c = blockIdx.x * 64 + lane;
  const bool active = c < E;
  const int cc = active ? c : E - 1;
  const int n0 = wave * NS;
  const int t_begin = seg * seg_len;
  const int T_seg = min(seg_len, T_len - t_begin);   // >= 1: the launch has ceil(T_len / seg_len) segments
  float a2[NS], h[NS];
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    a2[n] = A2[(int64_t)cc * N + n0 + n];
    h[n] = (!kSummary && h0) ? h0[b * h0_bstride + (int64_t)cc * N + n0 + n] : 0.f;
  }
  if constexpr (!kSummary) {
    for (int i = 0; i < seg; ++i) {   // carry the state over the segments before this one
      const int64_t ch = ((int64_t)i * nb + b) * E + cc;
      const float sd = seg_d[ch];
#pragma unroll
      for (int n = 0; n < NS; ++n) h[n] = fmaf(fast_exp2(sd * a2[n]), h[n], seg_h[ch * N + n0 + n]);
    }
  }
  const float Dc = Dp[cc];
  const float bias = dt_bias[cc];
  const int64_t row0 = (int64_t)b * T_len + t_begin;
  const T* up = u + row0 * ld + cc;
  const T* dp = dt + row0 * ld + cc;
  const float* bcrow = bc + row0 * ld_bc;
  T* yrow = y + row0 * ldy + c;
  const int last = T_seg - 1;
  float dsum = 0.f;   // summary: this wave's share of the segment's step sum

  T un[SPW], dn[SPW];
  float4 bcr[PER_T];
  // raw inputs of chunk t (rows clamped: always in bounds); this wave's steps s = wave + WPC j
  auto fetch = [&](int t) {
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int64_t r = min(t + wave + WPC * j, last);
      un[j] = up[r * ld];
      dn[j] = dp[r * ld];
    }
#pragma unroll
    for (int k = 0; k < PER_T; ++k) {
      const int i = threadIdx.x + 64 * WPC * k;
      if (i < ITEMS) {
        const int64_t r = min(t + i / ROW4, last);
        bcr[k] = *reinterpret_cast<const float4*>(bcrow + r * ld_bc + 4 * (i % ROW4));
      }
    }
  };
  // publish the chunk fetched for step t into LDS buffer bb; returns D * u of this wave's steps
  float skip_next[SPW];
  auto publish = [&](int bb, int t) {
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const float uv = static_cast<float>(un[j]);
      const float delta = softplus_f(static_cast<float>(dn[j]) + bias);
      dd[bb][wave + WPC * j][lane] = make_float2(delta, delta * uv);
      skip_next[j] = Dc * uv;
      if (kSummary && t + wave + WPC * j <= last) dsum += delta;
    }
#pragma unroll
    for (int k = 0; k < PER_T; ++k) {
      const int i = threadIdx.x + 64 * WPC * k;
      if (i < ITEMS) bcs[bb][i / ROW4][i % ROW4] = bcr[k];
    }
  };

  fetch(0);
  publish(0, 0);
  float skip[SPW];
#pragma unroll
  for (int j = 0; j < SPW; ++j) skip[j] = skip_next[j];
  fetch(kTC);
  __syncthreads();
  int buf = 0;
  for (int t0 = 0; t0 < T_seg; t0 += kTC) {
    publish(buf ^ 1, t0 + kTC);   // chunk t0 + kTC (fetched one chunk ago)
    fetch(t0 + 2 * kTC);
    const int len = min(kTC, T_seg - t0);
    const float* bcsf = reinterpret_cast<const float*>(&bcs[buf][0][0]);
    float part[kTC];
    // full chunks take a branch-free copy of the step loop; only the last chunk checks len
    auto steps = [&](auto full) {
#pragma unroll
      for (int s = 0; s < kTC; ++s) {
        part[s] = 0.f;
        if (decltype(full)::value || s < len) {
          const float2 d = dd[buf][s][lane];
          float bb[NS], cb[NS];
#pragma unroll
          for (int q = 0; q < NS / VW; ++q) {
            const BV vb = *reinterpret_cast<const BV*>(bcsf + s * 2 * N + n0 + VW * q);
            const float* pb = reinterpret_cast<const float*>(&vb);
#pragma unroll
            for (int e = 0; e < VW; ++e) bb[VW * q + e] = pb[e];
            if constexpr (!kSummary) {
              const BV vc = *reinterpret_cast<const BV*>(bcsf + s * 2 * N + N + n0 + VW * q);
              const float* pc = reinterpret_cast<const float*>(&vc);
#pragma unroll
              for (int e = 0; e < VW; ++e) cb[VW * q + e] = pc[e];
            }
          }
          float acc = 0.f;
#pragma unroll
          for (int n = 0; n < NS; ++n) {
            const float dA = fast_exp2(d.x * a2[n]);
            h[n] = fmaf(dA, h[n], d.y * bb[n]);
            if constexpr (!kSummary) acc = fmaf(cb[n], h[n], acc);
          }
          part[s] = acc;
        }
      }
    };
    if (len == kTC) steps(std::true_type{});
    else steps(std::false_type{});
    if constexpr (kSummary) {
      __syncthreads();         // the next chunk's LDS buffer is ready
    } else if constexpr (WPC == 1) {
#pragma unroll
      for (int s = 0; s < kTC; ++s)
        if (s < len && active) Elem<T>::store(yrow + (int64_t)(t0 + s) * ldy, part[s] + skip[s]);
      __syncthreads();         // the next chunk's LDS buffer is ready
    } else {
#pragma unroll
      for (int s = 0; s < kTC; ++s) ys[wave][s][lane] = part[s];
      __syncthreads();
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        const int s = wave + WPC * j;
        if (s < len) {
          float yv = skip[j];
#pragma unroll
          for (int w = 0; w < WPC; ++w) yv += ys[w][s][lane];
          if (active) Elem<T>::store(yrow + (int64_t)(t0 + s) * ldy, yv);
        }
      }
      __syncthreads();         // ys is rewritten by the next chunk
    }
#pragma unroll
    for (int j = 0; j < SPW; ++j) skip[j] = skip_next[j];
    buf ^= 1;
  }
  if constexpr (kSummary) {
    const int64_t ch = ((int64_t)seg * nb + b) * E + c;
    if (active) {
#pragma unroll
      for (int n = 0; n < NS; ++n) seg_h[ch * N + n0 + n] = h[n];
    }
    ys[WPC > 1 ? wave : 0][0][lane] = dsum;   // the waves' step sums, added in wave order
    __syncthreads();
    if (wave == 0) {
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < WPC; ++w) tot += ys[w][0][lane];
      if (active) seg_d[ch] = tot;
    }
  } else if (active && h_out && seg == (int)gridDim.z - 1) {
    float* ho = h_out + ((int64_t)b * E + c) * N + n0;
#pragma unroll
    for (int n = 0; n < NS; ++n) ho[n] = h[n];
  }
}

// Decode: one token per sequence.  N/4 consecutive lanes share a channel, each
// owning 4 states of two sequences (two 16-byte state loads in flight, then the two updates
// and stores); y is reduced across the lanes of a channel.
// grid (ceil(E * N/4 / 256), ceil(B / 2)): no division by a runtime size in the index math.
// kVec: the lane's 4 B and 4 C values come as two vector loads (the dispatcher
// checks their alignment) instead of eight scalar ones.
template <typename T> struct Four;
template <> struct Four<float> {
  __device__ static __forceinline__ void load(const float* p, float (&v)[4]) {
    const float4 w = *reinterpret_cast<const float4*>(p);
    v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
  }
};

template <typename T, int N, bool kVec>
__global__ __launch_bounds__(256) void ssm_step_kernel(StepArgs<T> a) {
  constexpr int LPC = N / 4;
  constexpr int RB = 2;   // sequences per thread: both states' loads are in flight together
  const int i = blockIdx.x * blockDim.x + threadIdx.x;   // lane within the sequence
  const bool active = i < a.E * LPC;
  const int i2 = active ? i : a.E * LPC - 1;
  const int q = i2 % LPC, c = i2 / LPC;
  const int64_t b0 = (int64_t)blockIdx.y * RB;
  // the second sequence of the last block row may not exist: it then repeats the first, unstored
  const bool has[RB] = {true, b0 + 1 < a.B};
  int64_t bs[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) bs[r] = has[r] ? b0 + r : b0;
  // The state is read and written once per step with non-temporal hints: written normally, its
  // 26 MB per 1.5B layer and 128 sequences would sit dirty in the 256 MB MALL and be written back
  // to HBM while the next kernels stream their K/V caches (the ring-decode pair step: 1.20 ->
  // 1.245 M tokens/s per layer, the producer's attention 45.8 -> 40.4 us in the step).
  f32x4_t hv[RB];
  float uv[RB], dv[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    hv[r] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(a.h + (bs[r] * a.E + c) * N + 4 * q));
    uv[r] = Elem<T>::load(a.u + bs[r] * a.ld + c);
    dv[r] = Elem<T>::load(a.dt + bs[r] * a.ld + c);
  }
  const float4 a2 = *reinterpret_cast<const float4*>(a.A2 + (int64_t)c * N + 4 * q);
  const float a2s[4] = {a2.x, a2.y, a2.z, a2.w};
  const float bias = a.dt_bias[c], dskip = a.D[c];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const float* row = a.bc + bs[r] * a.ld_bc;
    const float delta = softplus_f(dv[r] + bias);
    const float du = delta * uv[r];
    float bn[4], cn[4];
    if constexpr (kVec) {
      Four<float>::load(row + 4 * q, bn);
      Four<float>::load(row + N + 4 * q, cn);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bn[j] = row[4 * q + j];
        cn[j] = row[N + 4 * q + j];
      }
    }
    float hs[4] = {hv[r][0], hv[r][1], hv[r][2], hv[r][3]};
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      hs[j] = fmaf(fast_exp2(delta * a2s[j]), hs[j], du * bn[j]);
      part = fmaf(cn[j], hs[j], part);
    }
#pragma unroll
    for (int off = 1; off < LPC; off <<= 1) part += __shfl_xor(part, off);
    if (active && has[r]) {
      __builtin_nontemporal_store(f32x4_t{hs[0], hs[1], hs[2], hs[3]},
                                  reinterpret_cast<f32x4_t*>(a.h + (bs[r] * a.E + c) * N + 4 * q));
      if (q == 0) Elem<T>::store(a.y + bs[r] * a.ldy + c, part + dskip * uv[r]);
    }
  }
}

// States per wave: the fewest waves per channel group (largest NS, least
// per-step overhead) that still gives ~HYMBA_SCAN_WAVES waves over the 1024 SIMDs.
#ifndef HYMBA_SCAN_WAVES
#define HYMBA_SCAN_WAVES 3072
#endif
#ifndef HYMBA_SCAN_MAX_SEGMENTS
#define HYMBA_SCAN_MAX_SEGMENTS 8
#endif
constexpr int kMinSegLen = 256;   // shorter segments spend more on the summary pass than they gain

inline int scan_states_per_wave(int B, int E, int N) {
  const int64_t groups = (int64_t)B * ceil_div(E, 64);
  int ns = N < 8 ? N : 8;   // one wave holding all 16 states runs out of registers
  while (ns > 2 && groups * (N / ns) < HYMBA_SCAN_WAVES) ns >>= 1;
  return ns;
}

struct ScanPlan { int ns; int nseg; int seg_len; };

// One pass when the channel groups give ~HYMBA_SCAN_WAVES waves at 4 states per wave (or the
// sequences are short); otherwise 4 states per wave and enough time segments to get there.
ScanPlan scan_plan(int B, int T, int E, int N) {
  ScanPlan p{scan_states_per_wave(B, E, N), 1, T};
  const int64_t waves = (int64_t)B * ceil_div(E, 64) * (N / 4);
  int64_t nseg = std::min<int64_t>(HYMBA_SCAN_MAX_SEGMENTS, ceil_div(HYMBA_SCAN_WAVES, waves));
  nseg = std::min<int64_t>(nseg, T / kMinSegLen);
  if (nseg >= 2) {
    p.ns = 4;
    p.seg_len = static_cast<int>(ceil_div(ceil_div(T, nseg), kTC) * kTC);
    p.nseg = static_cast<int>(ceil_div(T, p.seg_len));
  }
  return p;
}

template <typename T, int N, int NS>
void scan_launch(const ScanArgs<T>& a, const ScanPlan& p, hipStream_t s) {
  dim3 block(64 * (N / NS));
  float* seg_h = a.seg;
  float* seg_d = a.seg + (int64_t)(p.nseg - 1) * a.B * a.E * N;
  if (p.nseg > 1) {
    dim3 g1(static_cast<unsigned>(ceil_div(a.E, 64)), a.B, p.nseg - 1);
    hipLaunchKernelGGL((selective_scan_kernel<T, N, NS, true>), g1, block, 0, s, a.u, a.dt, a.ld, a.bc, a.ld_bc,
                       a.A2, a.D, a.dt_bias, a.h0, a.h0_bstride, a.y, a.ldy, a.h_out, a.T, a.E, p.seg_len, seg_h,
                       seg_d);
  }
  dim3 grid(static_cast<unsigned>(ceil_div(a.E, 64)), a.B, p.nseg);
  hipLaunchKernelGGL((selective_scan_kernel<T, N, NS, false>), grid, block, 0, s, a.u, a.dt, a.ld, a.bc, a.ld_bc,
                     a.A2, a.D, a.dt_bias, a.h0, a.h0_bstride, a.y, a.ldy, a.h_out, a.T, a.E, p.seg_len, seg_h,
                     seg_d);
}

template <typename T>
hipError_t scan_dispatch(const ScanArgs<T>& a, hipStream_t s) {
  if (a.B < 1 || a.T < 1 || a.B > 65535) return hipErrorInvalidValue;
  ScanPlan p = scan_plan(a.B, a.T, a.E, a.N);
  if (p.nseg > 1 && (!a.seg || a.seg_bytes < scan_segment_bytes(a.B, a.T, a.E, a.N)))
    p = ScanPlan{scan_states_per_wave(a.B, a.E, a.N), 1, a.T};   // no room for the summaries: one pass
  if (a.N == 8) {
    if (p.ns == 8) scan_launch<T, 8, 8>(a, p, s);
    else if (p.ns == 4) scan_launch<T, 8, 4>(a, p, s);
    else scan_launch<T, 8, 2>(a, p, s);
  } else if (a.N == 16) {
    if (p.ns == 8) scan_launch<T, 16, 8>(a, p, s);
    else if (p.ns == 4) scan_launch<T, 16, 4>(a, p, s);
    else scan_launch<T, 16, 2>(a, p, s);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t step_dispatch(const StepArgs<T>& a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  if (a.B > 65535 || (int64_t)a.E * (a.N / 4) >= INT32_MAX) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(ceil_div((int64_t)a.E * (a.N / 4), 256)), static_cast<unsigned>(ceil_div(a.B, 2))),
      block(256);
  // B/C as vector loads when every row's 4-state groups are aligned to the vector size
  const bool vec = reinterpret_cast<uintptr_t>(a.bc) % 16 == 0 && a.ld_bc % 4 == 0 && a.N % 4 == 0;
  switch (a.N * 2 + (vec ? 1 : 0)) {
    case 16: hipLaunchKernelGGL((ssm_step_kernel<T, 8, false>), grid, block, 0, s, a); break;
    case 17: hipLaunchKernelGGL((ssm_step_kernel<T, 8, true>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((ssm_step_kernel<T, 16, false>), grid, block, 0, s, a); break;
    case 33: hipLaunchKernelGGL((ssm_step_kernel<T, 16, true>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

size_t scan_segment_bytes(int B, int T, int E, int N) {
  const ScanPlan p = scan_plan(B, T, E, N);
  return p.nseg > 1 ? (size_t)(p.nseg - 1) * B * E * (N + 1) * sizeof(float) : 0;
}

hipError_t launch_selective_scan(const ScanArgs<float>& a, hipStream_t s) { return scan_dispatch(a, s); }
hipError_t launch_selective_scan(const ScanArgs<half_t>& a, hipStream_t s) { return scan_dispatch(a, s); }
hipError_t launch_ssm_step(const StepArgs<float>& a, hipStream_t s) { return step_dispatch(a, s); }
hipError_t launch_ssm_step(const StepArgs<half_t>& a, hipStream_t s) { return step_dispatch(a, s); }

}  // namespace hymba
