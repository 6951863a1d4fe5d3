// Kernels of the Griffin recurrent block (Griffin summary, hyeon-jae.tistory.com,
// sections 2.3 and 2.4, appendix A): the causal separable Conv1D of width 4 and
// the RG-LRU recurrence merged with the GeLU branch.
//
// The RG-LRU state is one number per channel, so channels alone (B * R) give
// too few independent lanes to fill the chip; time is cut into S segments and
// h_t = a_t h_(t-1) + b_t runs as a chunked scan with carry propagation.
// Pass 1 runs segments 0 .. S-2 from zero and records (sum of log a_t, end
// state); record 0 holds the handed state h0.  Pass 2 folds the records before
// its segment into the start state (h = exp(sum log a) h + h_end), reruns the
// segment and writes y_t = h_t GeLU(v_t).  A segment's decay is kept as a sum
// of logs, so it neither under- nor overflows however long the segment.
// Lane = channel: a wave's loads of one time step cover 64 consecutive
// channels of a row (one 128-byte line for fp16 activations).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace hymba {

namespace {

constexpr int kConvTaps = 4;
constexpr int kStepChunk = 8;   // time steps whose loads are issued together

// thread per (row, 16-byte chunk of R)
template <typename T>
__global__ __launch_bounds__(256) void griffin_conv_kernel(GriffinConvArgs<T> a) {
  constexpr int V = Vec16<T>::n;
  constexpr int H = kConvTaps - 1;
  const int cpr = a.R / V;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)a.B * a.seq * cpr) return;
  const int r0 = static_cast<int>(i % cpr) * V;
  const int64_t row = i / cpr;
  const int t = static_cast<int>(row % a.seq);
  const int64_t b = row / a.seq;
  // input at time tt (>= -H) of this sequence and chunk
  auto input = [&](int tt, float (&u)[V]) {
    if (tt >= 0) {
      Vec16<T>::load(a.u + (b * a.seq + tt) * a.ld_u + r0, u);
    } else if (a.hist) {
      Vec16<float>::load(a.hist + (b * H + (H + tt)) * a.R + r0, *reinterpret_cast<float(*)[4]>(&u[0]));
      if constexpr (V == 8)
        Vec16<float>::load(a.hist + (b * H + (H + tt)) * a.R + r0 + 4, *reinterpret_cast<float(*)[4]>(&u[4]));
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e) u[e] = 0.f;
    }
  };
  float acc[V] = {};
#pragma unroll
  for (int k = 0; k < kConvTaps; ++k) {
    float u[V];
    input(t - k, u);
    float w[V];
    Vec16<float>::load(a.w + k * a.R + r0, *reinterpret_cast<float(*)[4]>(&w[0]));
    if constexpr (V == 8) Vec16<float>::load(a.w + k * a.R + r0 + 4, *reinterpret_cast<float(*)[4]>(&w[4]));
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] = fmaf(w[e], u[e], acc[e]);
  }
  Vec16<T>::store(a.xc + row * a.ld_xc + r0, acc);
  if (a.state_out && t == a.seq - 1) {
    // the last H inputs, oldest first; all are read before any is written (state_out may alias
    // hist only when seq == 1, and then only this thread touches this chunk of the state)
    float sv[H][V];
#pragma unroll
    for (int j = 0; j < H; ++j) input(a.seq - H + j, sv[j]);
#pragma unroll
    for (int j = 0; j < H; ++j) {
      float* sp = a.state_out + (b * H + j) * a.R + r0;
      Vec16<float>::store(sp, *reinterpret_cast<const float(*)[4]>(&sv[j][0]));
      if constexpr (V == 8) Vec16<float>::store(sp + 4, *reinterpret_cast<const float(*)[4]>(&sv[j][4]));
    }
  }
}

__device__ __forceinline__ float sigmoid_f(float x) { return 1.f / (1.f + __expf(-x)); }

// c softplus(-Lambda) = -c log sigmoid(Lambda)
__device__ __forceinline__ float decay_scale(float lam, float c) {
  return c * (fmaxf(-lam, 0.f) + log1pf(__expf(-fabsf(lam))));
}

// One segment [t0, t1) of channel r of sequence b: advances h (and the log-decay sum) and, with
// kOut, writes y_t = h_t GeLU(v_t).
template <typename T, bool kOut>
__device__ __forceinline__ void run_segment(const RglruArgs<T>& a, int64_t row0, int t0, int t1, int r,
                                            float c_sp, float& h, float& lsum) {
  const T* __restrict__ g = a.g + row0 * a.ld_g + r;
  const T* __restrict__ xc = a.xc + row0 * a.ld_xc + r;
  const T* __restrict__ v = a.v + row0 * a.ld_v + r;
  T* __restrict__ y = a.y + row0 * a.ldy + r;
  auto step = [&](float rho, float iota, float x, float vv, int64_t t) {
    const float la = -c_sp * sigmoid_f(rho);                 // log a_t = c r_t log sigmoid(Lambda)
    const float bt = sqrtf(-expm1f(2.f * la)) * sigmoid_f(iota) * x;
    h = fmaf(__expf(la), h, bt);
    if constexpr (kOut) {
      Elem<T>::store(y + t * a.ldy, h * (0.5f * vv * (1.f + erff(vv * 0.70710678118654752f))));
    } else {
      lsum += la;
    }
  };
  int t = t0;
  for (; t + kStepChunk <= t1; t += kStepChunk) {
    float rho[kStepChunk], iota[kStepChunk], x[kStepChunk], vv[kStepChunk];
#pragma unroll
    for (int j = 0; j < kStepChunk; ++j) {
      rho[j] = Elem<T>::load(g + (t + j) * a.ld_g);
      iota[j] = Elem<T>::load(g + (t + j) * a.ld_g + a.R);
      x[j] = Elem<T>::load(xc + (t + j) * a.ld_xc);
      if constexpr (kOut) vv[j] = Elem<T>::load(v + (t + j) * a.ld_v);
      else vv[j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < kStepChunk; ++j) step(rho[j], iota[j], x[j], vv[j], t + j);
  }
  for (; t < t1; ++t)
    step(Elem<T>::load(g + (int64_t)t * a.ld_g), Elem<T>::load(g + (int64_t)t * a.ld_g + a.R),
         Elem<T>::load(xc + (int64_t)t * a.ld_xc), kOut ? Elem<T>::load(v + (int64_t)t * a.ld_v) : 0.f, t);
}

// grid (ceil(R / 64), S - 1, B): segments 0 .. S-2; record seg + 1; segment 0 also writes record 0
template <typename T>
__global__ __launch_bounds__(64) void rglru_summary_kernel(RglruArgs<T> a) {
  const int r = blockIdx.x * 64 + threadIdx.x;
  const int seg = blockIdx.y, b = blockIdx.z;
  if (r >= a.R) return;
  float2* rec = a.summ + (int64_t)b * (a.S + 1) * a.R + r;
  if (seg == 0) rec[0] = make_float2(0.f, a.h0 ? a.h0[(int64_t)b * a.R + r] : 0.f);
  const int t0 = seg * a.L, t1 = min(a.seq, t0 + a.L);
  float h = 0.f, lsum = 0.f;
  run_segment<T, false>(a, (int64_t)b * a.seq, t0, t1, r, decay_scale(a.lam[r], a.c), h, lsum);
  rec[(int64_t)(seg + 1) * a.R] = make_float2(lsum, h);
}

// grid (ceil(R / 64), S, B)
template <typename T>
__global__ __launch_bounds__(64) void rglru_output_kernel(RglruArgs<T> a) {
  const int r = blockIdx.x * 64 + threadIdx.x;
  const int seg = blockIdx.y, b = blockIdx.z;
  if (r >= a.R) return;
  float h;
  if (a.S == 1) {
    h = a.h0 ? a.h0[(int64_t)b * a.R + r] : 0.f;
  } else {   // h0 comes through record 0, so h_out may alias h0
    const float2* rec = a.summ + (int64_t)b * (a.S + 1) * a.R + r;
    h = 0.f;
    for (int s = 0; s <= seg; ++s) {
      const float2 q = rec[(int64_t)s * a.R];
      h = fmaf(__expf(q.x), h, q.y);
    }
  }
  const int t0 = seg * a.L, t1 = min(a.seq, t0 + a.L);
  float unused = 0.f;
  run_segment<T, true>(a, (int64_t)b * a.seq, t0, t1, r, decay_scale(a.lam[r], a.c), h, unused);
  if (a.h_out && seg == a.S - 1) a.h_out[(int64_t)b * a.R + r] = h;
}

template <typename T>
hipError_t conv_dispatch(const GriffinConvArgs<T>& a, hipStream_t s) {
  constexpr int V = Vec16<T>::n;
  if (a.R % V) return hipErrorInvalidValue;
  const int64_t n = (int64_t)a.B * a.seq * (a.R / V);
  if (n <= 0) return hipSuccess;
  if (ceil_div(n, 256) > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((griffin_conv_kernel<T>), dim3(static_cast<unsigned>(ceil_div(n, 256))), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t rglru_dispatch(const RglruArgs<T>& a, hipStream_t s) {
  if (a.B <= 0 || a.seq <= 0) return hipSuccess;
  if (a.S < 1 || a.L < 1 || (int64_t)(a.S - 1) * a.L >= a.seq || (int64_t)a.S * a.L < a.seq)
    return hipErrorInvalidValue;   // every segment non-empty, together covering the sequence
  const unsigned gx = static_cast<unsigned>(ceil_div(a.R, 64));
  if (a.S > 1) {
    hipLaunchKernelGGL((rglru_summary_kernel<T>), dim3(gx, a.S - 1, a.B), dim3(64), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((rglru_output_kernel<T>), dim3(gx, a.S, a.B), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

// Segments of a B x T x R recurrence: about 8 waves per SIMD of the chip, segments of at least
// 64 steps; every segment non-empty.
void rglru_plan(int B, int T, int R, int* S, int* L) {
  int64_t s = 1;
  if (T > 0 && B > 0) {
    const int64_t waves_per_seg = (int64_t)B * ceil_div(R, 64);
    s = std::max<int64_t>(1, std::min<int64_t>(ceil_div(8192, waves_per_seg), T / 64));
  }
  const int64_t l = std::max<int64_t>(1, ceil_div(T, s));
  *L = static_cast<int>(l);
  *S = static_cast<int>(std::max<int64_t>(1, ceil_div(T, l)));
}

hipError_t launch_griffin_conv(const GriffinConvArgs<float>& a, hipStream_t s) { return conv_dispatch(a, s); }
hipError_t launch_griffin_conv(const GriffinConvArgs<half_t>& a, hipStream_t s) { return conv_dispatch(a, s); }
hipError_t launch_rglru(const RglruArgs<float>& a, hipStream_t s) { return rglru_dispatch(a, s); }
hipError_t launch_rglru(const RglruArgs<half_t>& a, hipStream_t s) { return rglru_dispatch(a, s); }

}  // namespace hymba
