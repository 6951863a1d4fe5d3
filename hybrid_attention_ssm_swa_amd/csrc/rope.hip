// Rotary position encoding of the q and k columns of the shared projection,
// in place.
//
// The Hymba summary (greeksharifa.github.io) section 2.5 "Hymba Model Family"
// says the 8K-context stage changes the base of the rotary positional
// encoding, and the Griffin summary (hyeon-jae.tistory.com) section 2.3 uses
// RoPE as its relative position encoding; neither prints the rotation, so the
// RoFormer definition is used: in every head vector the consecutive pair
// (x[2i], x[2i+1]) turns by the angle pos * base^(-2i/hd).  Meta rows sit at
// positions 0..M-1 and real token t at M + t; K is rotated before it is cached
// or handed to a consumer.
//
// One thread per (row, 16-byte chunk of a head vector): it forms the chunk's
// 4 (16-bit types) or 2 (fp32) rotations once -- the angle formed and reduced
// modulo 2 pi in fp64 from a per-pair frequency table computed on the host,
// so positions in the millions keep full fp32 accuracy in sin/cos -- and
// applies them to that chunk of every q and k head of the row (all heads share
// the position).  Consecutive threads cover consecutive chunks of a row, so
// each head access is a contiguous run.
#include "common.h"
#include "kernels.h"

namespace hymba {

namespace {

template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(RopeArgs<T> a) {
  constexpr int V = Vec16<T>::n;                 // elements per 16-byte chunk
  const int cph = a.head_dim / V;                // chunks per head vector
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= a.rows * cph) return;
  const int ch = static_cast<int>(i % cph);
  const int64_t row = i / cph;
  const int64_t pos = a.first + (a.pos ? a.pos[row] : row % a.T);
  constexpr double kTwoPi = 6.283185307179586476925286766559;
  float cs[V / 2], sn[V / 2];
#pragma unroll
  for (int j = 0; j < V / 2; ++j) {
    const double ang = static_cast<double>(pos) * a.theta[ch * (V / 2) + j];
    sincosf(static_cast<float>(ang - kTwoPi * floor(ang / kTwoPi)), &sn[j], &cs[j]);
  }
  T* prow = a.p + row * a.ld + ch * V;
  const int heads = a.n_q_heads + a.n_k_heads;
  for (int hv = 0; hv < heads; ++hv) {
    T* p = prow + (hv < a.n_q_heads ? (int64_t)hv * a.head_dim
                                    : a.k_off + (int64_t)(hv - a.n_q_heads) * a.head_dim);
    float x[V];
    Vec16<T>::load(p, x);
#pragma unroll
    for (int j = 0; j < V / 2; ++j) {
      const float x0 = x[2 * j], x1 = x[2 * j + 1];
      x[2 * j] = x0 * cs[j] - x1 * sn[j];
      x[2 * j + 1] = x0 * sn[j] + x1 * cs[j];
    }
    Vec16<T>::store(p, x);
  }
}

template <typename T>
hipError_t rope_dispatch(const RopeArgs<T>& a, hipStream_t s) {
  constexpr int V = Vec16<T>::n;
  if (a.head_dim % V || a.head_dim / 2 > kRopeMaxPairs) return hipErrorInvalidValue;
  const int64_t total = a.rows * (a.head_dim / V);
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL((rope_kernel<T>), dim3(static_cast<unsigned>(ceil_div(total, 256))), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope(const RopeArgs<float>& a, hipStream_t s) { return rope_dispatch(a, s); }
hipError_t launch_rope(const RopeArgs<half_t>& a, hipStream_t s) { return rope_dispatch(a, s); }

}  // namespace hymba
