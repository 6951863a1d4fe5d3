// Fused epilogue of the hybrid-head mixer (Eq. 3 before the output projection):
//   g = y * SiLU(z)                         (SSM output gate)
//   F = beta1 * Ao / sqrt(mean(Ao^2) + eps) + beta2 * g / sqrt(mean(g^2) + eps)
// Hymba summary (greeksharifa.github.io) section 2.1: the shared projection
// also yields the output gate that scales the SSM contribution; both branch
// outputs are normalised and scaled by learnable per-channel vectors because
// the SSM output is consistently larger, then summed.
//
// One wave per token row; each lane keeps up to MAXC 16-byte chunks of Ao and
// g in registers between the reduction and the write, so every input byte is
// read from HBM once.  Rows wider than 64 * MAXC chunks re-read the tail.
#include "common.h"
#include "kernels.h"

namespace hymba {

namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

template <typename T, int MAXC>
__global__ __launch_bounds__(256) void epilogue_kernel(EpiArgs<T> a) {
  constexpr int V = Vec16<T>::n;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= a.rows) return;   // whole wave leaves; no workgroup barrier below
  const T* ao = a.ao + row * a.ld_ao;
  const T* yy = a.y + row * a.ld_y;
  const T* zz = a.z + row * a.ld_z;
  T* ff = a.f + row * a.ld_f;
  const int nch = a.E / V;
  float xa[MAXC][V], xg[MAXC][V];
  float ss1 = 0.f, ss2 = 0.f;
#pragma unroll
  for (int k = 0; k < MAXC; ++k) {
    const int ch = lane + 64 * k;
    if (ch < nch) {
      float yv[V], zv[V];
      Vec16<T>::load(ao + ch * V, xa[k]);
      Vec16<T>::load(yy + ch * V, yv);
      Vec16<T>::load(zz + ch * V, zv);
#pragma unroll
      for (int j = 0; j < V; ++j) {
        xg[k][j] = yv[j] * silu_f(zv[j]);
        ss1 = fmaf(xa[k][j], xa[k][j], ss1);
        ss2 = fmaf(xg[k][j], xg[k][j], ss2);
      }
    }
  }
  for (int ch = lane + 64 * MAXC; ch < nch; ch += 64) {
    float av[V], yv[V], zv[V];
    Vec16<T>::load(ao + ch * V, av);
    Vec16<T>::load(yy + ch * V, yv);
    Vec16<T>::load(zz + ch * V, zv);
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const float gv = yv[j] * silu_f(zv[j]);
      ss1 = fmaf(av[j], av[j], ss1);
      ss2 = fmaf(gv, gv, ss2);
    }
  }
  ss1 = wave_sum(ss1);
  ss2 = wave_sum(ss2);
  const float inv_e = 1.f / static_cast<float>(a.E);
  const float r1 = 1.f / sqrtf(ss1 * inv_e + a.eps);
  const float r2 = 1.f / sqrtf(ss2 * inv_e + a.eps);
#pragma unroll
  for (int k = 0; k < MAXC; ++k) {
    const int ch = lane + 64 * k;
    if (ch < nch) {
      float out[V];
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const int e = ch * V + j;
        out[j] = fmaf(a.beta1[e] * r1, xa[k][j], a.beta2[e] * r2 * xg[k][j]);
      }
      Vec16<T>::store(ff + ch * V, out);
    }
  }
  for (int ch = lane + 64 * MAXC; ch < nch; ch += 64) {
    float av[V], yv[V], zv[V], out[V];
    Vec16<T>::load(ao + ch * V, av);
    Vec16<T>::load(yy + ch * V, yv);
    Vec16<T>::load(zz + ch * V, zv);
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int e = ch * V + j;
      out[j] = fmaf(a.beta1[e] * r1, av[j], a.beta2[e] * r2 * (yv[j] * silu_f(zv[j])));
    }
    Vec16<T>::store(ff + ch * V, out);
  }
}

template <typename T>
hipError_t epi_dispatch(const EpiArgs<T>& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>(ceil_div(a.rows, 4))), block(256);
  hipLaunchKernelGGL((epilogue_kernel<T, 8>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_epilogue(const EpiArgs<float>& a, hipStream_t s) { return epi_dispatch(a, s); }
hipError_t launch_epilogue(const EpiArgs<half_t>& a, hipStream_t s) { return epi_dispatch(a, s); }

}  // namespace hymba
