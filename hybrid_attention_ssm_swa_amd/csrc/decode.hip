// K/V movement and one-token decode attention of the hybrid-head mixer.
//
// Hymba summary (greeksharifa.github.io) section 2.2: most layers attend to a
// window of recent tokens, so the decode cache is a ring of `window` slots
// (real token r lives in slot r mod C), and consecutive layers share one
// cache (the consumer of a pair only reads what its producer wrote);
// section 2.3: the meta-token K/V are input independent, one copy serves the
// whole batch.  Decode is bound by reading the cache (Griffin summary,
// hyeon-jae.tistory.com section 4: decode time is dominated by loading
// parameters and cache).
#include "common.h"
#include "kernels.h"

namespace hymba {

namespace {

template <typename T>
__global__ __launch_bounds__(256) void kv_write_kernel(KvWriteArgs<T> a) {
  constexpr int V = 16 / sizeof(T);
  const int cpr = a.head_dim / V;                       // chunks per head row
  const int64_t per_tok = (int64_t)a.n_kv_heads * cpr;
  const int64_t total = (int64_t)a.B * a.T * per_tok;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t bt = i / per_tok;
  const int rem = static_cast<int>(i % per_tok);
  const int g = rem / cpr, ch = rem % cpr;
  const int t = static_cast<int>(bt % a.T);
  const int64_t b = bt / a.T;
  const int64_t src = bt * a.ld_src + g * a.head_dim + ch * V;
  const uint4 kv = *reinterpret_cast<const uint4*>(a.k_src + src);
  const uint4 vv = *reinterpret_cast<const uint4*>(a.v_src + src);
  if (a.k_full) {
    const int64_t dst = (bt * a.n_kv_heads + g) * a.head_dim + ch * V;
    *reinterpret_cast<uint4*>(a.k_full + dst) = kv;
    *reinterpret_cast<uint4*>(a.v_full + dst) = vv;
  }
  if (a.k_cache) {
    int64_t slot;
    if (a.pos) {
      if (a.pos[b] < 0) return;   // invalid position: write nothing
      slot = a.pos[b] % a.cache_len;
    } else {
      if (t < a.T - a.cache_len) return;
      slot = t % a.cache_len;
    }
    const int64_t dst = ((b * a.n_kv_heads + g) * a.cache_len + slot) * a.head_dim + ch * V;
    *reinterpret_cast<uint4*>(a.k_cache + dst) = kv;
    *reinterpret_cast<uint4*>(a.v_cache + dst) = vv;
  }
}

constexpr int kThreads = 256;
constexpr int kMaxKeysPerSplit = 512;
constexpr int kMaxGroup = 8;

// 8 consecutive elements -> floats
template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]) {
  if constexpr (Vec16<T>::n == 8) {
    Vec16<T>::load(p, v);
  } else {
    float a[4], b[4];
    Vec16<T>::load(p, a);
    Vec16<T>::load(p + 4, b);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
  }
}

// grid (splits, Hkv, B), 256 threads.  Phase 1: one thread per key computes the
// group's scores (q broadcast from LDS).  Phase 2: per-head max / exp / sum.
// Phase 3: threads = (key group, dim pair) accumulate P.V; key groups reduced
// through LDS.  Writes per-split partials (acc, max, sum).
template <typename T>
__global__ __launch_bounds__(kThreads) void decode_attn_kernel(DecAttnArgs<T> a) {
  __shared__ float qs[kMaxGroup][kDecodeMaxHd];
  __shared__ float ps[kMaxGroup][kMaxKeysPerSplit];
  __shared__ float red[kThreads / 64][kMaxGroup][kDecodeMaxHd];
  __shared__ float stat[kMaxGroup][2];
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int G = a.n_heads / a.n_kv_heads;
  const int hd = a.head_dim;
  const int C = a.cache_len;
  const int64_t p = a.pos[b];
  const int64_t weff = a.window > 0 ? a.window : C;
  const int64_t lo = p - weff + 1 > 0 ? p - weff + 1 : 0;
  const int nkeys = a.n_meta + static_cast<int>(p - lo + 1 > 0 ? p - lo + 1 : 0);
  const int per = static_cast<int>(ceil_div(nkeys, a.splits));
  const int k0 = split * per;
  const int k1 = min(nkeys, k0 + per);
  const int nk = max(0, k1 - k0);

  for (int i = tid; i < G * hd; i += kThreads) {
    const int hh = i / hd, d = i % hd;
    qs[hh][d] = Elem<T>::load(a.q + (int64_t)b * a.ld_q + (g * G + hh) * hd + d) * a.scale_log2;
  }
  __syncthreads();

  const T* kc = a.k_cache + ((int64_t)b * a.n_kv_heads + g) * C * hd;
  const T* vc = a.v_cache + ((int64_t)b * a.n_kv_heads + g) * C * hd;
  auto key_ptr = [&](const T* meta, const T* cache, int kk) -> const T* {
    if (kk < a.n_meta) return meta + (int64_t)kk * a.ld_meta + g * hd;
    const int64_t r = lo + (kk - a.n_meta);
    return cache + (r % C) * hd;
  };

  // phase 1: scores (log2 units)
  for (int j = tid; j < nk; j += kThreads) {
    const T* kr = key_ptr(a.k_meta, kc, k0 + j);
    float s[kMaxGroup];
#pragma unroll
    for (int hh = 0; hh < kMaxGroup; ++hh) s[hh] = 0.f;
    for (int d0 = 0; d0 < hd; d0 += 8) {
      float kv[8];
      load8<T>(kr + d0, kv);
#pragma unroll
      for (int hh = 0; hh < kMaxGroup; ++hh) {
        if (hh < G) {
#pragma unroll
          for (int e = 0; e < 8; ++e) s[hh] = fmaf(qs[hh][d0 + e], kv[e], s[hh]);
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < kMaxGroup; ++hh)
      if (hh < G) ps[hh][j] = s[hh];
  }
  __syncthreads();

  // phase 2: per-head max, exp, sum (one wave per head, heads strided by 4)
  const int wave = tid >> 6, lane = tid & 63;
  for (int hh = wave; hh < G; hh += kThreads / 64) {
    float m = -INFINITY;
    for (int j = lane; j < nk; j += 64) m = fmaxf(m, ps[hh][j]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (nk == 0) m = -1e30f;
    float l = 0.f;
    for (int j = lane; j < nk; j += 64) {
      const float e = fast_exp2(ps[hh][j] - m);
      ps[hh][j] = e;
      l += e;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);
    if (lane == 0) { stat[hh][0] = m; stat[hh][1] = l; }
  }
  __syncthreads();

  // phase 3: O = P.V ; thread = (key group kg, dim pair dp)
  const int npairs = hd / 2;
  const int ngroups = kThreads / npairs;
  const int dp = tid % npairs, kg = tid / npairs;
  float acc[kMaxGroup][2];
#pragma unroll
  for (int hh = 0; hh < kMaxGroup; ++hh) { acc[hh][0] = 0.f; acc[hh][1] = 0.f; }
  if (kg < ngroups) {
    for (int j = kg; j < nk; j += ngroups) {
      const T* vr = key_ptr(a.v_meta, vc, k0 + j);
      const float v0 = Elem<T>::load(vr + 2 * dp), v1 = Elem<T>::load(vr + 2 * dp + 1);
#pragma unroll
      for (int hh = 0; hh < kMaxGroup; ++hh) {
        if (hh < G) {
          const float w = ps[hh][j];
          acc[hh][0] = fmaf(w, v0, acc[hh][0]);
          acc[hh][1] = fmaf(w, v1, acc[hh][1]);
        }
      }
    }
  }
  // reduce key groups: first within a wave (groups sharing a wave), then across waves
  const int groups_per_wave = 64 / npairs;   // >= 1 since hd <= 128
#pragma unroll
  for (int hh = 0; hh < kMaxGroup; ++hh) {
    if (hh < G) {
      for (int off = npairs; off < 64; off <<= 1) {
        acc[hh][0] += __shfl_xor(acc[hh][0], off);
        acc[hh][1] += __shfl_xor(acc[hh][1], off);
      }
    }
  }
  (void)groups_per_wave;
  if (lane < npairs) {
#pragma unroll
    for (int hh = 0; hh < kMaxGroup; ++hh)
      if (hh < G) { red[wave][hh][2 * dp] = acc[hh][0]; red[wave][hh][2 * dp + 1] = acc[hh][1]; }
  }
  __syncthreads();
  const int nwaves = kThreads / 64;
  for (int i = tid; i < G * hd; i += kThreads) {
    const int hh = i / hd, d = i % hd;
    float s = 0.f;
    for (int w = 0; w < nwaves; ++w) s += red[w][hh][d];
    const int h = g * G + hh;
    float* out = a.part + (((int64_t)b * a.n_heads + h) * a.splits + split) * (hd + 2);
    out[d] = s;
    if (d == 0) { out[hd] = stat[hh][0]; out[hd + 1] = stat[hh][1]; }
  }
}

// grid B * H, block hd threads: merge the split partials of one (sequence, head).
template <typename T>
__global__ __launch_bounds__(kDecodeMaxHd) void decode_combine_kernel(DecAttnArgs<T> a) {
  const int bh = blockIdx.x;
  const int d = threadIdx.x;
  const int hd = a.head_dim;
  if (d >= hd) return;
  const float* part = a.part + (int64_t)bh * a.splits * (hd + 2);
  float m = -INFINITY;
  for (int s = 0; s < a.splits; ++s) m = fmaxf(m, part[s * (hd + 2) + hd]);
  float num = 0.f, den = 0.f;
  for (int s = 0; s < a.splits; ++s) {
    const float* ps = part + s * (hd + 2);
    const float w = fast_exp2(ps[hd] - m);
    num = fmaf(w, ps[d], num);
    den = fmaf(w, ps[hd + 1], den);
  }
  const int b = bh / a.n_heads, h = bh % a.n_heads;
  Elem<T>::store(a.o + (int64_t)b * a.ld_o + h * hd + d, num / den);
}

template <typename T>
hipError_t kv_dispatch(const KvWriteArgs<T>& a, hipStream_t s) {
  constexpr int V = 16 / sizeof(T);
  const int64_t total = (int64_t)a.B * a.T * a.n_kv_heads * (a.head_dim / V);
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL((kv_write_kernel<T>), dim3(static_cast<unsigned>(ceil_div(total, 256))), dim3(256),
                     0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t dec_dispatch(const DecAttnArgs<T>& a, hipStream_t s) {
  hipLaunchKernelGGL((decode_attn_kernel<T>), dim3(a.splits, a.n_kv_heads, a.B), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T>), dim3(a.B * a.n_heads), dim3(kDecodeMaxHd), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_write(const KvWriteArgs<float>& a, hipStream_t s) { return kv_dispatch(a, s); }
hipError_t launch_kv_write(const KvWriteArgs<half_t>& a, hipStream_t s) { return kv_dispatch(a, s); }
hipError_t launch_decode_attn(const DecAttnArgs<float>& a, hipStream_t s) { return dec_dispatch(a, s); }
hipError_t launch_decode_attn(const DecAttnArgs<half_t>& a, hipStream_t s) { return dec_dispatch(a, s); }

// Enough splits that every split holds at most kMaxKeysPerSplit keys and the
// grid has ~2048 workgroups (8 per CU).
int decode_attn_splits(int B, int n_kv_heads, int n_keys_max) {
  int s = static_cast<int>(ceil_div(n_keys_max, kMaxKeysPerSplit));
  if (s < 1) s = 1;
  const int64_t pairs = (int64_t)B * n_kv_heads;
  while (s < kDecodeMaxSplits && pairs * s < 2048 && ceil_div(n_keys_max, s * 2) >= 64) s *= 2;
  return s > kDecodeMaxSplits ? -1 : s;
}

}  // namespace hymba
