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
#include <algorithm>
#include <type_traits>

#include "attn_tile.h"
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
constexpr int kDecPasses = 8;   // keys per thread and load round

// Sum over the LPK lanes of one key row (aligned groups of LPK <= 16 lanes):
// quad swaps, then the half-row and row mirrors pair the partial sums of
// neighbouring groups (all DPP, no LDS).
template <int LPK>
__device__ __forceinline__ float row_group_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  if (LPK > 2)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  if (LPK > 4)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  if (LPK > 8)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
  return v;
}

// (m, l, acc) of two partial softmax sums over disjoint key sets, merged into the first.
template <int EPC>
__device__ __forceinline__ void merge_partial(float& m, float& l, float (&acc)[EPC], float m2, float l2,
                                              const float (&acc2)[EPC]) {
  const float mm = fmaxf(m, m2);
  const float f1 = fast_exp2(m - mm), f2 = fast_exp2(m2 - mm);
  l = l * f1 + l2 * f2;
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = acc[e] * f1 + acc2[e] * f2;
  m = mm;
}

// grid (splits, Hkv, B), 256 threads.  A split covers a contiguous run of the
// sequence's visible keys (meta keys, then the ring slots of real indices
// lo..p).  LPK lanes share one key row (16 bytes each), so the workgroup
// covers 256 / LPK keys per pass; passes go in rounds of kDecPasses whose K
// and V loads are all issued first, then every thread runs an online softmax
// (running max, sum, P.V over its 16 bytes of dims) for each of the G query
// heads of the KV group.  The partials
// of the key slots meet through lane shuffles, then across the four waves in
// LDS; the split's (acc, max, sum) per head go to `part` for the combine.
template <typename T, int G, int HD>
__global__ __launch_bounds__(kThreads) void decode_attn_kernel(DecAttnArgs<T> a) {
  constexpr int EPC = 16 / static_cast<int>(sizeof(T));   // elements per 16-byte chunk
  constexpr int LPK = HD / EPC;                             // lanes per key row
  constexpr int KPP = kThreads / LPK;                       // keys per pass
  static_assert(LPK >= 2 && LPK <= 16, "key row must span 2..16 lanes");
  __shared__ float red[kThreads / 64][G][HD + 2];
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid % LPK, slot = tid / LPK;
  const int C = a.cache_len;
  const int64_t p = a.pos[b];
  const int64_t weff = a.window > 0 ? a.window : C;
  const int64_t lo = p - weff + 1 > 0 ? p - weff + 1 : 0;
  const int nkeys = a.n_meta + static_cast<int>(p - lo + 1 > 0 ? p - lo + 1 : 0);
  const int per = static_cast<int>(ceil_div(nkeys, a.splits));
  const int k0 = split * per;
  const int k1 = min(nkeys, k0 + per);

  float qv[G][EPC];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    Vec16<T>::load(a.q + (int64_t)b * a.ld_q + (g * G + hh) * HD + c * EPC, qv[hh]);
#pragma unroll
    for (int e = 0; e < EPC; ++e) qv[hh][e] *= a.scale_log2;
  }
  float m[G], l[G], acc[G][EPC];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = -1e30f;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[hh][e] = 0.f;
  }

  const int64_t kvoff = ((int64_t)b * a.n_kv_heads + g) * C * HD + c * EPC;
  const int64_t moff = (int64_t)g * HD + c * EPC;
  // keys go in rounds of kDecPasses passes: every key of a round is loaded before any is used, so
  // a workgroup keeps a round of its split's K and V in flight; ring slots are tracked
  // incrementally from one 64-bit remainder
  int kk = k0 + slot;
  int64_t rs = kk >= a.n_meta ? (lo + (kk - a.n_meta)) % C : 0;
  const int step_mod = KPP % C;
  while (kk < k1) {   // uniform over the LPK lanes of a key row (they share kk)
    uint4 kr[kDecPasses], vr[kDecPasses];
    const int first = kk;
#pragma unroll
    for (int i = 0; i < kDecPasses; ++i) {
      if (kk < k1) {
        if (kk < a.n_meta) {
          const int64_t o = (int64_t)kk * a.ld_meta + moff;
          kr[i] = *reinterpret_cast<const uint4*>(a.k_meta + o);
          vr[i] = *reinterpret_cast<const uint4*>(a.v_meta + o);
        } else {
          const int64_t o = kvoff + rs * HD;
          kr[i] = *reinterpret_cast<const uint4*>(a.k_cache + o);
          vr[i] = *reinterpret_cast<const uint4*>(a.v_cache + o);
        }
      }
      const int next = kk + KPP;
      if (next >= a.n_meta) {
        if (kk >= a.n_meta) {
          rs += step_mod;
          if (rs >= C) rs -= C;
        } else {
          rs = (lo + (next - a.n_meta)) % C;
        }
      }
      kk = next;
    }
#pragma unroll
    for (int i = 0; i < kDecPasses; ++i) {
      if (first + i * KPP >= k1) break;
      float kf[EPC], vf[EPC];
      Vec16<T>::load(reinterpret_cast<const T*>(&kr[i]), kf);
      Vec16<T>::load(reinterpret_cast<const T*>(&vr[i]), vf);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float sdot = 0.f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) sdot = fmaf(qv[hh][e], kf[e], sdot);
        const float sc = row_group_sum<LPK>(sdot);
        if (sc > m[hh]) {   // the running max moves: rescale this lane's sums
          const float al = fast_exp2(m[hh] - sc);
          m[hh] = sc;
          l[hh] *= al;
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[hh][e] *= al;
        }
        const float pr = fast_exp2(sc - m[hh]);
        l[hh] += pr;
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[hh][e] = fmaf(pr, vf[e], acc[hh][e]);
      }
    }
  }

  // merge the key slots of a wave (lanes c, c + LPK, ... ), then the four waves
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float acc2[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc2[e] = __shfl_xor(acc[hh][e], off);
      const float m2 = __shfl_xor(m[hh], off), l2 = __shfl_xor(l[hh], off);
      merge_partial<EPC>(m[hh], l[hh], acc[hh], m2, l2, acc2);
    }
  }
  if (lane < LPK) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) red[wave][hh][c * EPC + e] = acc[hh][e];
      if (c == 0) {
        red[wave][hh][HD] = m[hh];
        red[wave][hh][HD + 1] = l[hh];
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < G * HD; i += kThreads) {
    const int hh = i / HD, d = i % HD;
    float mm = red[0][hh][HD];
    for (int w = 1; w < kThreads / 64; ++w) mm = fmaxf(mm, red[w][hh][HD]);
    float num = 0.f, den = 0.f;
    for (int w = 0; w < kThreads / 64; ++w) {
      const float f = fast_exp2(red[w][hh][HD] - mm);
      num = fmaf(f, red[w][hh][d], num);
      den = fmaf(f, red[w][hh][HD + 1], den);
    }
    float* out = a.part + (((int64_t)b * a.n_heads + g * G + hh) * a.splits + split) * (HD + 2);
    out[d] = num;
    if (d == 0) {
      out[HD] = mm;
      out[HD + 1] = den;
    }
  }
}

// MFMA decode attention (fp16 K/V, head dim 64): one wave per (split, KV head, sequence).  The
// G query heads of the KV group are the query columns of the prefill kernel's tile step
// (v_mfma_f32_32x32x16_f16, S^T = K Q^T; columns G..31 carry zero queries and are dropped).  The
// wave walks its split's keys in 64-key tiles: the next tile's K rows and V blocks are loaded
// into registers while the current one, staged in LDS (K rows straight, V transposed), goes
// through the online softmax.  The split's (acc, max, sum) per head go to `part` as in the VALU
// kernel, and the same combine kernel merges the splits.
template <int G>
__global__ __launch_bounds__(64) void decode_attn_mfma_kernel(DecAttnArgs<half_t> a) {
  using namespace attn;
  static_assert(G >= 1 && G <= kQB, "query heads of a KV group must fit one column block");
  __shared__ __align__(16) uint16_t ks[kKT * kKStr];
  __shared__ __align__(16) uint16_t vs[kHd * kVStr];
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x, col = lane & 31, half = lane >> 5;
  const int C = a.cache_len;
  const int64_t p = a.pos[b];
  const int64_t weff = a.window > 0 ? a.window : C;
  const int64_t lo = p - weff + 1 > 0 ? p - weff + 1 : 0;
  const int nkeys = a.n_meta + static_cast<int>(p - lo + 1 > 0 ? p - lo + 1 : 0);
  const int per = static_cast<int>(ceil_div(nkeys, a.splits));
  const int k0 = split * per;
  const int k1 = min(nkeys, k0 + per);
  const int lo_mod = static_cast<int>(lo % C);   // ring slot of the first window key

  // Q^T as the B operand: column col = head g G + col, k-step s = dims [16 s + 8 half, +8)
  Op<half_t>::vec qf[4];
  {
    const half_t* qrow = a.q + (int64_t)b * a.ld_q + (int64_t)(g * G + min(col, G - 1)) * kHd + 8 * half;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      U4 v = *reinterpret_cast<const U4*>(qrow + s4 * 16);
      if (col >= G) v = U4{0u, 0u, 0u, 0u};
      qf[s4] = as_vec<half_t>(v);
    }
  }
  WaveState st;
  st.acc[0] = f32x16_t{};
  st.acc[1] = f32x16_t{};
  st.m = -1e30f;
  st.l = 0.f;

  // key kk of the sequence -> its K (and V) row: a meta row, or ring slot lo + kk - M (mod C)
  const int64_t ring = ((int64_t)b * a.n_kv_heads + g) * C;
  auto row_off = [&](int kk) -> int64_t {
    if (kk < a.n_meta) return -1 - ((int64_t)kk * a.ld_meta + (int64_t)g * kHd);   // negative: meta
    int slot = lo_mod + (kk - a.n_meta);
    if (slot >= C) slot -= C;
    return (ring + slot) * kHd;
  };
  // a lane's 16 loads of the tile starting at key t0 with nvalid keys: items lane and lane + 64
  // of the K chunks (4 rows 16 apart each) and of the V blocks (4 consecutive keys x 8 dims);
  // rows past nvalid read the last valid row (their scores are masked)
  auto fetch = [&](int t0, int nvalid, U4 (&kr)[2][4], U4 (&vr)[2][4]) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int item = lane + 64 * it;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int krow = (item >> 3) + 16 * j, kcol = (item & 7) * 8;
        const int64_t ko = row_off(t0 + min(krow, nvalid - 1));
        kr[it][j] = *reinterpret_cast<const U4*>((ko < 0 ? a.k_meta + (-1 - ko) : a.k_cache + ko) + kcol);
        const int vrow = (item >> 3) * 4 + j, vcol = (item & 7) * 8;
        const int64_t vo = row_off(t0 + min(vrow, nvalid - 1));
        vr[it][j] = *reinterpret_cast<const U4*>((vo < 0 ? a.v_meta + (-1 - vo) : a.v_cache + vo) + vcol);
      }
    }
  };
  U4 kr[2][4], vr[2][4];
  if (k0 < k1) fetch(k0, min(kKT, k1 - k0), kr, vr);
  for (int t0 = k0; t0 < k1; t0 += kKT) {
    const int nvalid = min(kKT, k1 - t0);
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      item_store(kr[it], ks, vs, kVStr, 0, lane + 64 * it);         // K chunks
      item_store(vr[it], ks, vs, kVStr, 0, 128 + lane + 64 * it);   // V blocks, transposed
    }
    __syncthreads();
    if (t0 + kKT < k1) fetch(t0 + kKT, min(kKT, k1 - t0 - kKT), kr, vr);   // next tile in flight
    attend_tile<half_t>(st, qf, ks, vs, kVStr, a.scale_log2, lane, 0, 0, nvalid, -1, 0, nvalid < kKT);
    __syncthreads();
  }

  // this split's partials of heads g G + col (col < G): acc over the lane's 32 dims, max (log2
  // units) and the sum over both halves of the column
  const float ltot = sum_xor32(st.l);
  if (col >= G) return;
  float* out = a.part + (((int64_t)b * a.n_heads + g * G + col) * a.splits + split) * (kHd + 2);
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) out[db * 32 + 8 * (r >> 2) + 4 * half + (r & 3)] = st.acc[db][r];
  if (half == 0) {
    out[kHd] = st.m * a.scale_log2;
    out[kHd + 1] = ltot;
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

template <typename T, int HD>
hipError_t dec_dispatch_hd(const DecAttnArgs<T>& a, hipStream_t s) {
  const dim3 grid(a.splits, a.n_kv_heads, a.B), block(kThreads);
  switch (a.n_heads / a.n_kv_heads) {
    case 1: hipLaunchKernelGGL((decode_attn_kernel<T, 1, HD>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_attn_kernel<T, 2, HD>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((decode_attn_kernel<T, 3, HD>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_attn_kernel<T, 4, HD>), grid, block, 0, s, a); break;
    case 5: hipLaunchKernelGGL((decode_attn_kernel<T, 5, HD>), grid, block, 0, s, a); break;
    case 6: hipLaunchKernelGGL((decode_attn_kernel<T, 6, HD>), grid, block, 0, s, a); break;
    case 7: hipLaunchKernelGGL((decode_attn_kernel<T, 7, HD>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((decode_attn_kernel<T, 8, HD>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t dec_dispatch_mfma(const DecAttnArgs<half_t>& a, hipStream_t s) {
  const dim3 grid(a.splits, a.n_kv_heads, a.B), block(64);
  switch (a.n_heads / a.n_kv_heads) {
    case 1: hipLaunchKernelGGL((decode_attn_mfma_kernel<1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_attn_mfma_kernel<2>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((decode_attn_mfma_kernel<3>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_attn_mfma_kernel<4>), grid, block, 0, s, a); break;
    case 5: hipLaunchKernelGGL((decode_attn_mfma_kernel<5>), grid, block, 0, s, a); break;
    case 6: hipLaunchKernelGGL((decode_attn_mfma_kernel<6>), grid, block, 0, s, a); break;
    case 7: hipLaunchKernelGGL((decode_attn_mfma_kernel<7>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((decode_attn_mfma_kernel<8>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t dec_dispatch(const DecAttnArgs<T>& a, hipStream_t s) {
  hipError_t e;
  if constexpr (std::is_same<T, half_t>::value) {
    if (a.head_dim == 64) {
      e = dec_dispatch_mfma(a, s);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((decode_combine_kernel<T>), dim3(a.B * a.n_heads), dim3(kDecodeMaxHd), 0, s, a);
      return hipGetLastError();
    }
  }
  if (a.head_dim == 64) e = dec_dispatch_hd<T, 64>(a, s);
  else if (a.head_dim == 32) e = dec_dispatch_hd<T, 32>(a, s);
  else return hipErrorInvalidValue;
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T>), dim3(a.B * a.n_heads), dim3(kDecodeMaxHd), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_write(const KvWriteArgs<float>& a, hipStream_t s) { return kv_dispatch(a, s); }
hipError_t launch_kv_write(const KvWriteArgs<half_t>& a, hipStream_t s) { return kv_dispatch(a, s); }
hipError_t launch_decode_attn(const DecAttnArgs<float>& a, hipStream_t s) { return dec_dispatch(a, s); }
hipError_t launch_decode_attn(const DecAttnArgs<half_t>& a, hipStream_t s) { return dec_dispatch(a, s); }

// Splits per (sequence, KV head): enough for ~2048 workgroups (8 per CU), at
// least one load round (256 / lanes per key row * kDecPasses keys) per split
// when the key range allows, never fewer than 64 keys per split, at most
// kDecodeMaxSplits.  Longer splits run several rounds.
int decode_attn_splits(int B, int n_kv_heads, int n_keys_max, int head_dim, int elem_bytes) {
  const int lpk = head_dim * elem_bytes / 16;
  if (lpk < 2 || lpk > 16 || B < 1 || n_kv_heads < 1) return -1;
  const int64_t per_round = (int64_t)(kThreads / lpk) * kDecPasses;
  const int64_t pairs = (int64_t)B * n_kv_heads;
  int64_t s = std::max<int64_t>(ceil_div(n_keys_max, per_round), ceil_div(2048, pairs));
  s = std::min<int64_t>(s, std::max<int64_t>(1, ceil_div(n_keys_max, 64)));
  s = std::min<int64_t>(s, kDecodeMaxSplits);
  return static_cast<int>(std::max<int64_t>(s, 1));
}

}  // namespace hymba
