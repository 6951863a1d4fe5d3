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
  if (p < 0 && a.flags && split == 0 && g == 0 && tid == 0) a.flags[1] = 1u;   // reported by the layer check
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

// ---- the decode tile step on 16 query columns (v_mfma_f32_16x16x32_f16) ------------------
// A GQA group has at most 8 query heads, so 16 columns waste half as much softmax work as the
// prefill step's 32.  16x16x32 layouts: A lane l = row l%16, k [8(l/16), +8); B lane l =
// column l%16, the same k; C lane l = column l%16, rows 4(l/16) + 0..3.
struct WaveState16 {
  f32x4_t acc[4];   // O^T: dims 16 db + 4 (lane/16) + r of column lane%16
  float m;          // running max (raw score units)
  float l;          // partial sum over this lane's keys
};

__device__ __forceinline__ f32x4_t mfma16(attn::U4 a, attn::U4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0,
                                                0, 0);
}
// x combined with the same register of lane l ^ 16 (v_permlane16_swap with both operands x)
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One 64-key tile for 16 query columns, in two parts.  tile_scores16: S^T = K Q^T in four 16-key
// blocks, with the tile's K rows in registers in the A layout (kr[kb][h]: key 16 kb + lane % 16,
// dims 32 h + 8 (lane / 16) + 0..7), keys from nvalid on masked.  attend_tile16: online softmax
// (lazy rescale as in the prefill step) and O^T += V^T P^T in two 32-key steps, V rows in LDS
// (vs [64][kVStr16]).  The lane's scores s[kb][r] are keys 16 kb + 4 q + r (q = lane/16); as the
// B operand of PV step m they fill k-slots 8 q + j = keys 32 m + 4 q + j (j < 4) and
// 32 m + 16 + 4 q + j - 4 (j >= 4), and the V^T reads follow the same order, so P needs no
// cross-lane movement.
__device__ __forceinline__ void tile_scores16(f32x4_t (&s)[4], const attn::U4 (&qf)[2], const attn::U4 (&kr)[4][2],
                                              int lane, int nvalid) {
  using namespace attn;
  const int q = lane >> 4;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    s[kb] = f32x4_t{};
#pragma unroll
    for (int h = 0; h < 2; ++h) s[kb] = mfma16(kr[kb][h], qf[h], s[kb]);
  }
  if (nvalid < kKT) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (16 * kb + 4 * q + r >= nvalid) s[kb][r] = -INFINITY;
  }
}

__device__ __forceinline__ void attend_tile16(WaveState16& st, f32x4_t (&s)[4], const uint16_t* vs, float sc,
                                              int lane) {
  using namespace attn;
  const int q = lane >> 4;
  float mt = max3f(s[0][0], s[0][1], s[0][2]);
  mt = max3f(mt, s[0][3], s[1][0]);
  mt = max3f(mt, s[1][1], s[1][2]);
  mt = max3f(mt, s[1][3], s[2][0]);
  mt = max3f(mt, s[2][1], s[2][2]);
  mt = max3f(mt, s[2][3], s[3][0]);
  mt = max3f(mt, s[3][1], s[3][2]);
  mt = fmaxf(mt, s[3][3]);
  mt = max_xor32(max_xor16(mt));   // the column's max over its four lanes
  if (__builtin_amdgcn_ballot_w64((mt - st.m) * sc > kLazyLog2) != 0) {
    const float mnew = fmaxf(st.m, mt);
    const float alpha = fast_exp2((st.m - mnew) * sc);
    st.m = mnew;
    st.l *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) st.acc[db][r] *= alpha;
  }
  const float msc = st.m * sc;
  float psum = 0.f;
  U4 pf[2];
#pragma unroll
  for (int m2 = 0; m2 < 2; ++m2) {
    float p[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = fast_exp2(fmaf(s[2 * m2][r], sc, -msc));
      p[4 + r] = fast_exp2(fmaf(s[2 * m2 + 1][r], sc, -msc));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) psum += p[j];
    pf[m2].x = pack_f16x2(p[0], p[1]);
    pf[m2].y = pack_f16x2(p[2], p[3]);
    pf[m2].z = pack_f16x2(p[4], p[5]);
    pf[m2].w = pack_f16x2(p[6], p[7]);
  }
  st.l += psum;
  // A fragment (lane l: dim 16 db + l % 16, keys 32 m + 4 q + 0..3 and 32 m + 16 + 4 q + 0..3) from
  // two transposed reads: lane group q reads rows 32 m + 4 q (+ 16) + (l % 16) / 4, dims
  // 16 db + 4 (l % 4).
  const uint16_t* vlane = vs + (4 * q + ((lane & 15) >> 2)) * kVStr16 + 4 * (lane & 3);
#pragma unroll
  for (int db = 0; db < 4; ++db) {
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2) {
      const uint2 lo = v_tr4(vlane + 32 * m2 * kVStr16 + 16 * db);
      const uint2 hi = v_tr4(vlane + (32 * m2 + 16) * kVStr16 + 16 * db);
      st.acc[db] = mfma16(U4{lo.x, lo.y, hi.x, hi.y}, pf[m2], st.acc[db]);
    }
  }
}

// MFMA decode attention (fp16 K/V, head dim 64): one wave per (split, KV head, sequence).  The
// G query heads of the KV group are the query columns of a 16-column tile step
// (v_mfma_f32_16x16x32_f16, S^T = K Q^T; columns G..15 carry zero queries and are dropped).  The
// wave walks its split's keys in 64-key tiles.  K goes straight from memory into registers in the
// score MFMA's A layout (each lane loads 16 bytes of 8 rows; a load instruction covers 64
// bytes of 16 consecutive rows); V goes through LDS, whose transposed reads give the P.V
// product's A operand.  The next tile's loads are issued once the current tile's scores have
// consumed its K registers, and land during its softmax and P.V.  With only V in LDS (10 KB per
// wave) and one register set per operand, every wave of the ring decode can be resident at once.
// The split's (acc, max, sum) per head go to `part` as in the VALU kernel, and the same combine
// kernel merges the splits.
// 16 bytes of K or V.  NT: with the non-temporal hint, for the cache rows.  A decode step reads each
// cache row once per layer that attends to it (a KV-sharing pair: twice), and 128 sequences' caches
// are 169 MB at the 1.5B shape: left to allocate in the 256 MB MALL they would evict the ~100 MB of
// projection weights that every step re-reads.  Non-temporal cache reads keep the weights resident
// (the ring-decode pair: 1.25 -> 1.32 M tokens/s per layer, the input projection 21 -> 16 us, even
// though the consumer's attention no longer finds its producer's rows in the MALL).  The meta rows,
// shared by every sequence, load normally.
template <bool NT>
__device__ __forceinline__ attn::U4 kv_load(const half_t* p) {
  if constexpr (NT) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return attn::U4{v[0], v[1], v[2], v[3]};
  } else {
    return *reinterpret_cast<const attn::U4*>(p);
  }
}

template <int G>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4))) void decode_attn_mfma_kernel(
    DecAttnArgs<half_t> a) {
  using namespace attn;
  static_assert(G >= 1 && G <= 16, "query heads of a KV group must fit 16 columns");
  __shared__ __align__(16) uint16_t vs[kKT * kVStr16];
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int C = a.cache_len;
  const int64_t p = a.pos[b];
  if (p < 0 && a.flags && split == 0 && g == 0 && lane == 0) a.flags[1] = 1u;   // reported by the layer check
  const int64_t weff = a.window > 0 ? a.window : C;
  const int64_t lo = p - weff + 1 > 0 ? p - weff + 1 : 0;
  const int nkeys = a.n_meta + static_cast<int>(p - lo + 1 > 0 ? p - lo + 1 : 0);
  // whole tiles per split (a partial tile costs a full one); trailing splits may be empty
  const int per = static_cast<int>(ceil_div(ceil_div(nkeys, a.splits), kKT) * kKT);
  const int k0 = split * per;
  const int k1 = min(nkeys, k0 + per);
  const int lo_mod = static_cast<int>(lo % C);   // ring slot of the first window key

  // Q^T as the B operand: column c16 = head g G + c16, k-step h = dims [32 h + 8 q, +8)
  const int c16 = lane & 15, q = lane >> 4;
  U4 qf[2];
  {
    const half_t* qrow = a.q + (int64_t)b * a.ld_q + (int64_t)(g * G + min(c16, G - 1)) * kHd + 8 * q;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const U4 v = *reinterpret_cast<const U4*>(qrow + 32 * h);
      qf[h] = c16 < G ? v : U4{0u, 0u, 0u, 0u};
    }
  }
  WaveState16 st;
#pragma unroll
  for (int db = 0; db < 4; ++db) st.acc[db] = f32x4_t{};
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
  // the tile starting at key t0 with nvalid keys: K rows 16 kb + c16 at dims 32 h + 8 q (the A
  // layout), and V chunks lane + 64 it (rows (item >> 3) + 16 j, dims 8 (item & 7)); rows past
  // nvalid read the last valid row (their scores are masked)
  auto fetch = [&](int t0, int nvalid, U4 (&kr)[4][2], U4 (&vr)[2][4]) {
    // A full tile wholly in the meta rows, or wholly in one unwrapped stretch of the ring, is a
    // strided block: one base for the tile and 32-bit row offsets.  Other tiles (the one across
    // the meta/window boundary, the one across the ring's wrap, a partial last tile) take the
    // per-row mapping.
    const int meta_rows = min(max(a.n_meta - t0, 0), kKT);
    int s0 = lo_mod + (t0 + meta_rows - a.n_meta);   // ring slot of the tile's first window key
    if (s0 >= C) s0 -= C;
    if (nvalid == kKT && (meta_rows == kKT || (meta_rows == 0 && s0 + kKT <= C))) {   // uniform
      const bool meta = meta_rows == kKT;
      const half_t* kb = meta ? a.k_meta + (int64_t)t0 * a.ld_meta + g * kHd : a.k_cache + (ring + s0) * kHd;
      const half_t* vb = meta ? a.v_meta + (int64_t)t0 * a.ld_meta + g * kHd : a.v_cache + (ring + s0) * kHd;
      const int stride = meta ? static_cast<int>(a.ld_meta) : kHd;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          kr[kk][h] = meta ? kv_load<false>(kb + (16 * kk + c16) * stride + 32 * h + 8 * q)
                           : kv_load<true>(kb + (16 * kk + c16) * stride + 32 * h + 8 * q);
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int item = lane + 64 * it;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          vr[it][j] = meta ? kv_load<false>(vb + ((item >> 3) + 16 * j) * stride + (item & 7) * 8)
                           : kv_load<true>(vb + ((item >> 3) + 16 * j) * stride + (item & 7) * 8);
      }
      return;
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int64_t ko = row_off(t0 + min(16 * kk + c16, nvalid - 1));
      const half_t* krow = (ko < 0 ? a.k_meta + (-1 - ko) : a.k_cache + ko) + 8 * q;
#pragma unroll
      for (int h = 0; h < 2; ++h) kr[kk][h] = ko < 0 ? kv_load<false>(krow + 32 * h) : kv_load<true>(krow + 32 * h);
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int item = lane + 64 * it;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int vrow = (item >> 3) + 16 * j, vcol = (item & 7) * 8;
        const int64_t vo = row_off(t0 + min(vrow, nvalid - 1));
        vr[it][j] = vo < 0 ? kv_load<false>(a.v_meta + (-1 - vo) + vcol) : kv_load<true>(a.v_cache + vo + vcol);
      }
    }
  };
  U4 kr[4][2], vr[2][4];
  if (k0 < k1) fetch(k0, min(kKT, k1 - k0), kr, vr);
  for (int t0 = k0; t0 < k1; t0 += kKT) {
    const int nvalid = min(kKT, k1 - t0);
#pragma unroll
    for (int it = 0; it < 2; ++it) chunk_store(vr[it], vs, kVStr16, lane + 64 * it);   // V chunks
    __syncthreads();
    f32x4_t s[4];
    tile_scores16(s, qf, kr, lane, nvalid);
    if (t0 + kKT < k1) fetch(t0 + kKT, min(kKT, k1 - t0 - kKT), kr, vr);   // next tile in flight
    attend_tile16(st, s, vs, a.scale_log2, lane);
    __syncthreads();
  }

  // this split's partials of heads g G + c16 (c16 < G): acc over the lane's 16 dims, max (log2
  // units) and the sum over the column's four lanes
  const float ltot = sum_xor32(sum_xor16(st.l));
  if (c16 >= G) return;
  float* out = a.part + (((int64_t)b * a.n_heads + g * G + c16) * a.splits + split) * (kHd + 2);
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) out[16 * db + 4 * q + r] = st.acc[db][r];
  if (q == 0) {
    out[kHd] = st.m * a.scale_log2;
    out[kHd + 1] = ltot;
  }
}

// grid B * H, block hd threads: merge the split partials of one (sequence, head).
// One block per (sequence, head): thread t takes dim t % hd of the splits g, g + G, ... (group
// g = t / hd of G = blockDim / hd, about one group per 8 splits), merged online (running max, rescaled sums) eight splits at a
// time with all their loads issued first; the groups then meet in LDS in group order.  A split
// with no keys carries a max of -inf or a huge negative one, and weight 0.
constexpr int kCombineThreads = 256;   // at most; a multiple of every supported head dim
template <typename T>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(DecAttnArgs<T> a) {
  __shared__ float3 red[kCombineThreads];
  const int bh = blockIdx.x;
  const int hd = a.head_dim, G = blockDim.x / hd;
  const int d = threadIdx.x % hd, g = threadIdx.x / hd;
  const float* part = a.part + (int64_t)bh * a.splits * (hd + 2);
  float M = -INFINITY, num = 0.f, den = 0.f;
  auto merge = [&](float mb, float (&mv)[8], float (&ov)[8], float (&lv)[8], int n) {
    const float mn = fmaxf(M, mb);
    if (mn == -INFINITY) return;
    const float sc = M == mn ? 1.f : fast_exp2(M - mn);
    num *= sc;
    den *= sc;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < n) {
        const float w = fast_exp2(mv[j] - mn);   // mv = -inf gives 0
        num = fmaf(w, ov[j], num);
        den = fmaf(w, lv[j], den);
      }
    }
    M = mn;
  };
  for (int s0 = g; s0 < a.splits; s0 += 8 * G) {
    float mv[8], ov[8], lv[8];
    float mb = -INFINITY;
    int n = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int s = s0 + j * G;
      mv[j] = -INFINITY; ov[j] = 0.f; lv[j] = 0.f;
      if (s < a.splits) {
        const float* ps = part + (int64_t)s * (hd + 2);
        mv[j] = ps[hd];
        ov[j] = ps[d];
        lv[j] = ps[hd + 1];
        n = j + 1;
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) mb = fmaxf(mb, mv[j]);
    merge(mb, mv, ov, lv, n);
  }
  red[threadIdx.x] = make_float3(M, num, den);
  __syncthreads();
  if (g != 0) return;
  for (int k = 1; k < G; ++k) {
    const float3 o = red[k * hd + d];
    const float mn = fmaxf(M, o.x);
    if (mn == -INFINITY) continue;
    const float s1 = M == mn ? 1.f : fast_exp2(M - mn), s2 = o.x == mn ? 1.f : fast_exp2(o.x - mn);
    num = num * s1 + o.y * s2;
    den = den * s1 + o.z * s2;
    M = mn;
  }
  const int b = bh / a.n_heads, h = bh % a.n_heads;
  Elem<T>::store(a.o + (int64_t)b * a.ld_o + h * hd + d, num / den);
}

// Eight splits or fewer: one thread per (sequence, head, dim), 256 / hd heads to a block, the
// same single merge the kernel above makes with one group (so the same results).
template <typename T>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_few_kernel(DecAttnArgs<T> a) {
  const int hd = a.head_dim;
  const int64_t bh = (int64_t)blockIdx.x * (kCombineThreads / hd) + threadIdx.x / hd;
  if (bh >= (int64_t)a.B * a.n_heads) return;
  const int d = threadIdx.x % hd;
  const float* part = a.part + bh * a.splits * (hd + 2);
  float mv[8], ov[8], lv[8];
  float mb = -INFINITY;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    mv[j] = -INFINITY; ov[j] = 0.f; lv[j] = 0.f;
    if (j < a.splits) {
      const float* ps = part + (int64_t)j * (hd + 2);
      mv[j] = ps[hd];
      ov[j] = ps[d];
      lv[j] = ps[hd + 1];
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) mb = fmaxf(mb, mv[j]);
  float num = 0.f, den = 0.f;
  if (mb != -INFINITY) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < a.splits) {
        const float w = fast_exp2(mv[j] - mb);
        num = fmaf(w, ov[j], num);
        den = fmaf(w, lv[j], den);
      }
    }
  }
  const int64_t b = bh / a.n_heads;
  const int h = static_cast<int>(bh % a.n_heads);
  Elem<T>::store(a.o + b * a.ld_o + h * hd + d, num / den);
}

template <typename T>
hipError_t launch_combine(const DecAttnArgs<T>& a, hipStream_t s);

// groups of head_dim threads: about one per 8 splits, at most kCombineThreads threads
template <typename T>
unsigned combine_threads(const DecAttnArgs<T>& a) {
  const int gmax = kCombineThreads / a.head_dim;
  return static_cast<unsigned>(a.head_dim * std::min(gmax, std::max(1, (a.splits + 7) / 8)));
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
      return launch_combine(a, s);
    }
  }
  if (a.head_dim == 64) e = dec_dispatch_hd<T, 64>(a, s);
  else if (a.head_dim == 32) e = dec_dispatch_hd<T, 32>(a, s);
  else return hipErrorInvalidValue;
  if (e != hipSuccess) return e;
  return launch_combine(a, s);
}

template <typename T>
hipError_t launch_combine(const DecAttnArgs<T>& a, hipStream_t s) {
  if (a.splits <= 8) {
    const int per_block = kCombineThreads / a.head_dim;
    hipLaunchKernelGGL((decode_combine_few_kernel<T>),
                       dim3(static_cast<unsigned>(ceil_div((int64_t)a.B * a.n_heads, per_block))),
                       dim3(kCombineThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((decode_combine_kernel<T>), dim3(a.B * a.n_heads), dim3(combine_threads(a)), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_write(const KvWriteArgs<float>& a, hipStream_t s) { return kv_dispatch(a, s); }
hipError_t launch_kv_write(const KvWriteArgs<half_t>& a, hipStream_t s) { return kv_dispatch(a, s); }
hipError_t launch_decode_attn(const DecAttnArgs<float>& a, hipStream_t s) { return dec_dispatch(a, s); }
hipError_t launch_decode_attn(const DecAttnArgs<half_t>& a, hipStream_t s) { return dec_dispatch(a, s); }

// Splits per (sequence, KV head), never fewer than 64 keys per split, at most kDecodeMaxSplits.
//  * MFMA kernel (16-bit K/V, head dim 64; one wave per workgroup): as few splits as give about
//    five workgroups per CU (1280 in all), each a whole number of its 64-key tiles, at most 16,
//    and no split left empty at the longest key range.  The 1152-key ring at B = 128 then takes
//    2 splits of 9 tiles, the 8193-key global cache at B = 8 27 splits of 5 tiles.  A split
//    that ends in a nearly empty tile pays for the whole tile: with splits of ceil(keys / splits)
//    keys the global decode measured 116-117 k tokens/s per layer at 32 splits (261 keys: 4
//    tiles and 5 keys) and 120-122 k at 44 (190 keys, just under 3 tiles).  Measured against the
//    earlier rule (~2048 workgroups, at most 3 tiles per split: 6 and 52 splits): 1.38 against
//    1.32 M tokens/s per layer for the ring decode pair, 122-123 k against 116-117 k for the
//    global decode; more workgroups (~4096) were slower for both.
//  * VALU kernel: enough for ~2048 workgroups (8 per CU), at least one load round per split
//    (256 / lanes per key row * kDecPasses keys).
// Longer splits run several rounds.
int decode_attn_splits(int B, int n_kv_heads, int n_keys_max, int head_dim, int elem_bytes) {
  const int lpk = head_dim * elem_bytes / 16;
  if (lpk < 2 || lpk > 16 || B < 1 || n_kv_heads < 1) return -1;
  const bool mfma = elem_bytes == 2 && head_dim == attn::kHd;
  const int64_t pairs = (int64_t)B * n_kv_heads;
  int64_t s;
  if (mfma) {
    const int64_t tiles = std::max<int64_t>(1, ceil_div(n_keys_max, attn::kKT));
    int64_t s0 = std::max<int64_t>(ceil_div(tiles, 16), ceil_div(1280, pairs));
    s0 = std::min<int64_t>(s0, std::min<int64_t>(tiles, kDecodeMaxSplits));
    s = ceil_div(tiles, ceil_div(tiles, s0));   // the fewest splits of that many tiles each
  } else {
    s = std::max<int64_t>(ceil_div(n_keys_max, (int64_t)(kThreads / lpk) * kDecPasses), ceil_div(2048, pairs));
  }
  s = std::min<int64_t>(s, std::max<int64_t>(1, ceil_div(n_keys_max, 64)));
  s = std::min<int64_t>(s, kDecodeMaxSplits);
  return static_cast<int>(std::max<int64_t>(s, 1));
}

}  // namespace hymba
