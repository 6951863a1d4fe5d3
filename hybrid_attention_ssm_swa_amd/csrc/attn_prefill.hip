// Prefill attention of the hybrid-head mixer: softmax attention of every real
// query over (all meta-token keys) + (the most recent `window` real keys,
// causal), or over all earlier keys for a global layer.
//
// Method: Hymba summary (greeksharifa.github.io) section 2.2 (sliding-window
// attention in most layers, global in first/middle/last) and section 2.3
// (meta tokens prepended to every sequence, visible to every query); the
// window includes the query itself and does not count meta keys.  Grouped KV
// heads: query head h reads KV head floor(h * Hkv / H).
//
// Two kernels:
//  * swa_meta_attn (MFMA): hd = 64, 16-bit operands (fp16 for the layer's
//    activations, bf16 also instantiated) with v_mfma_f32_32x32x16_{f16,bf16}
//    and fp32 accumulation.
//    One workgroup = one (sequence, KV head) and a run of 32-query blocks; one
//    wave per query head of the group (GQA: the K/V tile staged in LDS serves
//    every head of the group).  The meta K and V^T tiles are loaded into LDS
//    once per workgroup and stay resident for all its query blocks; window
//    tiles of 64 keys stream through a double-buffered LDS stage.
//    Scores are computed transposed (S^T = K Q^T) so each lane owns one query
//    column and 16 keys of a 32-key block: the softmax max needs one exchange
//    with lane l^32, and the probabilities feed the P.V product as the B
//    operand without any cross-lane movement.
//  * attn_f32: fp32 storage, one thread per (query, head), online softmax on
//    the VALU; used for the fp32 workload and small head dims.
#include "common.h"
#include "kernels.h"

namespace hymba {

namespace {

constexpr int kHd = 64;          // head dim of the MFMA kernel
constexpr int kQB = 32;          // queries per wave (one MFMA column block)
constexpr int kKT = 64;          // keys per tile
constexpr int kKStr = kHd + 8;   // LDS row stride (bf16) of K tiles: 144 B
constexpr int kVStr = kKT + 4;   // LDS row stride (bf16) of V^T window tiles: 136 B
constexpr int kMaxMeta = 128;    // resident meta keys (the pages' meta-token count)
constexpr int kMetaVStr = kMaxMeta + 4;
constexpr int kMaxWaves = 8;

struct __align__(16) U4 { uint32_t x, y, z, w; };

template <typename ET> struct Op;
template <> struct Op<half_t> {
  typedef f16x8_t vec;
  __device__ static __forceinline__ f32x16_t mfma(vec a, vec b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct Op<bf16_t> {
  typedef bf16x8_t vec;
  __device__ static __forceinline__ f32x16_t mfma(vec a, vec b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <typename ET>
__device__ __forceinline__ typename Op<ET>::vec as_vec(U4 v) { return __builtin_bit_cast(typename Op<ET>::vec, v); }

// 16-bit elements stored as raw 16-bit words
struct AttnSmem {
  uint16_t kw[2][kKT * kKStr];        // window K tiles  [key][dim]
  uint16_t vw[2][kHd * kVStr];        // window V^T tiles [dim][key]
  uint16_t km[kMaxMeta * kKStr];      // meta K          [key][dim]
  uint16_t vm[kHd * kMetaVStr];       // meta V^T        [dim][key]
};

// Cooperative load of a 64-key tile (K rows straight, V transposed) for the
// whole workgroup: 128 work items, each owning 4 of the 512 16-byte K chunks
// (64 rows x 8) and a 4-key x 8-dim block of V.  Rows beyond `nvalid` are
// zero-filled.
struct TileRegs {
  U4 k[4];
  U4 v[4];
};

__device__ __forceinline__ uint32_t u4_get(const U4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ U4 masked_load(const void* p, bool keep) {
  const U4 x = *reinterpret_cast<const U4*>(p);
  U4 r;
  r.x = keep ? x.x : 0u;
  r.y = keep ? x.y : 0u;
  r.z = keep ? x.z : 0u;
  r.w = keep ? x.w : 0u;
  return r;
}

template <typename ET>
__device__ __forceinline__ void tile_fetch(TileRegs& r, const ET* __restrict__ kbase,
                                           const ET* __restrict__ vbase, int64_t ld,
                                           int nvalid, int item) {
  // item in [0, 128): K chunks item + 128 j (j < 4) of 512 (64 rows x 8 chunks);
  // V block: keys 4*(item/8) .. +3, dims 8*(item%8) .. +7
  // rows >= nvalid (>= 1) read a clamped, valid row and are zeroed by value
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = item + j * 128;
    const int row = c >> 3, col = (c & 7) * 8;
    r.k[j] = masked_load(kbase + (int64_t)min(row, nvalid - 1) * ld + col, row < nvalid);
  }
  const int key0 = (item >> 3) * 4, dim0 = (item & 7) * 8;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = key0 + j;
    r.v[j] = masked_load(vbase + (int64_t)min(row, nvalid - 1) * ld + dim0, row < nvalid);
  }
}

__device__ __forceinline__ void tile_store(const TileRegs& r, uint16_t* ks, uint16_t* vs, int vstr,
                                           int key_off, int item) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = item + j * 128;
    const int row = c >> 3, col = (c & 7) * 8;
    *reinterpret_cast<U4*>(ks + (key_off + row) * kKStr + col) = r.k[j];
  }
  // transpose 4 keys x 8 dims -> 8 rows (dims) of 4 consecutive keys
  const int key0 = key_off + (item >> 3) * 4, dim0 = (item & 7) * 8;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    // dims dim0+2p (low halves) and dim0+2p+1 (high halves)
    const uint32_t a = u4_get(r.v[0], p), b = u4_get(r.v[1], p);
    const uint32_t c = u4_get(r.v[2], p), d = u4_get(r.v[3], p);
    uint2 lo, hi;
    lo.x = __builtin_amdgcn_perm(b, a, 0x05040100u);   // (a.lo, b.lo)
    lo.y = __builtin_amdgcn_perm(d, c, 0x05040100u);
    hi.x = __builtin_amdgcn_perm(b, a, 0x07060302u);   // (a.hi, b.hi)
    hi.y = __builtin_amdgcn_perm(d, c, 0x07060302u);
    *reinterpret_cast<uint2*>(vs + (dim0 + 2 * p) * vstr + key0) = lo;
    *reinterpret_cast<uint2*>(vs + (dim0 + 2 * p + 1) * vstr + key0) = hi;
  }
}

struct WaveState {
  f32x16_t acc[2];    // O^T blocks: dims [0,32) and [32,64), column = query
  float m;            // running max (raw score units)
  float l;            // partial row sum over this lane's keys
};

// One 64-key tile: S^T = K Q^T, online softmax, O^T += V^T P^T.
// ks: [64][kKStr] K rows; vs: [64 dims][vstr] V^T; key0: first key index of
// the tile in the mask's coordinates.  With kMask, key j is kept iff
// lo_key <= j < hi_key and, for tq >= 0 (a real query tq), j <= tq and
// (win <= 0 or j > tq - win).
template <typename ET, bool kMask>
__device__ __forceinline__ void attend_tile(WaveState& st, const typename Op<ET>::vec (&qf)[4],
                                            const uint16_t* ks, const uint16_t* vs, int vstr,
                                            float sc, int lane, int key0, int lo_key, int hi_key,
                                            int tq, int win) {
  const int col = lane & 31, half = lane >> 5;
  f32x16_t s[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    s[kb] = f32x16_t{};
    const uint16_t* krow = ks + (kb * 32 + col) * kKStr + half * 8;
#pragma unroll
    for (int st4 = 0; st4 < 4; ++st4) {
      const auto a = as_vec<ET>(*reinterpret_cast<const U4*>(krow + st4 * 16));
      s[kb] = Op<ET>::mfma(a, qf[st4], s[kb]);
    }
  }
  if (kMask) {
    // key index of register r of block kb: key0 + 32 kb + 8 (r/4) + 4 half + r%4
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        bool vis = key >= lo_key && key < hi_key;          // tile bounds (meta count / T)
        if (tq >= 0) vis = vis && key <= tq && (win <= 0 || key > tq - win);
        if (!vis) s[kb][r] = -INFINITY;
      }
  }
  float mt = s[0][0];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
  mt = fmaxf(mt, __shfl_xor(mt, 32));
  const float mnew = fmaxf(st.m, mt);
  const float alpha = fast_exp2((st.m - mnew) * sc);
  st.m = mnew;
  const float msc = mnew * sc;
  float psum = 0.f;
  typename Op<ET>::vec pf[4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p[j] = fast_exp2(fmaf(s[kb][hh * 8 + j], sc, -msc));
        psum += p[j];
      }
      U4 w;
      w.x = Pair<ET>::pack(p[0], p[1]);
      w.y = Pair<ET>::pack(p[2], p[3]);
      w.z = Pair<ET>::pack(p[4], p[5]);
      w.w = Pair<ET>::pack(p[6], p[7]);
      pf[kb * 2 + hh] = as_vec<ET>(w);
    }
  }
  st.l = fmaf(st.l, alpha, psum);
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.acc[db][r] *= alpha;
  // O^T[dim][q] += sum_k V^T[dim][k] P^T[k][q]; PV k-step s covers tile keys
  // [16 s, 16 s + 16); k-index 8 h + j <-> key 16 s + 8 (j/4) + 4 h + j%4.
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    const uint16_t* vrow = vs + (db * 32 + col) * vstr + 4 * half;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const uint2 lo = *reinterpret_cast<const uint2*>(vrow + 16 * s4);
      const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16 * s4 + 8);
      U4 w = {lo.x, lo.y, hi.x, hi.y};
      st.acc[db] = Op<ET>::mfma(as_vec<ET>(w), pf[s4], st.acc[db]);
    }
  }
}

// grid: (n_work, Hkv, B); block: 64 * max(2, heads per group) threads: one wave
// per head of the group (a group of one gets a helper wave for the tile loads).
// Work item x covers query blocks [x*qb_per_wg, (x+1)*qb_per_wg) (ordered so
// the longest causal runs start first).
template <typename ET>
__global__ __launch_bounds__(512) void swa_meta_attn_kernel(AttnArgs<ET> a) {
  __shared__ AttnSmem sm;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int nthreads = blockDim.x;
  const int g = blockIdx.y, b = blockIdx.z;
  const int group = a.n_heads / a.n_kv_heads;
  const int h = g * group + wave;
  const float sc = a.scale_log2;
  const int n_items = 128;   // tile work items

  // ---- resident meta tiles -------------------------------------------------
  const int mpad = static_cast<int>(ceil_div(a.n_meta, kKT)) * kKT;
  for (int t0 = 0; t0 < mpad; t0 += kKT) {
    for (int it = tid; it < n_items; it += nthreads) {
      TileRegs r;
      tile_fetch(r, a.k_meta + (int64_t)t0 * a.ld_meta + g * kHd,
                 a.v_meta + (int64_t)t0 * a.ld_meta + g * kHd, a.ld_meta, a.n_meta - t0, it);
      tile_store(r, sm.km, sm.vm, kMetaVStr, t0, it);
    }
  }
  __syncthreads();

  const int nqb = static_cast<int>(ceil_div(a.T, kQB));
  const int work = gridDim.x - 1 - blockIdx.x;
  const int qb0 = work * a.qb_per_wg;
  const int qb1 = min(nqb, qb0 + a.qb_per_wg);
  const int col = lane & 31;
  const bool wave_active = wave < group;

  const ET* kseq = a.k + (int64_t)b * a.kv_seq_stride + g * kHd;
  const ET* vseq = a.v + (int64_t)b * a.kv_seq_stride + g * kHd;

  for (int qb = qb0; qb < qb1; ++qb) {
    const int q0 = qb * kQB;
    const int tq = min(q0 + col, a.T - 1);
    // Q^T fragments: k-step s holds dims 16 s + 8 (lane/32) .. +7 of query tq
    typename Op<ET>::vec qf[4];
    {
      // a helper wave (no head of its own) reads the group's first head
      const int hq = wave_active ? h : g * group;
      const ET* qrow = a.q + ((int64_t)b * a.T + tq) * a.ld_q + hq * kHd + (lane >> 5) * 8;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) qf[s4] = as_vec<ET>(*reinterpret_cast<const U4*>(qrow + s4 * 16));
    }
    WaveState st;
    st.acc[0] = f32x16_t{};
    st.acc[1] = f32x16_t{};
    st.m = -1e30f;
    st.l = 0.f;

    // meta keys: visible to every real query; mask only the padding tail
    if (wave_active) {
      for (int t0 = 0; t0 < mpad; t0 += kKT) {
        if (t0 + kKT <= a.n_meta)
          attend_tile<ET, false>(st, qf, sm.km + t0 * kKStr, sm.vm + t0, kMetaVStr, sc, lane, t0, 0,
                                 a.n_meta, -1, 0);
        else
          attend_tile<ET, true>(st, qf, sm.km + t0 * kKStr, sm.vm + t0, kMetaVStr, sc, lane, t0, 0,
                                a.n_meta, -1, 0);
      }
    }

    // window keys [lo, hi)
    const int qlast = min(q0 + kQB, a.T) - 1;
    const int lo = a.window > 0 ? max(0, q0 - a.window + 1) : 0;
    const int hi = qlast + 1;
    const int ntiles = static_cast<int>(ceil_div(hi - lo, kKT));
    TileRegs pre;
    if (tid < n_items)
      tile_fetch(pre, kseq + (int64_t)lo * a.ld_kv, vseq + (int64_t)lo * a.ld_kv, a.ld_kv,
                 hi - lo, tid);
    for (int i = 0; i < ntiles; ++i) {
      const int buf = i & 1;
      const int t0 = lo + i * kKT;
      if (tid < n_items) tile_store(pre, sm.kw[buf], sm.vw[buf], kVStr, 0, tid);
      __syncthreads();
      if (i + 1 < ntiles && tid < n_items) {
        const int t1 = t0 + kKT;
        tile_fetch(pre, kseq + (int64_t)t1 * a.ld_kv, vseq + (int64_t)t1 * a.ld_kv, a.ld_kv,
                   hi - t1, tid);
      }
      if (wave_active) {
        // the tile needs a mask unless every key is visible to every query of the block
        const bool full = (t0 + kKT - 1 <= q0) && (a.window <= 0 || t0 > qlast - a.window) &&
                          (t0 + kKT <= hi);
        if (full)
          attend_tile<ET, false>(st, qf, sm.kw[buf], sm.vw[buf], kVStr, sc, lane, t0, t0, hi, tq, a.window);
        else
          attend_tile<ET, true>(st, qf, sm.kw[buf], sm.vw[buf], kVStr, sc, lane, t0, t0, hi, tq, a.window);
      }
    }

    if (wave_active) {
      const float ltot = st.l + __shfl_xor(st.l, 32);
      const float inv = 1.f / ltot;
      const int t = q0 + col;
      if (t < a.T) {
        ET* orow = a.o + ((int64_t)b * a.T + t) * a.ld_o + h * kHd;
        const int half = lane >> 5;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int dim = db * 32 + 8 * r4 + 4 * half;
            uint2 w;
            w.x = Pair<ET>::pack(st.acc[db][r4 * 4 + 0] * inv, st.acc[db][r4 * 4 + 1] * inv);
            w.y = Pair<ET>::pack(st.acc[db][r4 * 4 + 2] * inv, st.acc[db][r4 * 4 + 3] * inv);
            *reinterpret_cast<uint2*>(orow + dim) = w;
          }
      }
    }
    __syncthreads();   // window buffers are reused by the next query block
  }
}

// ---- fp32 VALU kernel --------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(128) void attn_f32_kernel(AttnArgs<float> a) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.B * a.T * a.n_heads;
  if (gid >= total) return;
  const int h = static_cast<int>(gid % a.n_heads);
  const int64_t bt = gid / a.n_heads;
  const int t = static_cast<int>(bt % a.T);
  const int b = static_cast<int>(bt / a.T);
  const int g = h / (a.n_heads / a.n_kv_heads);
  float q[HD], acc[HD];
  const float* qrow = a.q + ((int64_t)b * a.T + t) * a.ld_q + h * HD;
#pragma unroll
  for (int d = 0; d < HD; ++d) { q[d] = qrow[d] * a.scale_log2; acc[d] = 0.f; }
  float m = -1e30f, l = 0.f;
  auto visit = [&](const float* krow, const float* vrow) {
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < HD; ++d) s = fmaf(q[d], krow[d], s);
    const float mn = fmaxf(m, s);
    const float al = fast_exp2(m - mn), p = fast_exp2(s - mn);
    l = fmaf(l, al, p);
#pragma unroll
    for (int d = 0; d < HD; ++d) acc[d] = fmaf(acc[d], al, p * vrow[d]);
    m = mn;
  };
  for (int j = 0; j < a.n_meta; ++j)
    visit(a.k_meta + (int64_t)j * a.ld_meta + g * HD, a.v_meta + (int64_t)j * a.ld_meta + g * HD);
  const int lo = a.window > 0 ? max(0, t - a.window + 1) : 0;
  const float* kseq = a.k + (int64_t)b * a.kv_seq_stride + g * HD;
  const float* vseq = a.v + (int64_t)b * a.kv_seq_stride + g * HD;
  for (int s = lo; s <= t; ++s) visit(kseq + (int64_t)s * a.ld_kv, vseq + (int64_t)s * a.ld_kv);
  const float inv = 1.f / l;
  float* orow = a.o + ((int64_t)b * a.T + t) * a.ld_o + h * HD;
#pragma unroll
  for (int d = 0; d < HD; ++d) orow[d] = acc[d] * inv;
}


template <typename ET>
hipError_t launch_mfma(const AttnArgs<ET>& args, hipStream_t stream) {
  AttnArgs<ET> a = args;
  const int group = a.n_heads / a.n_kv_heads;
  const int nqb = static_cast<int>(ceil_div(a.T, kQB));
  if (a.qb_per_wg <= 0) {
    // enough workgroups to fill the chip, but long runs so the meta tiles stay useful
    const int64_t per_seq_head = (int64_t)a.B * a.n_kv_heads;
    int q = 4;
    while (q > 1 && per_seq_head * ceil_div(nqb, q) < 2048) q >>= 1;
    a.qb_per_wg = q;
  }
  const int nwork = static_cast<int>(ceil_div(nqb, a.qb_per_wg));
  dim3 grid(nwork, a.n_kv_heads, a.B);
  dim3 block(64 * (group < 2 ? 2 : group));
  hipLaunchKernelGGL((swa_meta_attn_kernel<ET>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_prefill_mfma(const AttnArgs<half_t>& a, hipStream_t s) { return launch_mfma(a, s); }
hipError_t launch_attn_prefill_mfma(const AttnArgs<bf16_t>& a, hipStream_t s) { return launch_mfma(a, s); }

hipError_t launch_attn_prefill_f32(const AttnArgs<float>& a, hipStream_t stream) {
  const int64_t total = (int64_t)a.B * a.T * a.n_heads;
  dim3 grid(static_cast<unsigned>(ceil_div(total, 128))), block(128);
  switch (a.head_dim) {
    case 32: hipLaunchKernelGGL(attn_f32_kernel<32>, grid, block, 0, stream, a); break;
    case 64: hipLaunchKernelGGL(attn_f32_kernel<64>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool attn_mfma_supported(int head_dim, int n_heads, int n_kv_heads, int n_meta) {
  return head_dim == kHd && n_kv_heads > 0 && n_heads % n_kv_heads == 0 &&
         n_heads / n_kv_heads <= kMaxWaves && n_meta <= kMaxMeta;
}

}  // namespace hymba
