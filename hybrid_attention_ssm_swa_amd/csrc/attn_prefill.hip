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
//  * swa_meta_attn (MFMA): hd = 64, fp16 operands (the activation type of bf16
//    layers) with v_mfma_f32_32x32x16_f16 and fp32 accumulation.
//    One workgroup = 4 waves = 128 consecutive queries of one query head (a
//    32-query block per wave).  The K and V rows of the keys they can see
//    (meta, then the window span) stream through LDS in 32-key stages, four
//    buffers deep and loaded by the whole workgroup.  Each wave runs its stages as
//    a three-step software pipeline -- scores of stage h, softmax of stage
//    h - 1, P.V of stage h - 2 -- so that every step pairs 8 independent MFMAs
//    with the VALU work of one softmax in straight-line code.
//    Scores are computed transposed (S^T = K Q^T) so each lane owns one query
//    column and 16 keys of a 32-key stage: the softmax max needs one exchange
//    with lane l^32, and the probabilities feed the P.V product as the B
//    operand without any cross-lane movement.
//  * attn_f32: fp32 storage, one thread per (query, head), online softmax on
//    the VALU; used for the fp32 workload and small head dims.
#include "attn_tile.h"
#include "common.h"
#include "kernels.h"

namespace hymba {

namespace {

using namespace attn;

#ifndef HYMBA_ATTN_WAVES
#define HYMBA_ATTN_WAVES 4
#endif
constexpr int kWaves = HYMBA_ATTN_WAVES;   // waves per workgroup
constexpr int kQG = kWaves * kQB;          // queries per workgroup
constexpr int kHT = 32;                 // keys per LDS stage
constexpr int kStages = 4;              // LDS buffers (see the kernel's note on reuse)
constexpr int kXcds = 8;
constexpr int kLoadThreads = kWaves * 32;               // threads loading K (and as many loading V)
constexpr int kChunks = kHT * kHd * 2 / 16 / kLoadThreads;   // 16-byte chunks per thread and stage
constexpr int kRowStep = kLoadThreads / 8;              // rows between a thread's chunks
static_assert(kChunks >= 1 && kChunks * kLoadThreads * 16 == kHT * kHd * 2, "stage load shape");

typedef f16x8_t QV;

// Online-softmax state of one wave (lane l: query l % 32, 16 keys of each stage).  Each query
// keeps a reference m, the largest score seen when the reference last moved: a probability is
// 2^(sc s - sc m), one FMA and one exp per score, with no per-stage max.  The reference moves only
// when a stage would give some lane a probability sum above kGrowSum (every probability then stays
// far below fp16's overflow), or while the query has no reference yet; the rounding of sc m is
// common to every probability of the query and cancels in the normalisation.
struct Col {
  f32x16_t acc[2];   // O^T dims [0, 32) and [32, 64); column = query
  float m;           // reference, raw score units (-inf before the query's first visible key)
  float off;         // the exponent's offset -m sc (0 while m = -inf), kept with m
  float l;           // this lane's part of the row sum, relative to m
};
constexpr float kGrowSum = 4096.f;

// max of the lane's 16 scores of a stage, combined with lane l ^ 32 (the column's 32 keys)
__device__ __forceinline__ float block_max(const f32x16_t& s) {
  float mt = max3f(s[0], s[1], s[2]);
#pragma unroll
  for (int r = 3; r < 15; r += 2) mt = max3f(mt, s[r], s[r + 1]);
  mt = fmaxf(mt, s[15]);
  return max_xor32(mt);
}

// P^T of a stage as fp16 pairs (the B fragments of two P.V steps) and the lane's sum of exactly
// those rounded values: p = 2^(sc s + off), off = -sc m (0 for m = -inf; 0 for a masked score).
__device__ __forceinline__ float probs(const f32x16_t& s, float sc, float off, U4 (&pw)[2]) {
  float psum = 0.f;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    float p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = fast_exp2(fmaf(s[hh * 8 + j], sc, off));
    U4 w;
    w.x = pack_f16x2(p[0], p[1]);
    w.y = pack_f16x2(p[2], p[3]);
    w.z = pack_f16x2(p[4], p[5]);
    w.w = pack_f16x2(p[6], p[7]);
    psum = Op<half_t>::add_pair(w.x, psum);
    psum = Op<half_t>::add_pair(w.y, psum);
    psum = Op<half_t>::add_pair(w.z, psum);
    psum = Op<half_t>::add_pair(w.w, psum);
    pw[hh] = w;
  }
  return psum;
}

// Which keys of a stage the wave's queries may see.
struct Stage {
  int key0;             // index of its first key (meta index, or real index for window keys)
  int lo_key, hi_key;   // visible range before causality
  bool meta;            // meta keys: no causality, no window
  bool mask;            // some key of the stage is hidden from some query of the wave
};

// Mask of a stage: key j is kept iff lo_key <= j < hi_key and, for a real query tq, j <= tq and
// (win <= 0 or j > tq - win).  Register r holds key key0 + 4 half + o with o = 8 (r/4) + r%4
// (< 32); the lane's visible offsets form one range [a, b), kept as a 32-bit mask, so each score
// costs a bit extract and a bit select.
__device__ __forceinline__ void mask_stage(f32x16_t& s, const Stage& st, int tq, int win, int half) {
  int lo = st.lo_key, hi = st.hi_key;
  if (!st.meta) {
    hi = min(hi, tq + 1);
    if (win > 0) lo = max(lo, tq - win + 1);
  }
  const int base = st.key0 + 4 * half;
  const int a = min(max(lo - base, 0), 32), b = min(max(hi - base, 0), 32);
  const uint32_t below_b = b >= 32 ? ~0u : (1u << b) - 1u;
  const uint32_t below_a = a >= 32 ? ~0u : (1u << a) - 1u;
  const uint32_t keep = below_b & ~below_a;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int bit = 8 * (r >> 2) + (r & 3);
    const uint32_t m = static_cast<uint32_t>(static_cast<int32_t>(keep << (31 - bit)) >> 31);
    s[r] = __uint_as_float((__float_as_uint(s[r]) & m) | (0xff800000u & ~m));   // -inf: exp2 gives 0
  }
}

// S^T = K Q^T of a stage (K rows ks, row stride kKStr).
__device__ __forceinline__ void qk(f32x16_t& s, const QV (&q)[4], const uint16_t* ks, int lane) {
  const uint16_t* krow = ks + (lane & 31) * kKStr + (lane >> 5) * 8;
  s = f32x16_t{};
#pragma unroll
  for (int st4 = 0; st4 < 4; ++st4)
    s = Op<half_t>::mfma(as_vec<half_t>(*reinterpret_cast<const U4*>(krow + st4 * 16)), q[st4], s);
}

// O^T += V^T P^T over a stage.  PV k-step s2 covers the stage's keys [16 s2, 16 s2 + 16); k-index
// 8 h + j <-> key 16 s2 + 8 (j/4) + 4 h + j%4, which is where the score layout puts them.  The A
// fragment (lane l: dim 32 db + l % 32) comes from two transposed reads: lane group g = l / 16
// reads rows 16 s2 + 4 h (+ 8) + (l % 16) / 4 at dims 32 db + 16 (g % 2) + 4 (l % 4).
__device__ __forceinline__ void pv(Col& c, const U4 (&p)[2], const uint16_t* vs, int lane) {
  const uint16_t* vlane =
      vs + (4 * (lane >> 5) + ((lane & 15) >> 2)) * kVStr + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
  for (int db = 0; db < 2; ++db) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const uint2 lo = v_tr4(vlane + 16 * s2 * kVStr + 32 * db);
      const uint2 hi = v_tr4(vlane + (16 * s2 + 8) * kVStr + 32 * db);
      c.acc[db] = Op<half_t>::mfma(as_vec<half_t>(U4{lo.x, lo.y, hi.x, hi.y}), as_vec<half_t>(p[s2]), c.acc[db]);
    }
  }
}

// End of a step, for the stage whose probabilities p it just formed: if some lane's sum is too
// large, or some query has no reference yet, the reference moves to max(m, the stage max) -- the
// stage's scores recomputed from its K rows still in LDS and masked like it -- the accumulators and
// sums are rescaled and the probabilities recomputed; then the sums take the stage's.
__device__ __forceinline__ void settle(Col& c, U4 (&p)[2], float psum, const QV (&q)[4], const uint16_t* ks,
                                       const Stage& st, int tq, int win, float sc, int lane) {
  if (__builtin_amdgcn_ballot_w64(!(psum <= kGrowSum) || c.m == -INFINITY) != 0) {
    f32x16_t s;
    qk(s, q, ks, lane);
    if (st.mask) mask_stage(s, st, tq, win, lane >> 5);
    const float mnew = fmaxf(c.m, block_max(s));
    const float alpha = mnew == -INFINITY ? 1.f : fast_exp2((c.m - mnew) * sc);   // m = -inf: 0
    c.l *= alpha;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) c.acc[db][r] *= alpha;
    c.m = mnew;
    c.off = mnew == -INFINITY ? 0.f : -mnew * sc;
    psum = probs(s, sc, c.off, p);
  }
  c.l += psum;
}

// The calling thread's share of a stage (K rows at kbase, V rows at vbase, row stride ld elements,
// nvalid >= 1 valid rows): the first half of the workgroup's threads load K, the second half V (a
// wave-uniform choice); thread it's chunk j is row (it >> 3) + kRowStep j, dims 8 (it & 7) + 0..7,
// at byte offset voff + 2 kRowStep j ld for a full stage.  Rows past nvalid read the last valid
// row and are zero-filled.
struct StageRegs {
  U4 r[kChunks];
};
// A buffer resource for the 32 rows (row stride ld elements) from p: base and size are
// wave-uniform, so they live in scalar registers and a full stage's loads need no vector
// address arithmetic (the per-lane byte offset voff is computed once per kernel).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t stage_rsrc(const void* p, int ld) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32)));
  const uint64_t u = static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), 0, kHT * ld * 2, 0x00020000);
}
__device__ __forceinline__ void fetch_stage(StageRegs& t, const half_t* kbase, const half_t* vbase, int ld,
                                            uint32_t voff, int nvalid, bool is_k, int it) {
  const char* base = reinterpret_cast<const char*>(is_k ? kbase : vbase);
  if (nvalid >= kHT) {
    const auto rs = stage_rsrc(base, ld);
#pragma unroll
    for (int j = 0; j < kChunks; ++j)
      t.r[j] = __builtin_bit_cast(U4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, j * kRowStep * ld * 2, 0));
  } else {
    int row0 = it >> 3;
    const int col = (it & 7) * 8;
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const int row = row0 + kRowStep * j;
      t.r[j] = masked_load(base + (static_cast<int64_t>(min(row, nvalid - 1)) * ld + col) * 2, row < nvalid);
    }
  }
}
__device__ __forceinline__ void store_stage(const StageRegs& t, uint16_t* ks, uint16_t* vs, bool is_k, int it) {
  uint16_t* base = is_k ? ks : vs;
#pragma unroll
  for (int j = 0; j < kChunks; ++j)
    *reinterpret_cast<uint4*>(base + ((it >> 3) + kRowStep * j) * kKStr + (it & 7) * 8) =
        make_uint4(t.r[j].x, t.r[j].y, t.r[j].z, t.r[j].w);
}

struct AttnStages {
  uint16_t kw[kStages][kHT * kKStr];   // K rows [key][dim]
  uint16_t vw[kStages][kHT * kVStr];   // V rows [key][dim]
};

// Work items are numbered (sequence, KV head, query group, head of the group) -- so consecutive
// items share one window of K/V, or for a global layer one causal prefix, taken longest first --
// and consecutive items go to the same XCD (the dispatcher deals workgroups round-robin over the
// 8 XCDs), so an XCD's L2 holds the K/V its workgroups share.
//
// Step i of a wave: scores of stage i, the previous stage's softmax, the P.V product of stage i - 2:
//   S(i) = K(i) Q^T (4 MFMAs) ; O += V(i - 2)^T P(i - 2) (4 MFMAs) ; P(i - 1) = softmax(S(i - 1))
// The eight MFMAs are independent of the softmax, so they issue beside its VALU work.  A stage's
// K is read at step i and again (rare rescale) at step i + 1, its V at step i + 2.  Stage i is
// stored (into buffer i mod 4) after the barrier of stage i - 1, which every wave passes only once
// it has finished step i - 2; a wave still in step i - 1 reads stages i - 3 .. i - 1, so with four
// buffers and one barrier per stage no store overwrites what another wave still reads.
// Register budget: 4 waves per SIMD, at most 128 VGPRs (8 bytes of spills, outside the stage loop).
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(4))) void swa_meta_attn_kernel(
    AttnArgs<half_t> a) {
  __shared__ AttnStages sm;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, col = lane & 31;
  const int group = a.n_heads / a.n_kv_heads;
  const int nqg = static_cast<int>(ceil_div(a.T, kQG));
  const float sc = a.scale_log2;
  const int win = a.window;

  // ---- work item: XCD-aware renumbering, then (b, g, qg, hh) ------------------
  const int nwork = gridDim.x, L = blockIdx.x;
  const int xcd = L % kXcds, j = L / kXcds, per = nwork / kXcds, extra = nwork % kXcds;
  int work = (xcd < extra ? xcd * (per + 1) : extra * (per + 1) + (xcd - extra) * per) + j;
  const int hh = work % group;
  work /= group;
  int b, g, qg;
  qg = work % nqg; work /= nqg;
  g = work % a.n_kv_heads; b = work / a.n_kv_heads;
  if (win <= 0) qg = nqg - 1 - qg;   // global: the longest query groups of a (sequence, KV head) first
  const int h = g * group + hh;
  const int q0 = qg * kQG;
  const int qa = q0 + wave * kQB;               // this wave's first query
  const int qlast = min(qa + kQB, a.T) - 1;     // this wave's last query (qa - 1 for an idle wave)
  const int tq = min(qa + col, a.T - 1);

  // ---- stages: the meta keys, then the workgroup's window span [lo, hi) --------
  const int n_ms = static_cast<int>(ceil_div(a.n_meta, kHT));
  const int lo = win > 0 ? max(0, q0 - win + 1) : 0;
  const int hi = min(a.T, q0 + kQG);
  const int n_st = n_ms + static_cast<int>(ceil_div(hi - lo, kHT));
  const half_t* kseq = a.k + (int64_t)b * a.kv_seq_stride + g * kHd;
  const half_t* vseq = a.v + (int64_t)b * a.kv_seq_stride + g * kHd;
  const int ld_meta = static_cast<int>(a.ld_meta), ld_kv = static_cast<int>(a.ld_kv);
  const bool is_k = wave < kWaves / 2;
  const int it = tid & (kLoadThreads - 1);
  const uint32_t voff_meta = static_cast<uint32_t>(((it >> 3) * ld_meta + (it & 7) * 8) * 2);
  const uint32_t voff_kv = static_cast<uint32_t>(((it >> 3) * ld_kv + (it & 7) * 8) * 2);
  auto fetch = [&](StageRegs& r, int i) {
    if (i < n_ms) {
      const int64_t off = (int64_t)i * kHT * a.ld_meta + g * kHd;
      fetch_stage(r, a.k_meta + off, a.v_meta + off, ld_meta, voff_meta, a.n_meta - i * kHT, is_k, it);
    } else {
      const int t0 = lo + (i - n_ms) * kHT;
      fetch_stage(r, kseq + (int64_t)t0 * a.ld_kv, vseq + (int64_t)t0 * a.ld_kv, ld_kv, voff_kv, hi - t0, is_k,
                  it);
    }
  };
  auto stage_of = [&](int i) {   // branch-free (scalar selects)
    Stage st;
    const bool meta = i < n_ms;
    const int t0 = lo + (i - n_ms) * kHT;
    const bool full = (t0 + kHT - 1 <= qa) & ((win <= 0) | (t0 > qlast - win)) & (t0 + kHT <= hi);
    st.meta = meta;
    st.key0 = meta ? i * kHT : t0;
    st.lo_key = meta ? 0 : t0;
    st.hi_key = meta ? a.n_meta : hi;
    st.mask = meta ? (i * kHT + kHT > a.n_meta) : !full;
    return st;
  };
  // Whether some key of stage i is hidden from some query of the wave.  Window stage w = i - n_ms
  // starts at t0 = lo + 32 w, and it is whole for the wave iff t0 + 31 <= qa (below the diagonal),
  // t0 + 32 <= hi, and t0 > qlast - win (inside every query's window): w in [w_edge, w_end], one
  // range, fixed once per wave.  The meta stages are whole except a partial last one.  So the test
  // is two scalar compares per stage (floor divisions by 32 as arithmetic shifts).
  const int w_end = min((qa - lo - (kHT - 1)) >> 5, (hi - lo - kHT) >> 5);
  const int w_edge = win > 0 ? max(((qlast - win - lo) >> 5) + 1, 0) : 0;
  const int m_first = n_ms - (a.n_meta % kHT != 0 ? 1 : 0);   // first masked stage at or before the window
  const int i_edge = n_ms + w_edge, i_end = n_ms + w_end;
  auto masked = [&](int i) { return (i >= m_first && i < i_edge) || i > i_end; };
  // Q^T fragments: k-step s holds dims 16 s + 8 (lane/32) .. +7 of query tq
  QV qf[4];
  {
    const half_t* qrow = a.q + ((int64_t)b * a.T + tq) * a.ld_q + h * kHd + (lane >> 5) * 8;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) qf[s4] = as_vec<half_t>(*reinterpret_cast<const U4*>(qrow + s4 * 16));
  }
  Col c;
  c.acc[0] = c.acc[1] = f32x16_t{};
  c.m = -INFINITY;
  c.off = 0.f;
  c.l = 0.f;

  // pipeline registers: scores of stage i - 1, probabilities of stage i - 2
  f32x16_t s1 = f32x16_t{};
  U4 p2[2] = {};
  StageRegs pre;
  fetch(pre, 0);
  // the step's common part: scores of stage i (if any), P.V of stage i - 2 (if any), softmax of
  // stage i - 1 (if any); the rare settle and the edge masking come after it
  auto step = [&](int i, bool do_qk, bool do_pv, bool do_soft) {
    const int buf = i % kStages;
    const Stage st_cur = stage_of(i), st_prev = stage_of(i - 1);
    f32x16_t s0;
    if (do_qk) qk(s0, qf, sm.kw[buf], lane);
    if (do_pv) pv(c, p2, sm.vw[(i + 2) % kStages], lane);     // stage i - 2
    if (do_soft) {
      U4 p1[2];
      const float ps = probs(s1, sc, c.off, p1);
      if (do_qk && do_pv) {   // the steady step: one MFMA, then a share of the softmax VALU, eight times
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
        }
      }
      const int pb = (i + 3) % kStages;                        // stage i - 1
      settle(c, p1, ps, qf, sm.kw[pb], st_prev, tq, win, sc, lane);
      p2[0] = p1[0];
      p2[1] = p1[1];
    }
    if (do_qk) {
      if (masked(i)) mask_stage(s0, st_cur, tq, win, lane >> 5);
      s1 = s0;
    }
  };
  auto load = [&](int i) {   // stage i into its buffer, visible to the workgroup; stage i + 1 requested
    store_stage(pre, sm.kw[i % kStages], sm.vw[i % kStages], is_k, it);
    __syncthreads();
    fetch(pre, min(i + 1, n_st - 1));
  };
  // prologue (n_st >= 1)
  load(0);
  step(0, true, false, false);
  if (n_st > 1) {
    load(1);
    step(1, true, false, true);
  }
  // steady state: all three parts
  for (int i = 2; i < n_st; ++i) {
    load(i);
    step(i, true, true, true);
  }
  // drain
  step(n_st, false, n_st >= 2, true);
  step(n_st + 1, false, true, false);

  if (qa < a.T && qa + col < a.T) {
    const float inv = 1.f / sum_xor32(c.l);
    half_t* orow = a.o + ((int64_t)b * a.T + qa + col) * a.ld_o + h * kHd;
    const int half = lane >> 5;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dim = db * 32 + 8 * r4 + 4 * half;
        uint2 w;
        w.x = pack_f16x2(c.acc[db][r4 * 4 + 0] * inv, c.acc[db][r4 * 4 + 1] * inv);
        w.y = pack_f16x2(c.acc[db][r4 * 4 + 2] * inv, c.acc[db][r4 * 4 + 3] * inv);
        *reinterpret_cast<uint2*>(orow + dim) = w;
      }
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


}  // namespace

hipError_t launch_attn_prefill_mfma(const AttnArgs<half_t>& a, hipStream_t stream) {
  const int group = a.n_heads / a.n_kv_heads;
  const int64_t nwork = (int64_t)a.B * a.n_kv_heads * group * ceil_div(a.T, kQG);
  if (nwork > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(swa_meta_attn_kernel, dim3(static_cast<unsigned>(nwork)), dim3(kWaves * 64), 0, stream, a);
  return hipGetLastError();
}

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
  return head_dim == kHd && n_kv_heads > 0 && n_heads % n_kv_heads == 0 && n_meta >= 0;
}

}  // namespace hymba
