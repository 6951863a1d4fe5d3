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
//    One workgroup = 4 waves = 128 consecutive queries of one query head (a
//    32-query block per wave).  The K tiles and transposed V tiles of the keys
//    those queries can see (meta, then the window span) stream through a
//    double-buffered LDS stage loaded by all four waves; the heads of a GQA
//    group reuse the same K/V through the L2 of the XCD their workgroups run on.
//    Scores are computed transposed (S^T = K Q^T) so each lane owns one query
//    column and 16 keys of a 32-key block: the softmax max needs one exchange
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

// One workgroup = 4 waves = kQG consecutive queries (one 32-query block per
// wave) of one query head.  The workgroup streams the key tiles its queries
// can see -- the meta tiles, then the window span [q0 - W + 1, q0 + kQG) (all
// earlier keys for a global layer) -- through a double-buffered LDS stage that
// all four waves load and share; a wave skips tiles outside its own window.
// Work items are numbered (sequence, KV head, query group, head of the group)
// for SWA -- so consecutive items reuse one window of K/V -- and with the
// longest query groups first for global layers; consecutive items go to the
// same XCD (the dispatcher deals workgroups round-robin over the 8 XCDs), so
// an XCD's L2 holds the K/V its workgroups share.
constexpr int kQG = 4 * kQB;
constexpr int kXcds = 8;

template <typename ET>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void swa_meta_attn_kernel(AttnArgs<ET> a) {
  __shared__ AttnSmem sm;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31;
  const int group = a.n_heads / a.n_kv_heads;
  const int nqg = static_cast<int>(ceil_div(a.T, kQG));
  const float sc = a.scale_log2;

  // ---- work item: XCD-aware renumbering, then (b, g, qg, hh) ------------------
  const int nwork = gridDim.x, L = blockIdx.x;
  const int xcd = L % kXcds, j = L / kXcds, per = nwork / kXcds, extra = nwork % kXcds;
  int work = (xcd < extra ? xcd * (per + 1) : extra * (per + 1) + (xcd - extra) * per) + j;
  const int hh = work % group;
  work /= group;
  int b, g, qg;
  if (a.window > 0) {
    qg = work % nqg; work /= nqg;
    g = work % a.n_kv_heads; b = work / a.n_kv_heads;
  } else {
    g = work % a.n_kv_heads; work /= a.n_kv_heads;
    b = work % a.B; qg = nqg - 1 - work / a.B;
  }
  const int h = g * group + hh;
  const int q0 = qg * kQG;
  const int qa = q0 + wave * kQB;               // this wave's first query
  const bool wave_active = qa < a.T;
  const int qlast = min(qa + kQB, a.T) - 1;     // this wave's last query
  const int tq = min(qa + col, a.T - 1);

  // ---- key tiles: meta first, then the window span [lo, hi) ------------------
  const int n_mt = static_cast<int>(ceil_div(a.n_meta, kKT));
  const int lo = a.window > 0 ? max(0, q0 - a.window + 1) : 0;
  const int hi = min(a.T, q0 + kQG);
  const int n_tiles = n_mt + static_cast<int>(ceil_div(hi - lo, kKT));
  const ET* kseq = a.k + (int64_t)b * a.kv_seq_stride + g * kHd;
  const ET* vseq = a.v + (int64_t)b * a.kv_seq_stride + g * kHd;
  const int ld_meta = static_cast<int>(a.ld_meta), ld_kv = static_cast<int>(a.ld_kv);
  auto fetch = [&](TileRegs& r, int i) {
    if (i < n_mt) {
      const int64_t off = (int64_t)i * kKT * a.ld_meta + g * kHd;
      tile_fetch(r, a.k_meta + off, a.v_meta + off, ld_meta, a.n_meta - i * kKT, tid);
    } else {
      const int t0 = lo + (i - n_mt) * kKT;
      tile_fetch(r, kseq + (int64_t)t0 * a.ld_kv, vseq + (int64_t)t0 * a.ld_kv, ld_kv, hi - t0, tid);
    }
  };

  // Q^T fragments: k-step s holds dims 16 s + 8 (lane/32) .. +7 of query tq
  typename Op<ET>::vec qf[4];
  {
    const ET* qrow = a.q + ((int64_t)b * a.T + tq) * a.ld_q + h * kHd + (lane >> 5) * 8;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) qf[s4] = as_vec<ET>(*reinterpret_cast<const U4*>(qrow + s4 * 16));
  }
  WaveState st;
  st.acc[0] = f32x16_t{};
  st.acc[1] = f32x16_t{};
  st.m = -INFINITY;
  st.l = 0.f;
  st.bias = (lane >> 5) ? 0u : Pair<ET>::pack(INFINITY, 0.f);
  st.exact = false;

  TileRegs pre;
  fetch(pre, 0);
  for (int i = 0; i < n_tiles; ++i) {
    const int buf = i & 1;
    tile_store(pre, sm.kw[buf], sm.vw[buf], tid);
    __syncthreads();
    if (i + 1 < n_tiles) fetch(pre, i + 1);
    // Every wave runs every tile of the workgroup: a tile outside a wave's window (or a wave past
    // the end of the sequence) is simply all masked and adds nothing.  Branching around it splits
    // the loop-carried accumulators across paths and costs a 32-register copy per tile.
    int key0, lo_key, hi_key, tqm;
    bool mask;
    if (i < n_mt) {
      // meta keys: visible to every real query; only the padding tail is masked
      key0 = i * kKT; lo_key = 0; hi_key = a.n_meta; tqm = -1;
      mask = key0 + kKT > a.n_meta;
    } else {
      const int t0 = lo + (i - n_mt) * kKT;
      key0 = t0; lo_key = t0; hi_key = hi; tqm = tq;
      mask = !((t0 + kKT - 1 <= qa) && (a.window <= 0 || t0 > qlast - a.window) && (t0 + kKT <= hi));
    }
    attend_tile<ET>(st, qf, sm.kw[buf], sm.vw[buf], kVStr, sc, lane, key0, lo_key, hi_key, tqm, a.window, mask, i == 0);
  }

  if (wave_active) {
    const float ltot = sum_xor32(st.l);
    const float inv = 1.f / ltot;
    const int t = qa + col;
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
hipError_t launch_mfma(const AttnArgs<ET>& a, hipStream_t stream) {
  const int group = a.n_heads / a.n_kv_heads;
  const int64_t nwork = (int64_t)a.B * a.n_kv_heads * group * ceil_div(a.T, kQG);
  if (nwork > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((swa_meta_attn_kernel<ET>), dim3(static_cast<unsigned>(nwork)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_prefill_mfma(const AttnArgs<half_t>& a, hipStream_t s) { return launch_mfma(a, s); }

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
