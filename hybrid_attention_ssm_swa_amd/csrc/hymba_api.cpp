// C ABI of the hybrid-head mixer: validation, persistent/workspace carving,
// the meta-prefix preparation and the launch sequence of prefill and decode.
// Every step of the layer runs in this library's HIP kernels (attention,
// scan, epilogue, K/V movement, conversions) or its hipBLASLt projection GEMMs.
//
// Types: an fp32 layer stores and computes in fp32.  A bf16 layer keeps bf16
// at its boundary (x, y, weights) and uses fp16 activations inside (shared
// projection, attention operands and output, W_O output, scan output, fused
// epilogue output, the K/V it exchanges and caches) with fp32 accumulation
// and fp32 SSM state; its weights get fp16 copies in the persistent buffer.
#include "hymba_mixer.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <new>
#include <type_traits>
#include <string>
#include <vector>

#include "errors.h"
#include "gemm_blaslt.h"
#include "kernels.h"

using namespace hymba;

// Scratch of the allocation-free decode step (hymba_mixer_decode_static): every device the library
// runs on holds its own copy until the process ends.
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

struct hymba_layer {
  hymba_layer_cfg cfg;
  hymba_layer_weights w;
  // persistent buffer carve
  char* k_meta = nullptr;      // [M, Hkv, hd] activation type
  char* v_meta = nullptr;
  float* h_meta = nullptr;     // [E, N]
  char* y_meta = nullptr;      // [M, d] storage type
  float* A2 = nullptr;         // [E, N] A * log2(e)
  uint32_t* flags = nullptr;   // [3] device-side checks: non-finite branch statistic, bad decode position,
                               // a weight beyond fp16's range (sticky)
  half_t* w_in16 = nullptr;    // bf16 layers: fp16 copies of the weights
  half_t* w_o16 = nullptr;
  bool prepared = false;
  // second stream of a prefill (the SSM branch runs beside attention and W_O), created on first use
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  bool overlap = true;                     // prefill: SSM branch on the side stream (false: all on the call's stream)
  int side_device = -1;
  bool weights_ready = false;
  const hymba_layer* producer = nullptr;   // consumer: bound producer
  const hymba_layer* consumer = nullptr;   // producer: its bound consumer (pairs only)
  const void* prep_kmeta = nullptr;        // consumer: meta K/V used by the last prepare
  const void* prep_vmeta = nullptr;
  int gemm_backend = HYMBA_GEMM_LIBRARY;   // bf16 prefill projections (HYMBA_GEMM_LIBRARY or _TILED)
  // column offsets of the shared projection
  int64_t n_in = 0, ld_p = 0, off_k = 0, off_v = 0, off_u = 0, off_z = 0, off_dt = 0, off_b = 0;
  // stage timing: a pool of begin/end event pairs, one pair per timed interval of each hot call
  bool profiling = false;
  std::vector<hipEvent_t> ev;          // 2 * kProfPairs events once profiling was first enabled
  std::vector<int8_t> ev_stage;        // stage of each used pair
  int ev_next = 0;                     // pairs used since profiling was enabled
  int prof_calls = 0;                  // prefill/decode calls recorded since then
  bool prof_overflow = false;
};

namespace {
thread_local std::string g_err;
}  // namespace

int32_t hymba::set_error(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

namespace {

constexpr auto fail = hymba::set_error;

int32_t hip_fail(hipError_t e, const char* what) {
  return fail(HYMBA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(expr, what)                              \
  do {                                                   \
    hipError_t e_ = (expr);                              \
    if (e_ != hipSuccess) return hip_fail(e_, what);     \
  } while (0)

#define STATUS_TRY(expr)            \
  do {                              \
    int32_t s_ = (expr);            \
    if (s_ != HYMBA_OK) return s_;  \
  } while (0)

constexpr int kProfPairs = 1024;

// Brackets one stage interval with a pair of events from the layer's pool when it is profiling.
struct StageTimer {
  hymba_layer& L;
  hipStream_t s;
  int pair = -1;
  StageTimer(const hymba_layer& l, int stage, hipStream_t stream) : L(const_cast<hymba_layer&>(l)), s(stream) {
    if (!L.profiling) return;
    if (L.ev_next >= kProfPairs) { L.prof_overflow = true; return; }
    pair = L.ev_next++;
    L.ev_stage[pair] = static_cast<int8_t>(stage);
    hipEventRecord(L.ev[2 * pair], s);
  }
  ~StageTimer() {
    if (pair >= 0) hipEventRecord(L.ev[2 * pair + 1], s);
  }
};
enum { ST_IN_PROJ = 0, ST_KV = 1, ST_ATTN = 2, ST_WO = 3, ST_SSM = 4, ST_EPI = 5, ST_OUT = 6, ST_CVT = 7,
       ST_ROPE = 8 };
const char* kStageNames[HYMBA_N_STAGES] = {"in_proj", "kv_write", "attention", "w_o", "ssm",
                                           "epilogue", "out_proj", "convert", "rope"};

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline bool is_bf16(const hymba_layer_cfg& c) { return c.dtype == HYMBA_BF16; }
inline size_t storage_size(const hymba_layer_cfg& c) { return is_bf16(c) ? 2 : 4; }
inline size_t act_size(const hymba_layer_cfg& c) { return is_bf16(c) ? 2 : 4; }

int64_t n_in_of(const hymba_layer_cfg& c) {
  const int64_t q = (int64_t)c.n_heads * c.head_dim;
  const int64_t kv = c.own_kv ? 2 * (int64_t)c.n_kv_heads * c.head_dim : 0;
  return q + kv + 3 * (int64_t)c.d_inner + 2 * (int64_t)c.d_state;
}

int32_t check_cfg(const hymba_layer_cfg* c) {
  if (!c) return fail(HYMBA_ERR_INVALID_ARG, "cfg is NULL");
  if (c->d_model < 1 || c->n_heads < 1 || c->n_kv_heads < 1 || c->head_dim < 1 || c->d_inner < 1 ||
      c->d_state < 1 || c->n_meta < 0)
    return fail(HYMBA_ERR_INVALID_ARG, "dimensions must be positive (n_meta >= 0)");
  if (c->n_heads % c->n_kv_heads != 0)
    return fail(HYMBA_ERR_INVALID_ARG, "n_heads (%d) must be a multiple of n_kv_heads (%d)", c->n_heads,
                c->n_kv_heads);
  if (c->dtype != HYMBA_F32 && c->dtype != HYMBA_BF16)
    return fail(HYMBA_ERR_INVALID_ARG, "dtype must be HYMBA_F32 or HYMBA_BF16");
  if (c->own_kv != 0 && c->own_kv != 1) return fail(HYMBA_ERR_INVALID_ARG, "own_kv must be 0 or 1");
  if (!(c->rms_eps >= 0.f) || !std::isfinite(c->rms_eps))
    return fail(HYMBA_ERR_INVALID_ARG, "rms_eps must be finite and >= 0");
  if (!(c->rope_base >= 0.f) || !std::isfinite(c->rope_base))
    return fail(HYMBA_ERR_INVALID_ARG, "rope_base must be finite and >= 0");
  if (c->rope_base > 0.f && (c->head_dim % 8 != 0 || c->head_dim / 2 > kRopeMaxPairs))
    return fail(HYMBA_ERR_UNSUPPORTED, "rotary encoding needs head_dim a multiple of 8, at most 128");
  if (c->d_state != 8 && c->d_state != 16)
    return fail(HYMBA_ERR_UNSUPPORTED, "d_state must be 8 or 16 (got %d)", c->d_state);
  if (c->d_inner % 8 != 0) return fail(HYMBA_ERR_UNSUPPORTED, "d_inner must be a multiple of 8");
  if (c->d_model % 8 != 0) return fail(HYMBA_ERR_UNSUPPORTED, "d_model must be a multiple of 8");
  if (c->dtype == HYMBA_BF16) {
    if (!attn_mfma_supported(c->head_dim, c->n_heads, c->n_kv_heads, c->n_meta) || c->n_heads / c->n_kv_heads > 8)
      return fail(HYMBA_ERR_UNSUPPORTED, "bf16 layers need head_dim 64 and n_heads/n_kv_heads <= 8");
  } else {
    if (c->head_dim != 32 && c->head_dim != 64)
      return fail(HYMBA_ERR_UNSUPPORTED, "fp32 attention needs head_dim 32 or 64");
    if (c->n_heads / c->n_kv_heads > 8)
      return fail(HYMBA_ERR_UNSUPPORTED, "n_heads/n_kv_heads must be <= 8");
  }
  return HYMBA_OK;
}

struct PersistLayout {
  size_t k_meta, v_meta, h_meta, y_meta, A2, flags, w_in16, w_o16, total;
};

PersistLayout persist_layout(const hymba_layer_cfg& c) {
  const size_t as = act_size(c), ss = storage_size(c);
  PersistLayout p{};
  size_t off = 0;
  const size_t kv = (size_t)c.n_meta * c.n_kv_heads * c.head_dim * as;
  p.k_meta = off; off += align_up(kv);
  p.v_meta = off; off += align_up(kv);
  p.h_meta = off; off += align_up((size_t)c.d_inner * c.d_state * 4);
  p.y_meta = off; off += align_up((size_t)c.n_meta * c.d_model * ss);
  p.A2 = off; off += align_up((size_t)c.d_inner * c.d_state * 4);
  p.flags = off; off += align_up(3 * sizeof(uint32_t));
  if (is_bf16(c)) {
    const size_t hq = (size_t)c.n_heads * c.head_dim;
    p.w_in16 = off; off += align_up((size_t)n_in_of(c) * c.d_model * 2);
    p.w_o16 = off; off += align_up((size_t)c.d_inner * hq * 2);
  }
  p.total = off;
  return p;
}

struct WsLayout {
  size_t X16, P, bc32, O, Ao, Ys, F, gemm, part, seg, seg_bytes, total;
  int64_t rows;
  bool own_kernels_only = false;   // every projection on the hand-written GEMMs (no library workspace)
};

WsLayout ws_layout(const hymba_layer& L, int64_t batch, int64_t seq) {
  const hymba_layer_cfg& c = L.cfg;
  const size_t as = act_size(c);
  const bool b16 = is_bf16(c);
  const int64_t rows = std::max<int64_t>(batch * seq, c.n_meta);
  WsLayout w{};
  w.rows = rows;
  size_t off = 0;
  w.X16 = off; off += b16 ? align_up((size_t)rows * c.d_model * 2) : 0;
  w.P = off; off += align_up((size_t)rows * L.ld_p * as);
  w.bc32 = off; off += b16 ? align_up((size_t)rows * 2 * c.d_state * 4) : 0;
  w.O = off; off += align_up((size_t)rows * c.n_heads * c.head_dim * as);
  w.Ao = off; off += align_up((size_t)rows * c.d_inner * as);
  w.Ys = off; off += align_up((size_t)rows * c.d_inner * as);
  w.F = off; off += align_up((size_t)rows * c.d_inner * as);
  w.gemm = off; off += b16 ? kGemmWorkspaceBytes : 0;
  w.part = off;
  off += align_up((size_t)std::max<int64_t>(batch, 1) * c.n_heads * kDecodeMaxSplits * (c.head_dim + 2) * 4);
  // time-segment summaries of the prefill scan (and of the meta-prefix scan)
  w.seg = off;
  w.seg_bytes = std::max(scan_segment_bytes((int)std::max<int64_t>(batch, 1), (int)std::max<int64_t>(seq, 1),
                                            c.d_inner, c.d_state),
                         scan_segment_bytes(1, std::max(c.n_meta, 1), c.d_inner, c.d_state));
  off += align_up(w.seg_bytes);
  w.total = off;
  return w;
}

// Workspace of a decode step that runs every projection on the hand-written GEMMs: no x
// conversion buffer, no GEMM library workspace, and split-K partials for the call's own split
// count.  0 if the key range has no split plan.
WsLayout ws_layout_own_kernels(const hymba_layer& L, int64_t batch, int splits) {
  const hymba_layer_cfg& c = L.cfg;
  const size_t as = act_size(c);
  const bool b16 = is_bf16(c);
  WsLayout w{};
  w.rows = batch;
  w.own_kernels_only = true;
  size_t off = 0;
  w.X16 = off;
  w.P = off; off += align_up((size_t)batch * L.ld_p * as);
  w.bc32 = off; off += b16 ? align_up((size_t)batch * 2 * c.d_state * 4) : 0;
  w.O = off; off += align_up((size_t)batch * c.n_heads * c.head_dim * as);
  w.Ao = off; off += align_up((size_t)batch * c.d_inner * as);
  w.Ys = off; off += align_up((size_t)batch * c.d_inner * as);
  w.F = off; off += align_up((size_t)batch * c.d_inner * as);
  w.gemm = off;
  w.part = off; off += align_up((size_t)batch * c.n_heads * splits * (c.head_dim + 2) * 4);
  w.total = off;
  return w;
}

// Y[rows, out] = X[rows, in] . W[out, in]^T.  fp32 layers: fp32 kernel.  bf16
// layers: hipBLASLt with fp32 accumulation; fp16 operands and output for the
// input projection and W_O (bf16_out = false), bf16 operands and output for
// the output projection (bf16_out = true).
int32_t project(const hymba_layer& L, const void* X, int64_t ldx, const void* W, int64_t ldw, void* Y,
                int64_t ldy, int64_t rows, int64_t out, int64_t in, bool bf16_out, char* ws, const WsLayout& wl,
                hipStream_t s) {
  if (is_bf16(L.cfg) && (wl.own_kernels_only || skinny_fits(rows, out, in))) {   // few rows: weight streaming
    hipError_t e;
    if (bf16_out) {
      SkinnyArgs<bf16_t, bf16_t, bf16_t> a{static_cast<const bf16_t*>(W), ldw, static_cast<const bf16_t*>(X), ldx,
                                           static_cast<bf16_t*>(Y), ldy, nullptr, 0, 0, 0, static_cast<int>(rows),
                                           static_cast<int>(out), static_cast<int>(in)};
      e = launch_skinny_gemm(a, s);
    } else {
      SkinnyArgs<half_t, half_t, half_t> a{static_cast<const half_t*>(W), ldw, static_cast<const half_t*>(X), ldx,
                                           static_cast<half_t*>(Y), ldy, nullptr, 0, 0, 0, static_cast<int>(rows),
                                           static_cast<int>(out), static_cast<int>(in)};
      e = launch_skinny_gemm(a, s);
    }
    HIP_TRY(e, "projection (few rows) launch");
    return HYMBA_OK;
  }
  if (is_bf16(L.cfg) && L.gemm_backend == HYMBA_GEMM_TILED) {   // many rows: the tiled matrix-core GEMM
    MfmaGemmArgs a{X, ldx, W, ldw, Y, ldy, nullptr, 0, 0, 0, rows, static_cast<int>(out), static_cast<int>(in)};
    const int t = bf16_out ? GT_BF16 : GT_F16;
    if (!mfma_gemm_shape_ok(a)) return fail(HYMBA_ERR_UNSUPPORTED, "projection GEMM: unsupported shape or alignment");
    HIP_TRY(launch_mfma_gemm(a, t, t, s), "projection GEMM launch");
    return HYMBA_OK;
  }
  if (is_bf16(L.cfg)) {
    const char* err = nullptr;
    const GemmType t = bf16_out ? GT_BF16 : GT_F16;
    const int r = gemm_16(t, t, X, ldx, W, ldw, Y, ldy, rows, out, in, ws + wl.gemm, kGemmWorkspaceBytes, s, &err);
    if (r != 0) return fail(r == -2 ? HYMBA_ERR_UNSUPPORTED : HYMBA_ERR_HIP, "projection GEMM: %s", err);
    return HYMBA_OK;
  }
  HIP_TRY(launch_gemm_f32(static_cast<const float*>(X), ldx, static_cast<const float*>(W), ldw,
                          static_cast<float*>(Y), ldy, rows, static_cast<int>(out), static_cast<int>(in), s),
          "fp32 projection GEMM launch");
  return HYMBA_OK;
}

template <typename CT>
int32_t run_attention(const hymba_layer_cfg& c, const CT* q, int64_t ld_q, const CT* k, const CT* v,
                      int64_t ld_kv, int64_t seq_stride, const CT* k_meta, const CT* v_meta, int n_meta, CT* o,
                      int64_t ld_o, int B, int T_, int window, hipStream_t s) {
  AttnArgs<CT> a{};
  a.q = q; a.ld_q = ld_q;
  a.k = k; a.v = v; a.ld_kv = ld_kv; a.kv_seq_stride = seq_stride;
  a.k_meta = k_meta; a.v_meta = v_meta; a.ld_meta = (int64_t)c.n_kv_heads * c.head_dim; a.n_meta = n_meta;
  a.o = o; a.ld_o = ld_o;
  a.B = B; a.T = T_; a.n_heads = c.n_heads; a.n_kv_heads = c.n_kv_heads; a.head_dim = c.head_dim;
  a.window = window;
  a.scale_log2 = kLog2e / std::sqrt(static_cast<float>(c.head_dim));
  if constexpr (sizeof(CT) == 2) {
    HIP_TRY(launch_attn_prefill_mfma(a, s), "attention launch");
  } else {
    HIP_TRY(launch_attn_prefill_f32(a, s), "attention launch");
  }
  return HYMBA_OK;
}

// Meta K/V the layer attends to, or NULL if unavailable.
void meta_kv_of(const hymba_layer& L, const hymba_kv* kv, const void** km, const void** vm) {
  if (L.cfg.own_kv) { *km = L.k_meta; *vm = L.v_meta; return; }
  if (L.producer) { *km = L.producer->k_meta; *vm = L.producer->v_meta; return; }
  *km = kv ? kv->k_meta : nullptr;
  *vm = kv ? kv->v_meta : nullptr;
}

// Shared projection of `rows` rows of x (storage type) into P (activation type).  A bf16 layer
// also writes the B/C columns in fp32 to bc32 (from the fp32 accumulator): every channel's
// normalised SSM output depends on sum_n C[n] B[n] of its token, so those shared columns keep fp32.
template <typename CT>
int32_t in_projection(const hymba_layer& L, const void* x, int64_t rows, char* ws, const WsLayout& wl,
                      hipStream_t s) {
  const hymba_layer_cfg& c = L.cfg;
  float* bc32 = reinterpret_cast<float*>(ws + wl.bc32);
  if (is_bf16(c) && (wl.own_kernels_only || skinny_fits(rows, L.n_in, c.d_model))) {
    // few rows: one weight-streaming GEMM reads x in bf16 (converted to fp16 on the way in) and
    // writes P in fp16, plus the B/C columns in fp32
    StageTimer st(L, ST_IN_PROJ, s);
    SkinnyArgs<half_t, bf16_t, half_t> a{L.w_in16, c.d_model, static_cast<const bf16_t*>(x), c.d_model,
                                         reinterpret_cast<half_t*>(ws + wl.P), L.ld_p, bc32, 2 * c.d_state,
                                         static_cast<int>(L.off_b), static_cast<int>(L.off_b + 2 * c.d_state),
                                         static_cast<int>(rows), static_cast<int>(L.n_in), c.d_model};
    HIP_TRY(launch_skinny_gemm(a, s), "input projection (few rows) launch");
    return HYMBA_OK;
  }
  if (is_bf16(c) && L.gemm_backend == HYMBA_GEMM_TILED) {
    // many rows: the tiled GEMM multiplies bf16 x and W_in directly, writes P in fp16 and the
    // B/C columns in fp32 from its accumulator
    StageTimer st(L, ST_IN_PROJ, s);
    MfmaGemmArgs a{x, c.d_model, L.w.w_in, c.d_model, ws + wl.P, L.ld_p, bc32, 2 * c.d_state,
                   static_cast<int>(L.off_b), static_cast<int>(L.off_b + 2 * c.d_state), rows,
                   static_cast<int>(L.n_in), c.d_model};
    if (!mfma_gemm_shape_ok(a)) return fail(HYMBA_ERR_UNSUPPORTED, "input projection: unsupported shape or alignment");
    HIP_TRY(launch_mfma_gemm(a, GT_BF16, GT_F16, s), "input projection launch");
    return HYMBA_OK;
  }
  if (is_bf16(c)) {
    half_t* x16 = reinterpret_cast<half_t*>(ws + wl.X16);
    {
      // x to fp16 for the GEMM, fused with the fp32 B/C columns
      StageTimer st(L, ST_CVT, s);
      ConvBcArgs a{static_cast<const bf16_t*>(x), c.d_model, x16, c.d_model, L.w_in16 + L.off_b * c.d_model,
                   c.d_model, bc32, 2 * c.d_state, rows, c.d_model, 2 * c.d_state};
      HIP_TRY(launch_convert_bc(a, s), "input conversion");
    }
    StageTimer st(L, ST_IN_PROJ, s);
    return project(L, x16, c.d_model, L.w_in16, c.d_model, ws + wl.P, L.ld_p, rows, L.n_in, c.d_model, false, ws,
                   wl, s);
  }
  StageTimer st(L, ST_IN_PROJ, s);
  return project(L, x, c.d_model, L.w.w_in, c.d_model, ws + wl.P, L.ld_p, rows, L.n_in, c.d_model, false, ws, wl,
                 s);
}

// Rotary encoding of the q (and, for a producer, k) columns of `rows` projection rows in place:
// row r sits at position first + pos[r] (decode) or first + r % T.
template <typename CT>
int32_t apply_rope(const hymba_layer& L, char* ws, const WsLayout& wl, int64_t rows, int64_t T, int64_t first,
                   const int64_t* pos, hipStream_t s) {
  const hymba_layer_cfg& c = L.cfg;
  if (!(c.rope_base > 0.f)) return HYMBA_OK;
  StageTimer st(L, ST_ROPE, s);
  RopeArgs<CT> a{};
  a.p = reinterpret_cast<CT*>(ws + wl.P); a.ld = L.ld_p;
  a.rows = rows; a.T = T;
  a.n_q_heads = c.n_heads; a.k_off = L.off_k; a.n_k_heads = c.own_kv ? c.n_kv_heads : 0; a.head_dim = c.head_dim;
  a.first = first; a.pos = pos;
  for (int i = 0; i < c.head_dim / 2; ++i)
    a.theta[i] = std::pow(static_cast<double>(c.rope_base), -2.0 * i / c.head_dim);
  HIP_TRY(launch_rope(a, s), "rotary encoding launch");
  return HYMBA_OK;
}

// W_O of `rows` rows: attention output O -> Ao.
template <typename CT>
int32_t w_o_projection(const hymba_layer& L, char* ws, const WsLayout& wl, int64_t rows, hipStream_t s) {
  const hymba_layer_cfg& c = L.cfg;
  const int64_t hq = (int64_t)c.n_heads * c.head_dim;
  StageTimer st(L, ST_WO, s);
  return project(L, ws + wl.O, hq, is_bf16(c) ? (const void*)L.w_o16 : L.w.w_o, hq, ws + wl.Ao, c.d_inner, rows,
                 c.d_inner, hq, false, ws, wl, s);
}

// Fused epilogue and output projection of `rows` rows; y_out in storage type.
template <typename CT>
int32_t epilogue_and_out(const hymba_layer& L, char* ws, const WsLayout& wl, int64_t rows, void* y_out,
                         hipStream_t s) {
  const hymba_layer_cfg& c = L.cfg;
  const bool b16 = is_bf16(c);
  {
    // bf16 layers write F as bf16: the output projection then multiplies the layer's own bf16
    // W_out and writes y in bf16 directly (one rounding of the fp32 accumulator)
    typedef typename std::conditional<std::is_same<CT, float>::value, float, bf16_t>::type FT;
    StageTimer st(L, ST_EPI, s);
    EpiArgs<CT, FT> e{};
    const CT* P = reinterpret_cast<const CT*>(ws + wl.P);
    e.ao = reinterpret_cast<const CT*>(ws + wl.Ao); e.ld_ao = c.d_inner;
    e.y = reinterpret_cast<const CT*>(ws + wl.Ys); e.ld_y = c.d_inner;
    e.z = P + L.off_z; e.ld_z = L.ld_p;
    e.beta1 = L.w.beta1; e.beta2 = L.w.beta2;
    e.f = reinterpret_cast<FT*>(ws + wl.F); e.ld_f = c.d_inner;
    e.rows = rows; e.E = c.d_inner; e.eps = c.rms_eps;
    e.flags = L.flags;
    HIP_TRY(launch_epilogue(e, s), "epilogue launch");
  }
  StageTimer st(L, ST_OUT, s);
  return project(L, ws + wl.F, c.d_inner, L.w.w_out, c.d_inner, y_out, c.d_model, rows, c.d_model, c.d_inner,
                 b16, ws, wl, s);
}

// W_O, fused epilogue, output projection on one stream.
template <typename CT>
int32_t tail(const hymba_layer& L, char* ws, const WsLayout& wl, int64_t rows, void* y_out, hipStream_t s) {
  STATUS_TRY(w_o_projection<CT>(L, ws, wl, rows, s));
  return epilogue_and_out<CT>(L, ws, wl, rows, y_out, s);
}

// The side stream and fork/join events of a layer on the current device.
int32_t ensure_side_stream(hymba_layer& L) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
  if (L.side && L.side_device == dev) return HYMBA_OK;
  if (L.side) {
    hipStreamDestroy(L.side);
    hipEventDestroy(L.ev_fork);
    hipEventDestroy(L.ev_join);
    L.side = nullptr;
  }
  HIP_TRY(hipStreamCreateWithFlags(&L.side, hipStreamNonBlocking), "side stream create");
  HIP_TRY(hipEventCreateWithFlags(&L.ev_fork, hipEventDisableTiming), "event create");
  HIP_TRY(hipEventCreateWithFlags(&L.ev_join, hipEventDisableTiming), "event create");
  L.side_device = dev;
  return HYMBA_OK;
}

template <typename CT>
ScanArgs<CT> scan_args(const hymba_layer& L, char* ws, const WsLayout& wl, int B, int T_, const float* h0,
                       float* h_out) {
  const hymba_layer_cfg& c = L.cfg;
  const CT* P = reinterpret_cast<const CT*>(ws + wl.P);
  ScanArgs<CT> sa{};
  sa.u = P + L.off_u; sa.dt = P + L.off_dt; sa.ld = L.ld_p;
  if (is_bf16(c)) {
    sa.bc = reinterpret_cast<const float*>(ws + wl.bc32); sa.ld_bc = 2 * c.d_state;
  } else {
    sa.bc = reinterpret_cast<const float*>(P + L.off_b); sa.ld_bc = L.ld_p;
  }
  sa.A2 = L.A2; sa.D = L.w.D; sa.dt_bias = L.w.dt_bias;
  sa.h0 = h0; sa.h0_bstride = 0;
  sa.y = reinterpret_cast<CT*>(ws + wl.Ys); sa.ldy = c.d_inner;
  sa.h_out = h_out;
  sa.B = B; sa.T = T_; sa.E = c.d_inner; sa.N = c.d_state;
  sa.seg = reinterpret_cast<float*>(ws + wl.seg); sa.seg_bytes = wl.seg_bytes;
  return sa;
}

template <typename CT>
int32_t prepare_impl(hymba_layer& L, const hymba_kv* kv, char* ws, const WsLayout& wl, hipStream_t s) {
  const hymba_layer_cfg& c = L.cfg;
  const int M = c.n_meta;
  if (!L.weights_ready) {
    HIP_TRY(launch_fill(reinterpret_cast<float*>(L.flags), 3, 0.f, s), "check flags clear");
    HIP_TRY(launch_scale_copy(L.w.A, L.A2, (int64_t)c.d_inner * c.d_state, kLog2e, s), "A scaling");
    if (is_bf16(c)) {
      const int64_t hq = (int64_t)c.n_heads * c.head_dim;
      HIP_TRY(launch_convert(static_cast<const bf16_t*>(L.w.w_in), c.d_model, L.w_in16, c.d_model, L.n_in,
                             c.d_model, s), "weight conversion");
      HIP_TRY(launch_convert(static_cast<const bf16_t*>(L.w.w_o), hq, L.w_o16, hq, c.d_inner, hq, s),
              "weight conversion");
      // a bf16 weight beyond fp16's range is inf in the copies: recorded for hymba_layer_check
      HIP_TRY(launch_nonfinite16_check(L.w_in16, L.n_in * c.d_model, L.flags + 2, s), "weight range check");
      HIP_TRY(launch_nonfinite16_check(L.w_o16, (int64_t)c.d_inner * hq, L.flags + 2, s), "weight range check");
    }
    L.weights_ready = true;
  }
  const void *km = nullptr, *vm = nullptr;
  if (!c.own_kv) {
    meta_kv_of(L, kv, &km, &vm);
    if (M > 0 && L.producer && !L.producer->prepared)
      return fail(HYMBA_ERR_BIND, "the bound producer must be prepared before its consumer");
    if (M > 0 && (!km || !vm))
      return fail(HYMBA_ERR_INVALID_ARG, "an unbound consumer needs kv->k_meta and kv->v_meta");
  }
  if (M == 0) {
    HIP_TRY(launch_fill(L.h_meta, (int64_t)c.d_inner * c.d_state, 0.f, s), "state clear");
    L.prepared = true;
    L.prep_kmeta = km; L.prep_vmeta = vm;
    return HYMBA_OK;
  }
  STATUS_TRY(in_projection<CT>(L, L.w.meta, M, ws, wl, s));
  STATUS_TRY(apply_rope<CT>(L, ws, wl, M, M, 0, nullptr, s));   // meta rows at positions 0..M-1
  const CT* P = reinterpret_cast<const CT*>(ws + wl.P);
  const int64_t kvw = (int64_t)c.n_kv_heads * c.head_dim;
  const CT *kk, *vv;
  int64_t ld_kv;
  if (c.own_kv) {
    KvWriteArgs<CT> a{};
    a.k_src = P + L.off_k; a.v_src = P + L.off_v; a.ld_src = L.ld_p;
    a.k_full = reinterpret_cast<CT*>(L.k_meta); a.v_full = reinterpret_cast<CT*>(L.v_meta);
    a.B = 1; a.T = M; a.n_kv_heads = c.n_kv_heads; a.head_dim = c.head_dim;
    HIP_TRY(launch_kv_write(a, s), "meta K/V write");
    kk = P + L.off_k; vv = P + L.off_v; ld_kv = L.ld_p;
    km = L.k_meta; vm = L.v_meta;
  } else {
    kk = static_cast<const CT*>(km); vv = static_cast<const CT*>(vm); ld_kv = kvw;
  }
  // meta rows attend causally among themselves: a global pass with no prefix
  STATUS_TRY(run_attention<CT>(c, P, L.ld_p, kk, vv, ld_kv, (int64_t)M * ld_kv, nullptr, nullptr, 0,
                               reinterpret_cast<CT*>(ws + wl.O), (int64_t)c.n_heads * c.head_dim, 1, M, 0, s));
  HIP_TRY(launch_selective_scan(scan_args<CT>(L, ws, wl, 1, M, nullptr, L.h_meta), s), "meta scan launch");
  STATUS_TRY(tail<CT>(L, ws, wl, M, L.y_meta, s));
  L.prepared = true;
  L.prep_kmeta = km; L.prep_vmeta = vm;
  return HYMBA_OK;
}

int32_t ensure_prepared(hymba_layer& L, const hymba_kv* kv, char* ws, const WsLayout& wl, hipStream_t s) {
  if (L.prepared && !L.cfg.own_kv && !L.producer && L.cfg.n_meta > 0 && kv &&
      (kv->k_meta != L.prep_kmeta || kv->v_meta != L.prep_vmeta))
    L.prepared = false;   // an unbound consumer was handed different meta K/V
  if (L.prepared) return HYMBA_OK;
  const bool prof = L.profiling;   // the one-off meta-prefix pass is not part of a call's stage timings
  L.profiling = false;
  const int32_t r = is_bf16(L.cfg) ? prepare_impl<half_t>(L, kv, ws, wl, s) : prepare_impl<float>(L, kv, ws, wl, s);
  L.profiling = prof;
  return r;
}

template <typename CT>
int32_t prefill_impl(hymba_layer& L, const void* x, int B, int T_, void* y, const hymba_kv* kv, float* state_out,
                     char* ws, const WsLayout& wl, hipStream_t s) {
  if (L.profiling) ++L.prof_calls;
  const hymba_layer_cfg& c = L.cfg;
  const int64_t rows = (int64_t)B * T_;
  const int64_t kvw = (int64_t)c.n_kv_heads * c.head_dim;
  STATUS_TRY(in_projection<CT>(L, x, rows, ws, wl, s));
  STATUS_TRY(apply_rope<CT>(L, ws, wl, rows, T_, c.n_meta, nullptr, s));   // real token t at M + t
  const CT* P = reinterpret_cast<const CT*>(ws + wl.P);
  const CT *k, *v;
  int64_t ld_kv, seq_stride;
  if (c.own_kv) {
    k = P + L.off_k; v = P + L.off_v; ld_kv = L.ld_p; seq_stride = (int64_t)T_ * L.ld_p;
    if (kv && (kv->k || kv->k_cache)) {
      StageTimer st(L, ST_KV, s);
      KvWriteArgs<CT> a{};
      a.k_src = P + L.off_k; a.v_src = P + L.off_v; a.ld_src = L.ld_p;
      a.k_full = static_cast<CT*>(kv->k); a.v_full = static_cast<CT*>(kv->v);
      a.k_cache = static_cast<CT*>(kv->k_cache); a.v_cache = static_cast<CT*>(kv->v_cache);
      a.cache_len = kv->cache_len;
      a.B = B; a.T = T_; a.n_kv_heads = c.n_kv_heads; a.head_dim = c.head_dim;
      HIP_TRY(launch_kv_write(a, s), "K/V write");
    }
  } else {
    k = static_cast<const CT*>(kv->k); v = static_cast<const CT*>(kv->v);
    ld_kv = kvw; seq_stride = (int64_t)T_ * kvw;
  }
  const void *km, *vm;
  meta_kv_of(L, kv, &km, &vm);
  // The SSM branch depends only on the projection: it runs on the layer's side stream beside
  // attention and W_O, and the epilogue waits for both (or, with overlap off, first on the call's
  // stream, so that every kernel runs alone).
  hipStream_t ss = s;
  if (L.overlap) {
    STATUS_TRY(ensure_side_stream(L));
    HIP_TRY(hipEventRecord(L.ev_fork, s), "fork event");
    HIP_TRY(hipStreamWaitEvent(L.side, L.ev_fork, 0), "fork wait");
    ss = L.side;
  }
  {
    StageTimer st(L, ST_SSM, ss);
    HIP_TRY(launch_selective_scan(scan_args<CT>(L, ws, wl, B, T_, L.h_meta, state_out), ss), "scan launch");
  }
  if (L.overlap) HIP_TRY(hipEventRecord(L.ev_join, ss), "join event");
  {
    StageTimer st(L, ST_ATTN, s);
    STATUS_TRY(run_attention<CT>(c, P, L.ld_p, k, v, ld_kv, seq_stride, static_cast<const CT*>(km),
                                 static_cast<const CT*>(vm), c.n_meta, reinterpret_cast<CT*>(ws + wl.O),
                                 (int64_t)c.n_heads * c.head_dim, B, T_, c.window, s));
  }
  STATUS_TRY(w_o_projection<CT>(L, ws, wl, rows, s));
  if (L.overlap) HIP_TRY(hipStreamWaitEvent(s, L.ev_join, 0), "join wait");
  return epilogue_and_out<CT>(L, ws, wl, rows, y, s);
}

template <typename CT>
int32_t decode_impl(hymba_layer& L, const void* x, const int64_t* pos, int B, void* y, const hymba_kv* kv,
                    float* state, char* ws, const WsLayout& wl, hipStream_t s) {
  if (L.profiling) ++L.prof_calls;
  const hymba_layer_cfg& c = L.cfg;
  STATUS_TRY(in_projection<CT>(L, x, B, ws, wl, s));
  STATUS_TRY(apply_rope<CT>(L, ws, wl, B, 1, c.n_meta, pos, s));   // the new token at M + pos[b]
  const CT* P = reinterpret_cast<const CT*>(ws + wl.P);
  if (c.own_kv) {
    StageTimer st(L, ST_KV, s);
    KvWriteArgs<CT> a{};
    a.k_src = P + L.off_k; a.v_src = P + L.off_v; a.ld_src = L.ld_p;
    a.k_cache = static_cast<CT*>(kv->k_cache); a.v_cache = static_cast<CT*>(kv->v_cache);
    a.cache_len = kv->cache_len; a.pos = pos;
    a.B = B; a.T = 1; a.n_kv_heads = c.n_kv_heads; a.head_dim = c.head_dim;
    HIP_TRY(launch_kv_write(a, s), "cache slot write");
  }
  const void *km, *vm;
  meta_kv_of(L, kv, &km, &vm);
  const int weff = c.window > 0 ? c.window : kv->cache_len;
  const int splits = decode_attn_splits(B, c.n_kv_heads, c.n_meta + std::min(weff, kv->cache_len), c.head_dim,
                                        static_cast<int>(sizeof(CT)));
  if (splits < 1) return fail(HYMBA_ERR_UNSUPPORTED, "decode key range too long for the split-K kernel");
  {
    StageTimer st(L, ST_ATTN, s);
    DecAttnArgs<CT> a{};
    a.q = P; a.ld_q = L.ld_p;
    a.k_meta = static_cast<const CT*>(km); a.v_meta = static_cast<const CT*>(vm);
    a.ld_meta = (int64_t)c.n_kv_heads * c.head_dim; a.n_meta = c.n_meta;
    a.k_cache = static_cast<const CT*>(kv->k_cache); a.v_cache = static_cast<const CT*>(kv->v_cache);
    a.cache_len = kv->cache_len; a.pos = pos;
    a.o = reinterpret_cast<CT*>(ws + wl.O); a.ld_o = (int64_t)c.n_heads * c.head_dim;
    a.part = reinterpret_cast<float*>(ws + wl.part);
    a.B = B; a.n_heads = c.n_heads; a.n_kv_heads = c.n_kv_heads; a.head_dim = c.head_dim;
    a.window = c.window; a.splits = splits;
    a.flags = L.flags;
    a.scale_log2 = kLog2e / std::sqrt(static_cast<float>(c.head_dim));
    HIP_TRY(launch_decode_attn(a, s), "decode attention launch");
  }
  {
    StageTimer tm(L, ST_SSM, s);
    StepArgs<CT> st{};
    st.u = P + L.off_u; st.dt = P + L.off_dt; st.ld = L.ld_p;
    if (is_bf16(c)) {
      st.bc = reinterpret_cast<const float*>(ws + wl.bc32); st.ld_bc = 2 * c.d_state;
    } else {
      st.bc = reinterpret_cast<const float*>(P + L.off_b); st.ld_bc = L.ld_p;
    }
    st.A2 = L.A2; st.D = L.w.D; st.dt_bias = L.w.dt_bias; st.h = state;
    st.y = reinterpret_cast<CT*>(ws + wl.Ys); st.ldy = c.d_inner;
    st.B = B; st.E = c.d_inner; st.N = c.d_state;
    HIP_TRY(launch_ssm_step(st, s), "SSM step launch");
  }
  return tail<CT>(L, ws, wl, B, y, s);
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The kernels move activations, K/V rows and states in 16-byte vectors, and the workspace is carved
// into 256-byte-aligned regions from its start.
int32_t check_kv_alignment(const hymba_kv* kv) {
  if (kv && (!aligned(kv->k_meta, 16) || !aligned(kv->v_meta, 16) || !aligned(kv->k, 16) || !aligned(kv->v, 16) ||
             !aligned(kv->k_cache, 16) || !aligned(kv->v_cache, 16)))
    return fail(HYMBA_ERR_INVALID_ARG, "the K/V pointers of kv must be 16-byte aligned");
  return HYMBA_OK;
}

int32_t check_decode_args(const hymba_layer& L, const void* x_t, const int64_t* pos, int32_t B, const void* y_t,
                          const hymba_kv* kv, const float* ssm_state) {
  if (!x_t || !y_t || !pos || !ssm_state)
    return fail(HYMBA_ERR_INVALID_ARG, "x_t, pos, y_t and ssm_state must be non-NULL");
  if (B < 1) return fail(HYMBA_ERR_INVALID_ARG, "B must be >= 1");
  if (B > 65535) return fail(HYMBA_ERR_UNSUPPORTED, "a decode step takes at most 65535 sequences (got %d)", B);
  if (!aligned(x_t, 16) || !aligned(y_t, 16) || !aligned(ssm_state, 16) || !aligned(pos, 8))
    return fail(HYMBA_ERR_INVALID_ARG, "x_t, y_t and ssm_state must be 16-byte aligned, pos 8-byte aligned");
  STATUS_TRY(check_kv_alignment(kv));
  if (!kv || !kv->k_cache || !kv->v_cache) return fail(HYMBA_ERR_INVALID_ARG, "decode needs kv->k_cache and kv->v_cache");
  const hymba_layer_cfg& c = L.cfg;
  if (kv->cache_len < 1) return fail(HYMBA_ERR_INVALID_ARG, "cache_len must be >= 1");
  if (c.window > 0 && kv->cache_len < c.window)
    return fail(HYMBA_ERR_INVALID_ARG, "a sliding-window cache needs cache_len >= window (%d < %d)", kv->cache_len,
                c.window);
  if (!c.own_kv && !L.producer && c.n_meta > 0 && (!kv->k_meta || !kv->v_meta))
    return fail(HYMBA_ERR_INVALID_ARG, "an unbound consumer needs kv->k_meta and kv->v_meta");
  return HYMBA_OK;
}

// ---- the allocation-free decode step ---------------------------------------------------------
// Scratch of hymba_mixer_decode_static: one array per device, in the library's code object.  Host
// code never passes `scratch` itself (its name is a host-side stand-in, not a device address); it
// takes the device address from hipGetSymbolAddress once per device and uses that.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_dev[kMaxDevices] = {};

int32_t static_scratch(char** out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(HYMBA_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "scratch symbol address");
    if (!p) return fail(HYMBA_ERR_HIP, "scratch symbol address is NULL");
    g_scratch_dev[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_dev[dev];
  return HYMBA_OK;
}

}  // namespace

extern "C" {

size_t hymba_layer_persistent_bytes(const hymba_layer_cfg* cfg) {
  if (check_cfg(cfg) != HYMBA_OK) return 0;
  return persist_layout(*cfg).total;
}

int32_t hymba_layer_create(const hymba_layer_cfg* cfg, const hymba_layer_weights* w, void* persistent,
                           size_t persistent_bytes, hymba_layer** out) {
  if (!out) return fail(HYMBA_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  STATUS_TRY(check_cfg(cfg));
  if (!w) return fail(HYMBA_ERR_INVALID_ARG, "weights is NULL");
  if (!w->w_in || !w->w_o || !w->w_out || !w->A || !w->D || !w->dt_bias || !w->beta1 || !w->beta2)
    return fail(HYMBA_ERR_INVALID_ARG, "a weight pointer is NULL");
  if (cfg->n_meta > 0 && !w->meta) return fail(HYMBA_ERR_INVALID_ARG, "meta rows pointer is NULL");
  if (!aligned(w->w_in, 16) || !aligned(w->w_o, 16) || !aligned(w->w_out, 16) || !aligned(w->meta, 16))
    return fail(HYMBA_ERR_INVALID_ARG, "weight matrices and meta rows must be 16-byte aligned");
  if (!persistent) return fail(HYMBA_ERR_INVALID_ARG, "persistent buffer is NULL");
  if (!aligned(persistent, kAlign)) return fail(HYMBA_ERR_INVALID_ARG, "persistent buffer must be 256-byte aligned");
  const PersistLayout pl = persist_layout(*cfg);
  if (persistent_bytes < pl.total)
    return fail(HYMBA_ERR_WORKSPACE, "persistent buffer has %zu bytes, needs %zu", persistent_bytes, pl.total);
  hymba_layer* L = new (std::nothrow) hymba_layer();
  if (!L) return fail(HYMBA_ERR_INVALID_ARG, "host allocation failed");
  L->cfg = *cfg;
  L->w = *w;
  char* base = static_cast<char*>(persistent);
  L->k_meta = base + pl.k_meta;
  L->v_meta = base + pl.v_meta;
  L->h_meta = reinterpret_cast<float*>(base + pl.h_meta);
  L->y_meta = base + pl.y_meta;
  L->A2 = reinterpret_cast<float*>(base + pl.A2);
  L->flags = reinterpret_cast<uint32_t*>(base + pl.flags);
  if (is_bf16(*cfg)) {
    L->w_in16 = reinterpret_cast<half_t*>(base + pl.w_in16);
    L->w_o16 = reinterpret_cast<half_t*>(base + pl.w_o16);
  }
  const int64_t q = (int64_t)cfg->n_heads * cfg->head_dim, kvw = (int64_t)cfg->n_kv_heads * cfg->head_dim;
  L->n_in = n_in_of(*cfg);
  // row stride of the projection P: whole 64-element (128-byte for fp16) segments, so the
  // per-channel column slices the scan and epilogue read start on cache-line boundaries
  L->ld_p = (L->n_in + 63) / 64 * 64;
  L->off_k = q;
  L->off_v = q + kvw;
  L->off_u = q + (cfg->own_kv ? 2 * kvw : 0);
  L->off_z = L->off_u + cfg->d_inner;
  L->off_dt = L->off_z + cfg->d_inner;
  L->off_b = L->off_dt + cfg->d_inner;
  *out = L;
  return HYMBA_OK;
}

void hymba_layer_destroy(hymba_layer* L) {
  if (!L) return;
  for (hipEvent_t e : L->ev) hipEventDestroy(e);
  if (L->side) {
    hipStreamDestroy(L->side);
    hipEventDestroy(L->ev_fork);
    hipEventDestroy(L->ev_join);
  }
  if (L->producer && L->producer->consumer == L) const_cast<hymba_layer*>(L->producer)->consumer = nullptr;
  if (L->consumer && L->consumer->producer == L) const_cast<hymba_layer*>(L->consumer)->producer = nullptr;
  delete L;
}

int32_t hymba_kv_share_bind(hymba_layer* consumer, const hymba_layer* producer) {
  if (!consumer) return fail(HYMBA_ERR_INVALID_ARG, "consumer is NULL");
  if (producer == consumer) return fail(HYMBA_ERR_BIND, "a layer cannot share K/V with itself");
  if (consumer->cfg.own_kv) return fail(HYMBA_ERR_BIND, "the consumer must be created with own_kv = 0");
  if (!producer) {
    if (consumer->producer) const_cast<hymba_layer*>(consumer->producer)->consumer = nullptr;
    consumer->producer = nullptr;
    consumer->prepared = false;
    return HYMBA_OK;
  }
  const hymba_layer_cfg &c = consumer->cfg, &p = producer->cfg;
  if (!p.own_kv) return fail(HYMBA_ERR_BIND, "the producer must own its K/V (own_kv = 1)");
  if (c.n_kv_heads != p.n_kv_heads || c.head_dim != p.head_dim || c.n_meta != p.n_meta || c.dtype != p.dtype)
    return fail(HYMBA_ERR_BIND, "producer and consumer differ in n_kv_heads, head_dim, n_meta or dtype");
  if ((c.window > 0) != (p.window > 0) || (c.window > 0 && c.window != p.window))
    return fail(HYMBA_ERR_BIND, "producer and consumer must have the same attention window");
  if (c.rope_base != p.rope_base)
    return fail(HYMBA_ERR_BIND, "producer and consumer must use the same rotary encoding base");
  if (producer->consumer && producer->consumer != consumer)
    return fail(HYMBA_ERR_BIND, "the producer already has a consumer (K/V are shared by pairs)");
  if (consumer->producer && consumer->producer != producer)
    const_cast<hymba_layer*>(consumer->producer)->consumer = nullptr;
  consumer->producer = producer;
  const_cast<hymba_layer*>(producer)->consumer = consumer;
  consumer->prepared = false;
  return HYMBA_OK;
}

size_t hymba_mixer_workspace_bytes(const hymba_layer* L, int32_t batch, int32_t seq) {
  if (!L || batch < 1 || seq < 1) return 0;
  return ws_layout(*L, batch, seq).total;
}

int32_t hymba_layer_prepare(hymba_layer* L, const hymba_kv* kv, void* ws, size_t ws_bytes, void* stream) {
  if (!L) return fail(HYMBA_ERR_INVALID_ARG, "layer is NULL");
  if (!ws) return fail(HYMBA_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned(ws, kAlign)) return fail(HYMBA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  STATUS_TRY(check_kv_alignment(kv));
  const WsLayout wl = ws_layout(*L, 1, 1);
  if (ws_bytes < wl.total) return fail(HYMBA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, wl.total);
  L->prepared = false;
  return ensure_prepared(*L, kv, static_cast<char*>(ws), wl, static_cast<hipStream_t>(stream));
}

int32_t hymba_mixer_prefill(hymba_layer* L, const void* x, int32_t B, int32_t T, void* y, const hymba_kv* kv,
                            float* ssm_state_out, void* ws, size_t ws_bytes, void* stream) {
  if (!L) return fail(HYMBA_ERR_INVALID_ARG, "layer is NULL");
  if (!x || !y || !ws) return fail(HYMBA_ERR_INVALID_ARG, "x, y and workspace must be non-NULL");
  if (B < 1 || T < 1) return fail(HYMBA_ERR_INVALID_ARG, "B and T must be >= 1 (got %d, %d)", B, T);
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ssm_state_out, 16))
    return fail(HYMBA_ERR_INVALID_ARG, "x, y and ssm_state_out must be 16-byte aligned");
  if (!aligned(ws, kAlign)) return fail(HYMBA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  STATUS_TRY(check_kv_alignment(kv));
  const hymba_layer_cfg& c = L->cfg;
  if (!c.own_kv) {
    if (!kv || !kv->k || !kv->v) return fail(HYMBA_ERR_INVALID_ARG, "a consumer needs kv->k and kv->v");
    if (!L->producer && c.n_meta > 0 && (!kv->k_meta || !kv->v_meta))
      return fail(HYMBA_ERR_INVALID_ARG, "an unbound consumer needs kv->k_meta and kv->v_meta");
  } else if (kv) {
    if ((kv->k != nullptr) != (kv->v != nullptr)) return fail(HYMBA_ERR_INVALID_ARG, "kv->k and kv->v go together");
    if ((kv->k_cache != nullptr) != (kv->v_cache != nullptr))
      return fail(HYMBA_ERR_INVALID_ARG, "kv->k_cache and kv->v_cache go together");
    if (kv->k_cache && kv->cache_len < 1) return fail(HYMBA_ERR_INVALID_ARG, "cache_len must be >= 1");
  }
  const WsLayout wl = ws_layout(*L, B, T);
  if (ws_bytes < wl.total) return fail(HYMBA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, wl.total);
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  STATUS_TRY(ensure_prepared(*L, kv, w, wl, s));
  return is_bf16(c) ? prefill_impl<half_t>(*L, x, B, T, y, kv, ssm_state_out, w, wl, s)
                    : prefill_impl<float>(*L, x, B, T, y, kv, ssm_state_out, w, wl, s);
}

int32_t hymba_mixer_decode(hymba_layer* L, const void* x_t, const int64_t* pos, int32_t B, void* y_t,
                           const hymba_kv* kv, float* ssm_state, void* ws, size_t ws_bytes, void* stream) {
  if (!L) return fail(HYMBA_ERR_INVALID_ARG, "layer is NULL");
  if (!ws) return fail(HYMBA_ERR_INVALID_ARG, "workspace must be non-NULL");
  if (!aligned(ws, kAlign)) return fail(HYMBA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  STATUS_TRY(check_decode_args(*L, x_t, pos, B, y_t, kv, ssm_state));
  const hymba_layer_cfg& c = L->cfg;
  const WsLayout wl = ws_layout(*L, B, 1);
  if (ws_bytes < wl.total) return fail(HYMBA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, wl.total);
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  STATUS_TRY(ensure_prepared(*L, kv, w, wl, s));
  return is_bf16(c) ? decode_impl<half_t>(*L, x_t, pos, B, y_t, kv, ssm_state, w, wl, s)
                    : decode_impl<float>(*L, x_t, pos, B, y_t, kv, ssm_state, w, wl, s);
}

int32_t hymba_mixer_decode_static(hymba_layer* L, const void* x_t, const int64_t* pos, int32_t B, void* y_t,
                                  const hymba_kv* kv, float* ssm_state, void* stream) {
  if (!L) return fail(HYMBA_ERR_INVALID_ARG, "layer is NULL");
  STATUS_TRY(check_decode_args(*L, x_t, pos, B, y_t, kv, ssm_state));
  const hymba_layer_cfg& c = L->cfg;
  if (!L->prepared || (!c.own_kv && !L->producer && c.n_meta > 0 &&
                       (kv->k_meta != L->prep_kmeta || kv->v_meta != L->prep_vmeta)))
    return fail(HYMBA_ERR_INVALID_ARG, "the allocation-free decode needs the layer prepared (hymba_layer_prepare) "
                                       "with the meta K/V it is handed");
  const int weff = c.window > 0 ? c.window : kv->cache_len;
  const int splits = decode_attn_splits(B, c.n_kv_heads, c.n_meta + std::min(weff, kv->cache_len), c.head_dim,
                                        static_cast<int>(act_size(c)));
  if (splits < 1) return fail(HYMBA_ERR_UNSUPPORTED, "decode key range too long for the split-K kernel");
  const WsLayout wl = ws_layout_own_kernels(*L, B, splits);
  if (wl.total > kStaticScratchBytes)
    return fail(HYMBA_ERR_WORKSPACE, "the allocation-free decode needs %zu bytes of scratch, at most %zu are "
                "available (fewer sequences per call fit)", wl.total, kStaticScratchBytes);
  char* w = nullptr;
  STATUS_TRY(static_scratch(&w));
  hipStream_t s = static_cast<hipStream_t>(stream);
  return is_bf16(c) ? decode_impl<half_t>(*L, x_t, pos, B, y_t, kv, ssm_state, w, wl, s)
                    : decode_impl<float>(*L, x_t, pos, B, y_t, kv, ssm_state, w, wl, s);
}

int32_t hymba_layer_meta_outputs(const hymba_layer* L, const void** k_meta, const void** v_meta,
                                 const float** h_meta, const void** y_meta) {
  if (!L) return fail(HYMBA_ERR_INVALID_ARG, "layer is NULL");
  if (!L->prepared) return fail(HYMBA_ERR_INVALID_ARG, "layer is not prepared");
  if (k_meta) *k_meta = L->cfg.own_kv ? L->k_meta : nullptr;
  if (v_meta) *v_meta = L->cfg.own_kv ? L->v_meta : nullptr;
  if (h_meta) *h_meta = L->h_meta;
  if (y_meta) *y_meta = L->y_meta;
  return HYMBA_OK;
}

int32_t hymba_layer_check(hymba_layer* L, void* stream) {
  if (!L) return fail(HYMBA_ERR_INVALID_ARG, "layer is NULL");
  if (!L->weights_ready) return HYMBA_OK;   // nothing has run on the device yet
  HIP_TRY(hipStreamSynchronize(static_cast<hipStream_t>(stream)), "stream synchronize");
  uint32_t f[3] = {0u, 0u, 0u};
  HIP_TRY(hipMemcpy(f, L->flags, sizeof(f), hipMemcpyDeviceToHost), "check flags read");
  if (f[0] == 0u && f[1] == 0u && f[2] == 0u) return HYMBA_OK;
  const uint32_t zero[2] = {0u, 0u};   // the weight record stays: the weights do not change
  HIP_TRY(hipMemcpy(L->flags, zero, sizeof(zero), hipMemcpyHostToDevice), "check flags clear");
  if (f[2])
    return fail(HYMBA_ERR_RANGE, "a weight of W_in or W_O is beyond fp16's range (|w| > 65504): bf16 layers compute "
                                 "with fp16 copies of these weights%s",
                f[0] ? "; a branch output was not finite" : "");
  if (f[0])
    return fail(HYMBA_ERR_RANGE, "a row's attention or SSM branch output was not finite: an activation left the "
                                 "range of the activation type (fp16 for bf16 layers: |value| > 65504) or the input "
                                 "held inf/NaN%s", f[1] ? "; also a decode position was negative" : "");
  return fail(HYMBA_ERR_RANGE, "a decode position was negative");
}

int32_t hymba_layer_set_overlap(hymba_layer* L, int32_t enable) {
  if (!L) return fail(HYMBA_ERR_INVALID_ARG, "layer is NULL");
  L->overlap = enable != 0;
  return HYMBA_OK;
}

int32_t hymba_layer_set_gemm(hymba_layer* layer, int32_t backend) {
  if (!layer) return fail(HYMBA_ERR_INVALID_ARG, "NULL layer");
  if (backend != HYMBA_GEMM_LIBRARY && backend != HYMBA_GEMM_TILED)
    return fail(HYMBA_ERR_INVALID_ARG, "backend must be HYMBA_GEMM_LIBRARY or HYMBA_GEMM_TILED");
  layer->gemm_backend = backend;
  return HYMBA_OK;
}

int32_t hymba_layer_profile(hymba_layer* L, int32_t enable) {
  if (!L) return fail(HYMBA_ERR_INVALID_ARG, "layer is NULL");
  if (!enable) {
    L->profiling = false;
    return HYMBA_OK;
  }
  if (L->ev.empty()) {
    L->ev.assign(2 * kProfPairs, nullptr);
    L->ev_stage.assign(kProfPairs, 0);
    for (hipEvent_t& e : L->ev) {
      const hipError_t r = hipEventCreate(&e);
      if (r != hipSuccess) {
        for (hipEvent_t& f : L->ev)
          if (f) hipEventDestroy(f);
        L->ev.clear();
        return hip_fail(r, "event create");
      }
    }
  }
  L->profiling = true;
  L->ev_next = 0;
  L->prof_calls = 0;
  L->prof_overflow = false;
  return HYMBA_OK;
}

int32_t hymba_layer_profile_read(hymba_layer* L, float* stage_ms, int32_t n) {
  if (!L || !stage_ms || n < 0) return fail(HYMBA_ERR_INVALID_ARG, "bad arguments");
  for (int i = 0; i < n; ++i) stage_ms[i] = 0.f;
  if (L->prof_overflow)
    return fail(HYMBA_ERR_WORKSPACE, "more than %d timed intervals since profiling was enabled", kProfPairs);
  double sum[HYMBA_N_STAGES] = {};
  if (L->ev_next > 0) HIP_TRY(hipEventSynchronize(L->ev[2 * L->ev_next - 1]), "event synchronize");
  for (int p = 0; p < L->ev_next; ++p) {
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, L->ev[2 * p], L->ev[2 * p + 1]), "event elapsed time");
    sum[L->ev_stage[p]] += ms;
  }
  const int calls = L->prof_calls > 0 ? L->prof_calls : 1;
  for (int i = 0; i < n && i < HYMBA_N_STAGES; ++i) stage_ms[i] = static_cast<float>(sum[i] / calls);
  return HYMBA_OK;
}

const char* hymba_stage_name(int32_t stage) {
  return (stage >= 0 && stage < HYMBA_N_STAGES) ? kStageNames[stage] : "unknown";
}

const char* hymba_last_error(void) { return g_err.c_str(); }

const char* hymba_status_string(int32_t status) {
  switch (status) {
    case HYMBA_OK: return "HYMBA_OK";
    case HYMBA_ERR_INVALID_ARG: return "HYMBA_ERR_INVALID_ARG";
    case HYMBA_ERR_UNSUPPORTED: return "HYMBA_ERR_UNSUPPORTED";
    case HYMBA_ERR_WORKSPACE: return "HYMBA_ERR_WORKSPACE";
    case HYMBA_ERR_BIND: return "HYMBA_ERR_BIND";
    case HYMBA_ERR_HIP: return "HYMBA_ERR_HIP";
    case HYMBA_ERR_RANGE: return "HYMBA_ERR_RANGE";
    default: return "HYMBA_UNKNOWN_STATUS";
  }
}

int32_t hymba_kernel_attention(int32_t dtype, const void* q, int64_t ld_q, const void* k, const void* v,
                               int64_t ld_kv, int64_t kv_seq_stride, const void* k_meta, const void* v_meta,
                               int32_t n_meta, void* o, int64_t ld_o, int32_t B, int32_t T, int32_t n_heads,
                               int32_t n_kv_heads, int32_t head_dim, int32_t window, void* stream) {
  if (!q || !k || !v || !o || (n_meta > 0 && (!k_meta || !v_meta)))
    return fail(HYMBA_ERR_INVALID_ARG, "NULL pointer");
  if (B < 1 || T < 1 || n_meta < 0 || n_heads < 1 || n_kv_heads < 1 || n_heads % n_kv_heads)
    return fail(HYMBA_ERR_INVALID_ARG, "bad dimensions");
  hymba_layer_cfg c{};
  c.n_heads = n_heads; c.n_kv_heads = n_kv_heads; c.head_dim = head_dim;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == HYMBA_BF16)
    return fail(HYMBA_ERR_UNSUPPORTED, "16-bit attention runs on fp16 operands (HYMBA_F16): bf16 probabilities "
                                       "would round the P.V operand to 8 significand bits");
  if (dtype == HYMBA_F16) {
    if (!attn_mfma_supported(head_dim, n_heads, n_kv_heads, n_meta))
      return fail(HYMBA_ERR_UNSUPPORTED, "16-bit attention shape not supported");
    // 16-byte rows for the vector loads; row offsets within a 64-key tile fit 32 bits
    const int64_t hq = (int64_t)n_heads * head_dim, hkv = (int64_t)n_kv_heads * head_dim;
    if (ld_q < hq || ld_o < hq || ld_kv < hkv || ld_q % 8 || ld_o % 8 || ld_kv % 8 || kv_seq_stride % 8 ||
        ld_kv >= (1 << 24) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        (n_meta > 0 && (!aligned(k_meta, 16) || !aligned(v_meta, 16))))
      return fail(HYMBA_ERR_INVALID_ARG, "strides: rows >= heads * hd, multiples of 8 elements, 16-byte aligned");
    return run_attention<half_t>(c, static_cast<const half_t*>(q), ld_q, static_cast<const half_t*>(k),
                                 static_cast<const half_t*>(v), ld_kv, kv_seq_stride,
                                 static_cast<const half_t*>(k_meta), static_cast<const half_t*>(v_meta), n_meta,
                                 static_cast<half_t*>(o), ld_o, B, T, window, s);
  }
  if (dtype != HYMBA_F32) return fail(HYMBA_ERR_INVALID_ARG, "bad dtype");
  if (head_dim != 32 && head_dim != 64) return fail(HYMBA_ERR_UNSUPPORTED, "fp32 attention head_dim");
  return run_attention<float>(c, static_cast<const float*>(q), ld_q, static_cast<const float*>(k),
                              static_cast<const float*>(v), ld_kv, kv_seq_stride, static_cast<const float*>(k_meta),
                              static_cast<const float*>(v_meta), n_meta, static_cast<float*>(o), ld_o, B, T, window,
                              s);
}

int32_t hymba_kernel_selective_scan(int32_t dtype, const void* u, const void* dt, int64_t ld, const float* bc,
                                    int64_t ld_bc, const float* A, const float* D, const float* dt_bias,
                                    const float* h0, void* y, int64_t ldy, float* h_out, int32_t B, int32_t T,
                                    int32_t E, int32_t N, void* ws, size_t ws_bytes, void* stream) {
  if (!u || !dt || !bc || !A || !D || !dt_bias || !y || !ws) return fail(HYMBA_ERR_INVALID_ARG, "NULL pointer");
  if (B < 1 || T < 1 || E < 1) return fail(HYMBA_ERR_INVALID_ARG, "bad dimensions");
  if (N != 8 && N != 16) return fail(HYMBA_ERR_UNSUPPORTED, "N must be 8 or 16");
  if (ld < E || ldy < E || ld_bc < 2 * N || ld_bc % 4 != 0 || !aligned(bc, 16))
    return fail(HYMBA_ERR_INVALID_ARG, "strides: ld, ldy >= E; ld_bc >= 2N, a multiple of 4, bc 16-byte aligned");
  if (dtype != HYMBA_F16 && dtype != HYMBA_F32)
    return fail(HYMBA_ERR_INVALID_ARG, "scan dtype must be HYMBA_F32 or HYMBA_F16");
  if (ws_bytes < (size_t)E * N * 4) return fail(HYMBA_ERR_WORKSPACE, "workspace too small");
  if (B > 65535) return fail(HYMBA_ERR_UNSUPPORTED, "at most 65535 sequences per call");
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* A2 = static_cast<float*>(ws);
  // beyond the scaled A: room for the time-segment summaries, if the caller gave it
  const size_t a2_bytes = align_up((size_t)E * N * 4);
  float* seg = ws_bytes > a2_bytes ? reinterpret_cast<float*>(static_cast<char*>(ws) + a2_bytes) : nullptr;
  const size_t seg_bytes = seg ? ws_bytes - a2_bytes : 0;
  HIP_TRY(launch_scale_copy(A, A2, (int64_t)E * N, kLog2e, s), "A scaling");
  if (dtype == HYMBA_F16) {
    ScanArgs<half_t> a{static_cast<const half_t*>(u), static_cast<const half_t*>(dt), ld, bc, ld_bc, A2, D,
                       dt_bias, h0, 0, static_cast<half_t*>(y), ldy, h_out, B, T, E, N, seg, seg_bytes};
    HIP_TRY(launch_selective_scan(a, s), "scan launch");
  } else if (dtype == HYMBA_F32) {
    ScanArgs<float> a{static_cast<const float*>(u), static_cast<const float*>(dt), ld, bc, ld_bc, A2, D, dt_bias,
                      h0, 0, static_cast<float*>(y), ldy, h_out, B, T, E, N, seg, seg_bytes};
    HIP_TRY(launch_selective_scan(a, s), "scan launch");
  } else {
    return fail(HYMBA_ERR_INVALID_ARG, "scan dtype must be HYMBA_F32 or HYMBA_F16");
  }
  return HYMBA_OK;
}

int32_t hymba_kernel_epilogue(int32_t dtype, const void* ao, int64_t ld_ao, const void* y, int64_t ld_y,
                              const void* z, int64_t ld_z, const float* beta1, const float* beta2, void* f,
                              int64_t ld_f, int64_t rows, int32_t E, float eps, void* stream) {
  if (!ao || !y || !z || !beta1 || !beta2 || !f) return fail(HYMBA_ERR_INVALID_ARG, "NULL pointer");
  if (rows < 0 || E < 1) return fail(HYMBA_ERR_INVALID_ARG, "bad dimensions");
  if (E % 8) return fail(HYMBA_ERR_UNSUPPORTED, "E must be a multiple of 8");
  const int64_t vw = dtype == HYMBA_F32 ? 4 : 8;
  if (ld_ao < E || ld_y < E || ld_z < E || ld_f < E || ld_ao % vw || ld_y % vw || ld_z % vw || ld_f % vw ||
      !aligned(ao, 16) || !aligned(y, 16) || !aligned(z, 16) || !aligned(f, 16))
    return fail(HYMBA_ERR_INVALID_ARG, "strides: >= E, whole 16-byte chunks, 16-byte aligned rows");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == HYMBA_F16) {
    EpiArgs<half_t, bf16_t> a{static_cast<const half_t*>(ao), ld_ao, static_cast<const half_t*>(y), ld_y,
                              static_cast<const half_t*>(z), ld_z, beta1, beta2, static_cast<bf16_t*>(f), ld_f,
                              rows, E, eps};
    HIP_TRY(launch_epilogue(a, s), "epilogue launch");
  } else if (dtype == HYMBA_F32) {
    EpiArgs<float> a{static_cast<const float*>(ao), ld_ao, static_cast<const float*>(y), ld_y,
                     static_cast<const float*>(z), ld_z, beta1, beta2, static_cast<float*>(f), ld_f, rows, E, eps};
    HIP_TRY(launch_epilogue(a, s), "epilogue launch");
  } else {
    return fail(HYMBA_ERR_INVALID_ARG, "epilogue dtype must be HYMBA_F32 or HYMBA_F16");
  }
  return HYMBA_OK;
}

size_t hymba_kernel_selective_scan_workspace(int32_t B, int32_t T, int32_t E, int32_t N) {
  if (B < 1 || T < 1 || E < 1 || (N != 8 && N != 16)) return 0;
  return align_up((size_t)E * N * 4) + scan_segment_bytes(B, T, E, N);
}

int32_t hymba_kernel_gemm_tiles(int32_t in_dtype, int32_t y_dtype, const void* w, int64_t ldw, const void* x,
                                int64_t ldx, void* y, int64_t ldy, float* y32, int64_t ldy32, int32_t c0, int32_t c1,
                                int64_t M, int32_t N, int32_t K, void* stream) {
  if (!w || !x || !y) return fail(HYMBA_ERR_INVALID_ARG, "NULL pointer");
  if (M < 0 || N < 1 || K < 1) return fail(HYMBA_ERR_INVALID_ARG, "bad dimensions");
  if ((in_dtype != HYMBA_F16 && in_dtype != HYMBA_BF16) || (y_dtype != HYMBA_F16 && y_dtype != HYMBA_BF16))
    return fail(HYMBA_ERR_UNSUPPORTED, "types: x and w HYMBA_F16 or HYMBA_BF16, y HYMBA_F16 or HYMBA_BF16");
  if (N % 4 || K % 8) return fail(HYMBA_ERR_UNSUPPORTED, "N must be a multiple of 4 and K of 8");
  MfmaGemmArgs a{x, ldx, w, ldw, y, ldy, y32, ldy32, c0, c1, M, N, K};
  if (!mfma_gemm_shape_ok(a))
    return fail(HYMBA_ERR_INVALID_ARG, "strides: ldw, ldx >= K, multiples of 8 (16-byte aligned x, w); ldy >= N, "
                                       "a multiple of 4 (8-byte aligned y); y32: 0 <= c0 <= c1 <= N multiples of 4, "
                                       "ldy32 >= c1 - c0 (of 4), 16-byte aligned");
  if (M == 0) return HYMBA_OK;
  const int ti = in_dtype == HYMBA_BF16 ? GT_BF16 : GT_F16, to = y_dtype == HYMBA_BF16 ? GT_BF16 : GT_F16;
  HIP_TRY(launch_mfma_gemm(a, ti, to, static_cast<hipStream_t>(stream)), "tiled GEMM launch");
  return HYMBA_OK;
}

size_t hymba_kernel_gemm_rows_workspace(int32_t M, int32_t N, int32_t K) {
  (void)M; (void)N; (void)K;
  return 0;   // the kernel never splits K across workgroups
}

int32_t hymba_kernel_gemm_rows(int32_t w_dtype, int32_t x_dtype, int32_t y_dtype, const void* w, int64_t ldw,
                               const void* x, int64_t ldx, void* y, int64_t ldy, float* y32, int64_t ldy32,
                               int32_t c0, int32_t c1, int32_t M, int32_t N, int32_t K, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (!w || !x || !y) return fail(HYMBA_ERR_INVALID_ARG, "NULL pointer");
  if (M < 0 || N < 1 || K < 1) return fail(HYMBA_ERR_INVALID_ARG, "bad dimensions");
  if (N % 4 || K % 8) return fail(HYMBA_ERR_UNSUPPORTED, "N must be a multiple of 4 and K of 8");
  if (ldw < K || ldx < K || ldy < N || ldw % 8 || ldx % 8 || ldy % 4 || !aligned(w, 16) || !aligned(x, 16) ||
      !aligned(y, 16))
    return fail(HYMBA_ERR_INVALID_ARG, "strides: ldw, ldx >= K, multiples of 8; ldy >= N, a multiple of 4; "
                                       "16-byte aligned pointers");
  if (y32 && (c0 < 0 || c1 > N || c0 > c1 || c0 % 4 || c1 % 4 || ldy32 < c1 - c0 || ldy32 % 4 || !aligned(y32, 16)))
    return fail(HYMBA_ERR_INVALID_ARG, "y32: 0 <= c0 <= c1 <= N multiples of 4, ldy32 >= c1 - c0 (of 4), aligned");
  if (M == 0) return HYMBA_OK;
  (void)workspace; (void)workspace_bytes;   // none needed (hymba_kernel_gemm_rows_workspace is 0)
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (w_dtype == HYMBA_F16 && x_dtype == HYMBA_F16 && y_dtype == HYMBA_F16) {
    SkinnyArgs<half_t, half_t, half_t> a{static_cast<const half_t*>(w), ldw, static_cast<const half_t*>(x), ldx,
                                         static_cast<half_t*>(y), ldy, y32, ldy32, c0, c1, M, N, K};
    e = launch_skinny_gemm(a, s);
  } else if (w_dtype == HYMBA_F16 && x_dtype == HYMBA_BF16 && y_dtype == HYMBA_F16) {
    SkinnyArgs<half_t, bf16_t, half_t> a{static_cast<const half_t*>(w), ldw, static_cast<const bf16_t*>(x), ldx,
                                         static_cast<half_t*>(y), ldy, y32, ldy32, c0, c1, M, N, K};
    e = launch_skinny_gemm(a, s);
  } else if (w_dtype == HYMBA_F16 && x_dtype == HYMBA_F16 && y_dtype == HYMBA_BF16) {
    SkinnyArgs<half_t, half_t, bf16_t> a{static_cast<const half_t*>(w), ldw, static_cast<const half_t*>(x), ldx,
                                         static_cast<bf16_t*>(y), ldy, y32, ldy32, c0, c1, M, N, K};
    e = launch_skinny_gemm(a, s);
  } else if (w_dtype == HYMBA_BF16 && x_dtype == HYMBA_BF16 && y_dtype == HYMBA_BF16) {
    SkinnyArgs<bf16_t, bf16_t, bf16_t> a{static_cast<const bf16_t*>(w), ldw, static_cast<const bf16_t*>(x), ldx,
                                         static_cast<bf16_t*>(y), ldy, y32, ldy32, c0, c1, M, N, K};
    e = launch_skinny_gemm(a, s);
  } else {
    return fail(HYMBA_ERR_UNSUPPORTED, "unsupported (w, x, y) type combination");
  }
  HIP_TRY(e, "few-row GEMM launch");
  return HYMBA_OK;
}

}  // extern "C"
