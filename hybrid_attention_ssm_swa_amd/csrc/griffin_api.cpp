// C ABI of the Griffin recurrent block: validation, workspace carving and the
// launch sequence in_proj GEMM -> conv -> gate GEMM -> RG-LRU (+ GeLU branch)
// -> out_proj GEMM.  bf16 blocks convert x to fp16, run their GEMMs through
// hipBLASLt on fp16 operands (fp16 output, fp32 accumulation) against the fp16
// weight copies of the persistent buffer, and convert y back to bf16; fp32
// blocks run the library's fp32 GEMM kernel.
#include "griffin_block.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "errors.h"
#include "gemm_blaslt.h"
#include "kernels.h"

using namespace hymba;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

#define G_HIP_TRY(expr, what)                                                                   \
  do {                                                                                          \
    hipError_t e_ = (expr);                                                                     \
    if (e_ != hipSuccess) return set_error(HYMBA_ERR_HIP, "%s: %s", what, hipGetErrorString(e_)); \
  } while (0)

#define G_STATUS_TRY(expr)          \
  do {                              \
    int32_t s_ = (expr);            \
    if (s_ != HYMBA_OK) return s_;  \
  } while (0)

bool is_bf16(const griffin_block_cfg& c) { return c.dtype == HYMBA_BF16; }
size_t elem(const griffin_block_cfg& c) { return is_bf16(c) ? 2 : 4; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// few rows: all three projections on the weight-streaming kernel (x read in bf16, y written in
// bf16 by it); else the library GEMMs with the x and y conversions
bool few_rows(const griffin_block_cfg& c, int64_t rows) {
  const int64_t R = c.d_rnn, D = c.d_model;
  return skinny_fits(rows, 2 * R, D) && skinny_fits(rows, 2 * R, R) && skinny_fits(rows, D, R);
}

int32_t check_cfg(const griffin_block_cfg* c) {
  if (!c) return set_error(HYMBA_ERR_INVALID_ARG, "cfg is NULL");
  if (c->d_model <= 0 || c->d_rnn <= 0) return set_error(HYMBA_ERR_INVALID_ARG, "d_model and d_rnn must be positive");
  if (c->dtype != HYMBA_F32 && c->dtype != HYMBA_BF16)
    return set_error(HYMBA_ERR_INVALID_ARG, "dtype must be HYMBA_F32 or HYMBA_BF16");
  if (!std::isfinite(c->c) || c->c <= 0.f) return set_error(HYMBA_ERR_INVALID_ARG, "c must be finite and > 0");
  if (c->d_model % 8 || c->d_rnn % 8)
    return set_error(HYMBA_ERR_UNSUPPORTED, "d_model and d_rnn must be multiples of 8");
  return HYMBA_OK;
}

struct Ws {
  size_t x16 = 0, uv = 0, xc = 0, g = 0, hy = 0, gemm = 0, total = 0;
};

// x16 (bf16 blocks: x in fp16, later y in fp16) | uv | xc | g | hy | GEMM workspace
Ws layout(const griffin_block_cfg& c, int B, int T) {
  Ws w;
  const size_t rows = static_cast<size_t>(B) * T, R = c.d_rnn, D = c.d_model, e = elem(c);
  size_t o = 0;
  w.x16 = o;  o += is_bf16(c) ? align_up(rows * D * 2) : 0;
  w.uv = o;   o += align_up(rows * 2 * R * e);
  w.xc = o;   o += align_up(rows * R * e);
  w.g = o;    o += align_up(rows * 2 * R * e);
  w.hy = o;   o += align_up(rows * R * e);
  w.gemm = o; o += is_bf16(c) ? kGemmWorkspaceBytes : 0;
  w.total = o;
  return w;
}

// fp16 weight copies of a bf16 block
struct Persist {
  size_t w_in = 0, w_gate = 0, w_out = 0, total = 0;
};

Persist persist_layout(const griffin_block_cfg& c) {
  Persist p;
  if (!is_bf16(c)) return p;
  const size_t R = c.d_rnn, D = c.d_model;
  size_t o = 0;
  p.w_in = o;   o += align_up(2 * R * D * 2);
  p.w_gate = o; o += align_up(2 * R * R * 2);
  p.w_out = o;  o += align_up(D * R * 2);
  p.total = o;
  return p;
}

// Y[rows, out] = X[rows, in] . W[out, in]^T; bf16 blocks: fp16 X and W, output fp16 (or bf16 with
// bf16_out, few rows only)
int32_t project(const griffin_block_cfg& c, const void* X, const void* W, void* Y, int64_t rows, int64_t out,
                int64_t in, char* ws, const Ws& wl, hipStream_t s, bool bf16_out = false) {
  if (is_bf16(c) && few_rows(c, rows)) {   // few rows (decode): the weight-streaming kernel
    hipError_t e;
    if (bf16_out) {
      SkinnyArgs<half_t, half_t, bf16_t> a{static_cast<const half_t*>(W), in, static_cast<const half_t*>(X), in,
                                           static_cast<bf16_t*>(Y), out, nullptr, 0, 0, 0, static_cast<int>(rows),
                                           static_cast<int>(out), static_cast<int>(in)};
      e = launch_skinny_gemm(a, s);
    } else {
      SkinnyArgs<half_t, half_t, half_t> a{static_cast<const half_t*>(W), in, static_cast<const half_t*>(X), in,
                                           static_cast<half_t*>(Y), out, nullptr, 0, 0, 0, static_cast<int>(rows),
                                           static_cast<int>(out), static_cast<int>(in)};
      e = launch_skinny_gemm(a, s);
    }
    G_HIP_TRY(e, "Griffin projection (few rows) launch");
    return HYMBA_OK;
  }
  if (is_bf16(c)) {
    const char* err = nullptr;
    const int r = gemm_16(GT_F16, GT_F16, X, in, W, in, Y, out, rows, out, in, ws + wl.gemm, kGemmWorkspaceBytes,
                          s, &err);
    if (r != 0) return set_error(r == -2 ? HYMBA_ERR_UNSUPPORTED : HYMBA_ERR_HIP, "Griffin projection GEMM: %s", err);
    return HYMBA_OK;
  }
  G_HIP_TRY(launch_gemm_f32(static_cast<const float*>(X), in, static_cast<const float*>(W), in, static_cast<float*>(Y),
                            out, rows, static_cast<int>(out), static_cast<int>(in), s),
            "fp32 Griffin projection GEMM launch");
  return HYMBA_OK;
}

enum { GS_IN = 0, GS_CONV = 1, GS_GATE = 2, GS_RGLRU = 3, GS_OUT = 4 };

struct Timer {   // stage events of a measured call
  hipEvent_t ev[GRIFFIN_N_STAGES + 1] = {};
  bool on = false;
  ~Timer() {
    for (auto& e : ev)
      if (e) hipEventDestroy(e);
  }
  int32_t start(hipStream_t s) {
    for (auto& e : ev) G_HIP_TRY(hipEventCreate(&e), "hipEventCreate");
    on = true;
    G_HIP_TRY(hipEventRecord(ev[0], s), "hipEventRecord");
    return HYMBA_OK;
  }
  int32_t mark(int stage, hipStream_t s) {
    if (on) G_HIP_TRY(hipEventRecord(ev[stage + 1], s), "hipEventRecord");
    return HYMBA_OK;
  }
  int32_t finish(float* ms) {
    G_HIP_TRY(hipEventSynchronize(ev[GRIFFIN_N_STAGES]), "hipEventSynchronize");
    for (int i = 0; i < GRIFFIN_N_STAGES; ++i)
      G_HIP_TRY(hipEventElapsedTime(&ms[i], ev[i], ev[i + 1]), "hipEventElapsedTime");
    return HYMBA_OK;
  }
};

// The stages on activations of type ET (fp32, or fp16 in a bf16 block); X/Y are the block's input
// and output in ET, W* the weight matrices in ET.
template <typename ET>
int32_t run(const griffin_block_cfg& c, const griffin_block_weights& w, const void* W_in, const void* W_gate,
            const void* W_out, const void* X, int B, int T, void* Y, const float* conv_state, const float* h,
            float* conv_state_out, float* h_out, char* ws, const Ws& wl, hipStream_t s, Timer& tm,
            bool projected = false) {
  const int64_t rows = static_cast<int64_t>(B) * T, R = c.d_rnn, D = c.d_model;
  ET* uv = reinterpret_cast<ET*>(ws + wl.uv);
  ET* xc = reinterpret_cast<ET*>(ws + wl.xc);
  ET* g = reinterpret_cast<ET*>(ws + wl.g);
  ET* hy = reinterpret_cast<ET*>(ws + wl.hy);
  // projected: the input projection has run already (uv written) and Y takes the block's bf16 y
  if (!projected) G_STATUS_TRY(project(c, X, W_in, uv, rows, 2 * R, D, ws, wl, s));
  G_STATUS_TRY(tm.mark(GS_IN, s));
  GriffinConvArgs<ET> ca{uv, 2 * R, w.conv_w, conv_state, conv_state_out, xc, R, B, T, c.d_rnn};
  G_HIP_TRY(launch_griffin_conv(ca, s), "Griffin conv launch");
  G_STATUS_TRY(tm.mark(GS_CONV, s));
  G_STATUS_TRY(project(c, xc, W_gate, g, rows, 2 * R, R, ws, wl, s));
  G_STATUS_TRY(tm.mark(GS_GATE, s));
  RglruArgs<ET> ra{g, 2 * R, xc, R, uv + R, 2 * R, hy, R, w.lam, c.c, h, h_out, B, T, c.d_rnn};
  G_HIP_TRY(launch_rglru(ra, s), "RG-LRU launch");
  G_STATUS_TRY(tm.mark(GS_RGLRU, s));
  G_STATUS_TRY(project(c, hy, W_out, Y, rows, D, R, ws, wl, s, projected));
  return HYMBA_OK;
}

int32_t forward(const griffin_block_cfg& c, const griffin_block_weights& w, const void* persistent, const void* x,
                int B, int T, void* y, const float* conv_state, const float* h, float* conv_state_out, float* h_out,
                char* ws, const Ws& wl, hipStream_t s, float* stage_ms) {
  Timer tm;
  if (stage_ms) G_STATUS_TRY(tm.start(s));
  const int64_t rows = static_cast<int64_t>(B) * T, D = c.d_model;
  if (is_bf16(c) && few_rows(c, rows)) {
    // few rows: the input projection reads x in bf16 and the output projection writes y in bf16
    const Persist pl = persist_layout(c);
    const char* pw = static_cast<const char*>(persistent);
    const int64_t R = c.d_rnn;
    half_t* uv = reinterpret_cast<half_t*>(ws + wl.uv);
    SkinnyArgs<half_t, bf16_t, half_t> in{reinterpret_cast<const half_t*>(pw + pl.w_in), D,
                                          static_cast<const bf16_t*>(x), D, uv, 2 * R, nullptr, 0, 0, 0,
                                          static_cast<int>(rows), static_cast<int>(2 * R), static_cast<int>(D)};
    G_HIP_TRY(launch_skinny_gemm(in, s),
              "Griffin input projection (few rows) launch");
    G_STATUS_TRY(run<half_t>(c, w, nullptr, pw + pl.w_gate, pw + pl.w_out, nullptr, B, T, y, conv_state, h,
                             conv_state_out, h_out, ws, wl, s, tm, true));
  } else if (is_bf16(c)) {
    const Persist pl = persist_layout(c);
    const char* pw = static_cast<const char*>(persistent);
    half_t* x16 = reinterpret_cast<half_t*>(ws + wl.x16);
    G_HIP_TRY(launch_convert(static_cast<const bf16_t*>(x), D, x16, D, rows, D, s), "x conversion launch");
    // the fp16 y reuses x16 (x is consumed by the input projection)
    G_STATUS_TRY(run<half_t>(c, w, pw + pl.w_in, pw + pl.w_gate, pw + pl.w_out, x16, B, T, x16, conv_state, h,
                             conv_state_out, h_out, ws, wl, s, tm));
    G_HIP_TRY(launch_convert(x16, D, static_cast<bf16_t*>(y), D, rows, D, s), "y conversion launch");
  } else {
    G_STATUS_TRY(run<float>(c, w, w.w_in, w.w_gate, w.w_out, x, B, T, y, conv_state, h, conv_state_out, h_out, ws,
                            wl, s, tm));
  }
  G_STATUS_TRY(tm.mark(GS_OUT, s));
  if (stage_ms) G_STATUS_TRY(tm.finish(stage_ms));
  return HYMBA_OK;
}

int32_t check_weights(const griffin_block_weights* w) {
  if (!w) return set_error(HYMBA_ERR_INVALID_ARG, "weights is NULL");
  if (!w->w_in || !w->conv_w || !w->w_gate || !w->lam || !w->w_out)
    return set_error(HYMBA_ERR_INVALID_ARG, "a weight pointer is NULL");
  if (!aligned16(w->w_in) || !aligned16(w->conv_w) || !aligned16(w->w_gate) || !aligned16(w->w_out))
    return set_error(HYMBA_ERR_INVALID_ARG, "weight matrices and conv_w must be 16-byte aligned");
  return HYMBA_OK;
}

int32_t check_call(const griffin_block_cfg* cfg, const griffin_block_weights* w, const void* persistent,
                   const void* x, int B, int T, const void* y, void* ws, size_t ws_bytes, size_t* need) {
  G_STATUS_TRY(check_cfg(cfg));
  G_STATUS_TRY(check_weights(w));
  if (is_bf16(*cfg) && (!persistent || reinterpret_cast<uintptr_t>(persistent) % kAlign))
    return set_error(HYMBA_ERR_INVALID_ARG, "bf16 blocks need the prepared persistent buffer (256-byte aligned)");
  if (B < 0 || T < 0) return set_error(HYMBA_ERR_INVALID_ARG, "batch and seq must be >= 0");
  if (B > 65535) return set_error(HYMBA_ERR_UNSUPPORTED, "batch beyond 65535");
  if (static_cast<int64_t>(B) * T > (int64_t(1) << 31) / 2)
    return set_error(HYMBA_ERR_UNSUPPORTED, "batch * seq beyond 2^30 rows");
  if (B == 0 || T == 0) { *need = 0; return HYMBA_OK; }
  if (static_cast<int64_t>(T) * 2 * cfg->d_rnn * static_cast<int64_t>(elem(*cfg)) >= (int64_t(1) << 31))
    return set_error(HYMBA_ERR_UNSUPPORTED, "one sequence's gate activations (seq x 2 d_rnn) must stay below 2 GiB");
  if (!x || !y || !ws) return set_error(HYMBA_ERR_INVALID_ARG, "x, y and workspace must be non-NULL");
  if (!aligned16(x) || !aligned16(y)) return set_error(HYMBA_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(ws) % kAlign)
    return set_error(HYMBA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  *need = layout(*cfg, B, T).total;
  if (ws_bytes < *need) return set_error(HYMBA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, *need);
  return HYMBA_OK;
}

}  // namespace

extern "C" {

size_t griffin_block_persistent_bytes(const griffin_block_cfg* cfg) {
  if (check_cfg(cfg) != HYMBA_OK) return 0;
  return persist_layout(*cfg).total;
}

int32_t griffin_block_prepare(const griffin_block_cfg* cfg, const griffin_block_weights* w, void* persistent,
                              size_t persistent_bytes, void* stream) {
  G_STATUS_TRY(check_cfg(cfg));
  G_STATUS_TRY(check_weights(w));
  if (!is_bf16(*cfg)) return HYMBA_OK;
  const Persist pl = persist_layout(*cfg);
  if (!persistent || reinterpret_cast<uintptr_t>(persistent) % kAlign)
    return set_error(HYMBA_ERR_INVALID_ARG, "persistent buffer must be non-NULL and 256-byte aligned");
  if (persistent_bytes < pl.total)
    return set_error(HYMBA_ERR_WORKSPACE, "persistent buffer has %zu bytes, needs %zu", persistent_bytes, pl.total);
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* p = static_cast<char*>(persistent);
  const int64_t R = cfg->d_rnn, D = cfg->d_model;
  G_HIP_TRY(launch_convert(static_cast<const bf16_t*>(w->w_in), D, reinterpret_cast<half_t*>(p + pl.w_in), D, 2 * R, D, s),
            "weight conversion launch");
  G_HIP_TRY(launch_convert(static_cast<const bf16_t*>(w->w_gate), R, reinterpret_cast<half_t*>(p + pl.w_gate), R, 2 * R,
                           R, s),
            "weight conversion launch");
  G_HIP_TRY(launch_convert(static_cast<const bf16_t*>(w->w_out), R, reinterpret_cast<half_t*>(p + pl.w_out), R, D, R, s),
            "weight conversion launch");
  return HYMBA_OK;
}

size_t griffin_workspace_bytes(const griffin_block_cfg* cfg, int32_t batch, int32_t seq) {
  if (check_cfg(cfg) != HYMBA_OK || batch <= 0 || seq <= 0) return 0;
  return layout(*cfg, batch, seq).total;
}

int32_t griffin_block_prefill(const griffin_block_cfg* cfg, const griffin_block_weights* w, const void* persistent,
                              const void* x, int32_t B, int32_t T, void* y, const float* conv_state, const float* h,
                              float* conv_state_out, float* h_out, void* workspace, size_t workspace_bytes,
                              void* stream, float* stage_ms) {
  size_t need = 0;
  G_STATUS_TRY(check_call(cfg, w, persistent, x, B, T, y, workspace, workspace_bytes, &need));
  if (B == 0 || T == 0) return HYMBA_OK;
  if (conv_state && conv_state_out == conv_state && T > 1)
    return set_error(HYMBA_ERR_INVALID_ARG, "conv_state_out may alias conv_state only when seq == 1");
  if ((conv_state && !aligned16(conv_state)) || (conv_state_out && !aligned16(conv_state_out)))
    return set_error(HYMBA_ERR_INVALID_ARG, "conv states must be 16-byte aligned");
  return forward(*cfg, *w, persistent, x, B, T, y, conv_state, h, conv_state_out, h_out,
                 static_cast<char*>(workspace), layout(*cfg, B, T), static_cast<hipStream_t>(stream), stage_ms);
}

int32_t griffin_block_decode(const griffin_block_cfg* cfg, const griffin_block_weights* w, const void* persistent,
                             const void* x_t, int32_t B, void* y_t, float* conv_state, float* h, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (!conv_state || !h) return set_error(HYMBA_ERR_INVALID_ARG, "decode needs conv_state and h");
  return griffin_block_prefill(cfg, w, persistent, x_t, B, 1, y_t, conv_state, h, conv_state, h, workspace,
                               workspace_bytes, stream, nullptr);
}

}  // extern "C"
