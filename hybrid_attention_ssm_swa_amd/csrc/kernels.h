// Kernel launch interface used by the C-ABI layer (host side).  Every pointer
// is device memory; row-major layouts with explicit leading dimensions (in
// elements) so kernels can read column slices of the shared projection.
// "Activation type" CT is fp32 for fp32 layers and fp16 for bf16 layers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace hymba {

// ---- prefill attention ------------------------------------------------------
// Q: row (b*T + t), head h at column h*hd.  K/V real rows: row t of sequence b
// at k + b*kv_seq_stride + t*ld_kv, KV head g at column g*hd.  Meta K/V:
// [n_meta, Hkv, hd] (row stride ld_meta).  O: row (b*T + t), head h at h*hd.
template <typename ET>
struct AttnArgs {
  const ET* q; int64_t ld_q;
  const ET* k; const ET* v; int64_t ld_kv; int64_t kv_seq_stride;
  const ET* k_meta; const ET* v_meta; int64_t ld_meta; int n_meta;
  ET* o; int64_t ld_o;
  int B, T, n_heads, n_kv_heads, head_dim, window;
  float scale_log2;   // log2(e) / sqrt(hd)
};
// MFMA kernel (hd = 64), fp16 or bf16 operands, fp32 accumulation.
hipError_t launch_attn_prefill_mfma(const AttnArgs<half_t>& a, hipStream_t s);
// VALU kernel, fp32 (hd 32 or 64).
hipError_t launch_attn_prefill_f32(const AttnArgs<float>& a, hipStream_t s);
bool attn_mfma_supported(int head_dim, int n_heads, int n_kv_heads, int n_meta);

// ---- selective scan (prefill) and one-token state update (decode) -------------
// u, dt: [rows, E] slices (row stride ld); bc: fp32 rows with B_t at
// bc[0..N) and C_t at bc[N..2N) (row stride ld_bc).  A2 = A * log2(e) [E, N];
// h0 [E, N] per sequence stride h0_bstride (0 = shared by the batch, null =
// zeros).  y: [rows, E] (row stride ldy), the ungated SSM output; h_out:
// [B, E, N] final state (nullable).
template <typename CT>
struct ScanArgs {
  const CT* u; const CT* dt; int64_t ld;
  const float* bc; int64_t ld_bc;
  const float* A2; const float* D; const float* dt_bias;
  const float* h0; int64_t h0_bstride;
  CT* y; int64_t ldy;
  float* h_out;
  int B, T, E, N;
  float* seg = nullptr; size_t seg_bytes = 0;   // time-segment summaries (scan_segment_bytes); may be NULL
};
// Workspace for the time-segment summaries of a scan of B sequences of T steps (0: one pass).
size_t scan_segment_bytes(int B, int T, int E, int N);
hipError_t launch_selective_scan(const ScanArgs<float>& a, hipStream_t s);
hipError_t launch_selective_scan(const ScanArgs<half_t>& a, hipStream_t s);

// h: [B, E, N] fp32 updated in place; row b of u/dt/bc is sequence b (bc in the
// activation type, B at bc[0..N), C at bc[N..2N)).
template <typename CT>
struct StepArgs {
  const CT* u; const CT* dt; int64_t ld;
  const float* bc; int64_t ld_bc;   // B_t at bc[0, N), C_t at bc[N, 2N) of row b (fp32)
  const float* A2; const float* D; const float* dt_bias;
  float* h;
  CT* y; int64_t ldy;
  int B, E, N;
};
hipError_t launch_ssm_step(const StepArgs<float>& a, hipStream_t s);
hipError_t launch_ssm_step(const StepArgs<half_t>& a, hipStream_t s);

// ---- fused epilogue: F = beta1*rms(Ao) + beta2*rms(y*silu(z)) ------------------
// Inputs in the activation type CT; the fused output F in FT (bf16 layers
// write F as bf16, the operand type of their output projection).
template <typename CT, typename FT = CT>
struct EpiArgs {
  const CT* ao; int64_t ld_ao;
  const CT* y; int64_t ld_y;
  const CT* z; int64_t ld_z;
  const float* beta1; const float* beta2;
  FT* f; int64_t ld_f;
  int64_t rows; int E; float eps;
  uint32_t* flags;   // or null: word 0 set to 1 when a row's branch statistic is not finite
};
hipError_t launch_epilogue(const EpiArgs<float>& a, hipStream_t s);
hipError_t launch_epilogue(const EpiArgs<half_t, bf16_t>& a, hipStream_t s);

// ---- K/V movement -------------------------------------------------------------
// Source rows (b*T + t) with KV head g at column g*hd.  Writes, when non-null,
// the full K/V [B, T, Hkv, hd] and the cache [B, Hkv, C, hd]: with pos == null
// (prefill) token t >= T - C goes to slot t mod C; with pos != null (decode,
// T == 1) the token goes to slot pos[b] mod C (nothing for pos[b] < 0).
template <typename CT>
struct KvWriteArgs {
  const CT* k_src; const CT* v_src; int64_t ld_src;
  CT* k_full; CT* v_full;
  CT* k_cache; CT* v_cache; int cache_len;
  const int64_t* pos;
  int B, T, n_kv_heads, head_dim;
};
hipError_t launch_kv_write(const KvWriteArgs<float>& a, hipStream_t s);
hipError_t launch_kv_write(const KvWriteArgs<half_t>& a, hipStream_t s);

// ---- decode attention -----------------------------------------------------------
// One query token per sequence (row b of q).  Keys: n_meta meta keys, then the
// real tokens max(0, p-Weff+1)..p (p = pos[b]) read from cache slot r mod C,
// Weff = window > 0 ? window : C.  Split over `splits` key ranges; partials
// [B, H, splits, hd + 2] in `part`, combined into o (row b, head h at h*hd).
template <typename CT>
struct DecAttnArgs {
  const CT* q; int64_t ld_q;
  const CT* k_meta; const CT* v_meta; int64_t ld_meta; int n_meta;
  const CT* k_cache; const CT* v_cache; int cache_len;
  const int64_t* pos;
  CT* o; int64_t ld_o;
  float* part;
  int B, n_heads, n_kv_heads, head_dim, window, splits;
  float scale_log2;
  uint32_t* flags;   // or null: word 1 set to 1 when a sequence's position is negative
};
hipError_t launch_decode_attn(const DecAttnArgs<float>& a, hipStream_t s);
hipError_t launch_decode_attn(const DecAttnArgs<half_t>& a, hipStream_t s);
int decode_attn_splits(int B, int n_kv_heads, int n_keys_max, int head_dim, int elem_bytes);
constexpr int kDecodeMaxSplits = 64;
constexpr int kDecodeMaxHd = 128;

// ---- rotary position encoding of the projection's q and k columns, in place ----------
// Row r (of `rows`) holds q heads at columns [0, n_q_heads * hd) and k heads at
// [k_off, k_off + n_k_heads * hd); its position is first + pos[r] (pos != null,
// decode) or first + r % T.  theta[i] = base^(-2i/hd) for the pairs of a head.
constexpr int kRopeMaxPairs = 64;
template <typename CT>
struct RopeArgs {
  CT* p; int64_t ld;
  int64_t rows; int64_t T;
  int n_q_heads; int64_t k_off; int n_k_heads; int head_dim;
  int64_t first; const int64_t* pos;
  double theta[kRopeMaxPairs];
};
hipError_t launch_rope(const RopeArgs<float>& a, hipStream_t s);
hipError_t launch_rope(const RopeArgs<half_t>& a, hipStream_t s);

// ---- fp32 GEMM: Y[rows, out] = X[rows, in] . W[out, in]^T ----------------------
hipError_t launch_gemm_f32(const float* X, int64_t ldx, const float* W, int64_t ldw, float* Y,
                           int64_t ldy, int64_t rows, int out, int in, hipStream_t s);

// ---- element-type conversion of a strided [rows, cols] block (cols % 4 == 0) -----
hipError_t launch_convert(const bf16_t* src, int64_t ld_src, half_t* dst, int64_t ld_dst, int64_t rows,
                          int64_t cols, hipStream_t s);
hipError_t launch_convert(const half_t* src, int64_t ld_src, float* dst, int64_t ld_dst, int64_t rows,
                          int64_t cols, hipStream_t s);
hipError_t launch_convert(const float* src, int64_t ld_src, bf16_t* dst, int64_t ld_dst, int64_t rows,
                          int64_t cols, hipStream_t s);
hipError_t launch_convert(const half_t* src, int64_t ld_src, bf16_t* dst, int64_t ld_dst, int64_t rows,
                          int64_t cols, hipStream_t s);

// ---- Griffin recurrent block: causal width-4 conv and the RG-LRU recurrence ------
// conv: xc[row, r] = sum_k w[k, r] u[row - k, r] within a sequence; inputs before t = 0 come
// from hist [B, 3, R] fp32 (oldest first; null: zeros); state_out [B, 3, R] (null: none) gets
// the last three inputs (may alias hist only when seq == 1).
template <typename T>
struct GriffinConvArgs {
  const T* u; int64_t ld_u;
  const float* w;
  const float* hist; float* state_out;
  T* xc; int64_t ld_xc;
  int B; int seq; int R;
};
hipError_t launch_griffin_conv(const GriffinConvArgs<float>& a, hipStream_t s);
hipError_t launch_griffin_conv(const GriffinConvArgs<half_t>& a, hipStream_t s);

// RG-LRU + GeLU branch: g [rows, 2R] holds the gate pre-activations (W_a xc | W_x xc); y = h GeLU(v);
// h0 [B, R] (null: zeros) -> h_out [B, R] (null: none; may alias h0).  R even, B <= 65535.
template <typename T>
struct RglruArgs {
  const T* g; int64_t ld_g;
  const T* xc; int64_t ld_xc;
  const T* v; int64_t ld_v;
  T* y; int64_t ldy;
  const float* lam; float c;
  const float* h0; float* h_out;
  int B; int seq; int R;
};
hipError_t launch_rglru(const RglruArgs<float>& a, hipStream_t s);
hipError_t launch_rglru(const RglruArgs<half_t>& a, hipStream_t s);

// ---- weight-streaming GEMM for few rows: Y[M, N] = X[M, K] . W[N, K]^T -------------
// 16-bit W and X (X converted to W's type in registers), fp32 accumulation, output OT; the
// output columns [c0, c1) are also written in fp32 to y32[m, c - c0] when y32 is set.
// N % 4 == 0, K % 8 == 0, 16-byte aligned rows (ldw, ldx multiples of 8; ldy, ldy32, c0, c1 of 4).
template <typename WT, typename XT, typename OT>
struct SkinnyArgs {
  const WT* w; int64_t ldw;
  const XT* x; int64_t ldx;
  OT* y; int64_t ldy;
  float* y32; int64_t ldy32; int c0; int c1;
  int M; int N; int K;
};
// Launch plan: feature tile F (64 or 32).  The kernel needs no workspace: K is never split
// across workgroups.
struct SkinnyPlan { int F = 64; };
SkinnyPlan skinny_plan(int M, int N, int K);
hipError_t launch_skinny_gemm(const SkinnyArgs<half_t, half_t, half_t>& a, hipStream_t s);
hipError_t launch_skinny_gemm(const SkinnyArgs<half_t, bf16_t, half_t>& a, hipStream_t s);
hipError_t launch_skinny_gemm(const SkinnyArgs<half_t, half_t, bf16_t>& a, hipStream_t s);
hipError_t launch_skinny_gemm(const SkinnyArgs<bf16_t, bf16_t, bf16_t>& a, hipStream_t s);
constexpr int kSkinnyMaxRows = 256;   // the callers use it up to this many rows
// ... and for weights up to this size: a larger weight (the 1.5B layer's 36 MB input
// projection) goes through the library GEMM, about twice as fast there as through this
// kernel, whose 32-row workgroups each re-read W's tile from L2 and X once per feature tile
constexpr int64_t kSkinnyMaxWeightBytes = int64_t(24) << 20;
inline bool skinny_fits(int64_t rows, int64_t n, int64_t k) {
  return rows > 0 && rows <= kSkinnyMaxRows && n * k * 2 <= kSkinnyMaxWeightBytes;
}

// ---- many-row projection GEMM on the matrix cores ----------------------------------
// Y[m, n] = sum_k X[m, k] W[n, k] (16-bit X and W of one type, fp32 accumulation, 16-bit Y);
// the columns [c0, c1) are also written in fp32 to y32[m, n - c0] when y32 is set.
// K % 8 == 0, N % 4 == 0, ldx and ldw multiples of 8, ldy of 4, 16-byte aligned X and W,
// 8-byte aligned Y; c0, c1, ldy32 multiples of 4 and y32 16-byte aligned.
struct MfmaGemmArgs {
  const void* x; int64_t ldx;
  const void* w; int64_t ldw;
  void* y; int64_t ldy;
  float* y32; int64_t ldy32; int c0; int c1;
  int64_t M; int N; int K;
};
bool mfma_gemm_shape_ok(const MfmaGemmArgs& a);
// in_type, out_type: 0 = fp16, 1 = bf16 (the GEMM type codes of the library path)
hipError_t launch_mfma_gemm(const MfmaGemmArgs& a, int in_type, int out_type, hipStream_t s);

// ---- input conversion fused with the fp32 B/C columns -------------------------------
// x16 [rows, d] = fp16(x [rows, d] bf16); bc [rows, nbc] fp32 = x . wbc^T (wbc fp16 [nbc, d],
// nbc = 2N = 16 or 32).  d, ldx, ldx16, ldw multiples of 8; 16-byte aligned rows.
struct ConvBcArgs {
  const bf16_t* x; int64_t ldx;
  half_t* x16; int64_t ldx16;
  const half_t* wbc; int64_t ldw;
  float* bc; int64_t ldbc;
  int64_t rows; int d; int nbc;
};
hipError_t launch_convert_bc(const ConvBcArgs& a, hipStream_t s);
// *flag = 1 if any of the n fp16 values at p (16-byte aligned) is inf or NaN; else untouched.
hipError_t launch_nonfinite16_check(const half_t* p, int64_t n, uint32_t* flag, hipStream_t s);

// ---- misc ----------------------------------------------------------------------
hipError_t launch_scale_copy(const float* src, float* dst, int64_t n, float scale, hipStream_t s);
hipError_t launch_fill(float* dst, int64_t n, float value, hipStream_t s);
// Keeps the stream busy for about `microseconds` (one thread, a bounded wait on the wall clock), so
// that work queued behind it meanwhile then runs back to back.
hipError_t launch_spin(int microseconds, hipStream_t s);

}  // namespace hymba
