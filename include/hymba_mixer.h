/*
 * hymba_mixer.h -- C ABI of the Hymba hybrid-head mixer library for AMD
 * Instinct MI355X (gfx950).
 *
 * The layer (Hymba summary, greeksharifa.github.io, section 2.1, Eq. 3):
 *
 *     X~ = [meta rows ; X]                                   (section 2.3)
 *     [Q | K | V | U | Z | dt | B | C] = X~ W_in^T           (one shared projection)
 *     Ao = SWA_or_global_attention(Q, K, V) W_O^T            (section 2.2)
 *     y  = selective_scan(U, dt, B, C; A, D, dt_bias)        (SSM heads)
 *     F  = beta1 * rms(Ao) + beta2 * rms(y * SiLU(Z))        (normalise, scale, sum)
 *     Y  = F W_out^T
 *
 * Attention: a real query sees all meta keys plus the `window` most recent
 * real keys including itself (window <= 0: every earlier key); query head h
 * uses KV head floor(h * n_kv_heads / n_heads).  Consecutive layers may share
 * K/V (section 2.2): a consumer layer has no K/V columns in W_in and reads its
 * producer's K/V.  The meta rows are input independent (section 2.3), so their
 * K/V, SSM state and outputs are computed once per layer ("prepare") and
 * reused by every call.
 *
 * Widths: Nin = H*hd + (own_kv ? 2*Hkv*hd : 0) + 3*E + 2*N.  All matrices are
 * row-major.  Weights are [out_features, in_features]: W_in [Nin, d],
 * W_O [E, H*hd], W_out [d, E].
 *
 * Memory: every pointer passed to the library is device memory owned by the
 * caller, except the configuration structs, which are read on the host during
 * the call.  The library allocates no device memory of its own: per-layer
 * state lives in the caller's `persistent` buffer, scratch in the caller's
 * workspace (the GEMM library creates its per-device handle on first use).
 * Weight pointers are borrowed and must stay valid for the lifetime of the
 * handle.
 *
 * Streams: `stream` is a hipStream_t (NULL = the default stream).  Work is
 * enqueued asynchronously; a call returns after validation and launch.
 * Argument errors are reported synchronously before any device work; a
 * device fault surfaces at the caller's next synchronisation.
 *
 * Errors: every int32_t function returns HYMBA_OK (0) or a negative status;
 * hymba_last_error() returns a thread-local description of the last failure.
 * No C++ exception crosses this interface.  A handle must not be used from
 * two threads or two streams at the same time.
 */
#ifndef HYMBA_MIXER_H
#define HYMBA_MIXER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HYMBA_OK 0
#define HYMBA_ERR_INVALID_ARG (-1) /* null pointer, bad dimension, T < 1, H % Hkv != 0 */
#define HYMBA_ERR_UNSUPPORTED (-2) /* dtype, head dim or shape with no kernel          */
#define HYMBA_ERR_WORKSPACE (-3)   /* workspace or persistent buffer too small          */
#define HYMBA_ERR_BIND (-4)        /* KV-sharing misuse                                  */
#define HYMBA_ERR_HIP (-5)         /* HIP runtime / library error                         */
#define HYMBA_ERR_RANGE (-6)       /* device-side check failed (see hymba_layer_check)    */

/* Layer types (hymba_layer_cfg.dtype):
 *   HYMBA_F32:  x, y, weights and activations fp32.
 *   HYMBA_BF16: x, y and weight matrices bf16; activations (the shared
 *               projection, attention operands/outputs, the K/V exchanged
 *               through hymba_kv and kept in caches, the SSM output) fp16
 *               with fp32 accumulation; the fused output F bf16 (the
 *               operand of the bf16 output projection); SSM state and the
 *               vector parameters fp32.  fp16 keeps 11 significand bits where
 *               bf16 keeps 8, at the same MFMA rate and the same bytes moved.
 * HYMBA_F16 names fp16 operands for the per-kernel entry points only. */
#define HYMBA_F32 0
#define HYMBA_BF16 1
#define HYMBA_F16 2

typedef struct hymba_layer_cfg {
  int32_t d_model;    /* d                                                         */
  int32_t n_heads;    /* H query heads                                             */
  int32_t n_kv_heads; /* Hkv key/value heads (H % Hkv == 0)                         */
  int32_t head_dim;   /* hd: 64 for bf16; 32 or 64 for fp32                        */
  int32_t d_inner;    /* E: SSM channels = fused width (multiple of 8)             */
  int32_t d_state;    /* N: SSM state per channel (8 or 16)                        */
  int32_t n_meta;     /* M meta tokens (>= 0)                                       */
  int32_t window;     /* > 0: sliding window of real keys incl. self; <= 0: global */
  int32_t own_kv;     /* 1: projects its own K/V (producer); 0: consumer           */
  int32_t dtype;      /* HYMBA_F32 or HYMBA_BF16                                   */
  float rms_eps;      /* epsilon inside the RMS norm's square root (e.g. 1e-6)     */
  float rope_base;    /* > 0: rotary position encoding of q and k (RoFormer pairs
                         (2i, 2i+1) turned by pos * base^(-2i/hd); meta rows at
                         positions 0..M-1, real token t at M + t; K is rotated
                         before it is cached or handed on), the base the Hymba
                         summary's section 2.5 says the 8K stage changes;
                         0: no position encoding                              */
} hymba_layer_cfg;

/* Device pointers.  Matrices in the storage dtype, 16-byte aligned; vectors
 * fp32. */
typedef struct hymba_layer_weights {
  const void* w_in;     /* [Nin, d]                                         */
  const void* w_o;      /* [E, H*hd]                                        */
  const void* w_out;    /* [d, E]                                           */
  const void* meta;     /* [M, d] meta-token rows                           */
  const float* A;       /* [E, N]  state decay rates (negative)             */
  const float* D;       /* [E]     skip weights                             */
  const float* dt_bias; /* [E]     added before softplus                    */
  const float* beta1;   /* [E]     attention-branch scale                   */
  const float* beta2;   /* [E]     SSM-branch scale                         */
} hymba_layer_weights;

/* K/V handed between layers and kept for decode.  Device pointers in the
 * layer's activation type (fp32 for HYMBA_F32, fp16 for HYMBA_BF16), 16-byte
 * aligned; any of them may be NULL where noted. */
typedef struct hymba_kv {
  /* Meta K/V [M, Hkv, hd] of an unbound consumer (read).  Ignored by a
   * producer and by a consumer bound with hymba_kv_share_bind. */
  const void* k_meta;
  const void* v_meta;
  /* Prefill K/V of the real tokens [B, T, Hkv, hd]: a producer writes them
   * when non-NULL; a consumer reads them (required). */
  void* k;
  void* v;
  /* Decode cache [B, Hkv, cache_len, hd]; real token r lives in slot
   * r mod cache_len.  Prefill of a producer writes the last cache_len tokens
   * when non-NULL; decode of a producer writes slot pos mod cache_len and
   * then attends; decode of a consumer only reads.  A sliding-window layer
   * needs cache_len >= window; a global layer attends to the last cache_len
   * real tokens. */
  void* k_cache;
  void* v_cache;
  int32_t cache_len;
} hymba_kv;

typedef struct hymba_layer hymba_layer;

/* Bytes of the caller-owned per-layer buffer (meta-prefix K/V, SSM state and
 * outputs, scaled decay rates).  0 if cfg is invalid. */
size_t hymba_layer_persistent_bytes(const hymba_layer_cfg* cfg);

/* Validates cfg, records the weights and carves `persistent` (device, at least
 * hymba_layer_persistent_bytes bytes, 256-byte aligned).  *out receives the
 * handle.  No device work. */
int32_t hymba_layer_create(const hymba_layer_cfg* cfg, const hymba_layer_weights* w,
                           void* persistent, size_t persistent_bytes, hymba_layer** out);

void hymba_layer_destroy(hymba_layer* layer);

/* Cross-layer KV sharing (Hymba summary section 2.2): `consumer` (own_kv == 0)
 * will read the K/V of `producer` (own_kv == 1), whose meta K/V it uses for
 * its own meta prefix.  Shapes (Hkv, hd, M, dtype) must match; pairs only;
 * producer == NULL unbinds.  Invalidates the consumer's prepared prefix.  Host
 * only; returns HYMBA_ERR_BIND on misuse. */
int32_t hymba_kv_share_bind(hymba_layer* consumer, const hymba_layer* producer);

/* Workspace bytes for prefill of [batch, seq] or decode (seq = 1) of `batch`
 * sequences; covers the meta-prefix preparation as well.  Every call that
 * takes a workspace needs it 256-byte aligned, and x, y and the SSM states
 * 16-byte aligned (HYMBA_ERR_INVALID_ARG otherwise, before any device work). */
size_t hymba_mixer_workspace_bytes(const hymba_layer* layer, int32_t batch, int32_t seq);

/* Runs the layer on its meta rows alone (Hymba summary section 2.3): fills
 * the meta K/V (producer), the SSM state after the prefix and the meta rows'
 * outputs in the persistent buffer.  A consumer needs its producer prepared
 * (bound) or kv->k_meta / kv->v_meta (unbound).  prefill/decode call it
 * themselves when needed; calling it explicitly keeps it out of timed work. */
int32_t hymba_layer_prepare(hymba_layer* layer, const hymba_kv* kv, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Prefill of B sequences of T real tokens, continuing from the meta prefix.
 * x [B, T, d] -> y [B, T, d].  ssm_state_out [B, E, N] fp32 receives the final
 * SSM state (may be NULL).  kv as described above.
 * The SSM branch runs on a second stream owned by the layer (created on the
 * first prefill on the current device, non-blocking, default priority),
 * forked from and joined back into `stream` with events: to the caller all
 * work is ordered on `stream`, and the pattern is legal under graph capture. */
int32_t hymba_mixer_prefill(hymba_layer* layer, const void* x, int32_t B, int32_t T, void* y,
                            const hymba_kv* kv, float* ssm_state_out, void* workspace,
                            size_t workspace_bytes, void* stream);

/* One decode step: x_t [B, d] -> y_t [B, d] for the token at real index
 * pos[b] (device int64 [B]).  ssm_state [B, E, N] fp32 holds the state after
 * token pos-1 and is updated in place.  A producer writes its new K/V into
 * slot pos mod cache_len before attending; the consumer of the pair must be
 * called after it with the same kv.  1 <= B <= 65535 (HYMBA_ERR_UNSUPPORTED
 * above: the sequence index is a launch grid dimension). */
int32_t hymba_mixer_decode(hymba_layer* layer, const void* x_t, const int64_t* pos, int32_t B,
                           void* y_t, const hymba_kv* kv, float* ssm_state, void* workspace,
                           size_t workspace_bytes, void* stream);

/* The decode step of hymba_mixer_decode without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  The call allocates
 * nothing: its scratch is a 32 MiB array in the library's device code object,
 * one copy per GPU, held until the process ends (its address is taken once
 * per device, on the first call there).  Every projection runs on the
 * library's own few-row MFMA GEMM (no GEMM-library workspace).  The layer must
 * already be prepared (hymba_layer_prepare, which may allocate) with the meta
 * K/V it is handed, else HYMBA_ERR_INVALID_ARG.  Scratch need: B * (Nin
 * rounded up to 64, + 3*E + H*hd, all in the activation type, + 2*N fp32 for
 * bf16 layers) + B * H * splits * (hd + 2) * 4 bytes (splits <= 64, each
 * region rounded to 256 bytes); a call needing more than 32 MiB returns
 * HYMBA_ERR_WORKSPACE before any device work (about 560 sequences of the
 * 1.5B-shaped layer fit).  Results equal hymba_mixer_decode's up to the order
 * of the projections' fp32 sums.  All calls on one GPU share its scratch and
 * it keeps the last call's contents: calls that overlap on one GPU (two
 * streams, two threads) race and must be serialised by the caller. */
int32_t hymba_mixer_decode_static(hymba_layer* layer, const void* x_t, const int64_t* pos, int32_t B,
                                  void* y_t, const hymba_kv* kv, float* ssm_state, void* stream);

/* Device pointers of the prepared meta prefix inside the persistent buffer:
 * K/V [M, Hkv, hd] in the activation type (producer only, else NULL), SSM
 * state after the prefix [E, N] fp32, outputs of the meta rows [M, d] in the
 * storage type.  HYMBA_ERR_INVALID_ARG if the layer is not prepared. */
int32_t hymba_layer_meta_outputs(const hymba_layer* layer, const void** k_meta,
                                 const void** v_meta, const float** h_meta, const void** y_meta);

const char* hymba_last_error(void);
const char* hymba_status_string(int32_t status);

/* ---- stage timing ----------------------------------------------------------
 * hymba_layer_profile(layer, 1) starts a recording: from then on every
 * prefill/decode call brackets each of its stage intervals with a pair of HIP
 * events on the call's stream (the one-off meta-prefix pass of a prepare is
 * not recorded).  Each timed interval covers exactly one kernel launch.
 * Stages:
 *   0 shared input projection GEMM   1 K/V write            2 attention
 *   3 W_O projection GEMM            4 SSM (scan / step)    5 fused epilogue
 *   6 output projection GEMM         7 storage/activation type conversions
 *   8 rotary encoding of q and k (layers with rope_base > 0)
 * hymba_layer_profile(layer, 0) stops recording and keeps what was recorded.
 * hymba_layer_profile_read waits for the last recorded event and writes, per
 * stage, the summed interval time divided by the number of recorded calls
 * (mean milliseconds per call; 0 for stages that did not run) into
 * stage_ms[0..n).  At most 1024 intervals are kept per recording; beyond
 * that the read fails with HYMBA_ERR_WORKSPACE (stage_ms zeroed).  The first
 * enable creates the events (HYMBA_ERR_HIP on failure); nothing else touches
 * the device.                                                               */
#define HYMBA_N_STAGES 9

/* Device-side checks (async).  Every prefill and decode of the layer records
 * in its persistent buffer whether (a) a row's attention or SSM branch output
 * was not finite, which means an activation left the activation type's range
 * (bf16 layers compute in fp16: any |x|, weight or projected value above
 * 65504 overflows; values below 2^-14 lose relative precision as fp16
 * subnormals, an absolute error of at most 2^-25 per element) or the input held
 * inf/NaN, or (b) a decode position pos[b] was negative (such a sequence
 * writes no cache slot and attends to the meta keys only).  Outputs are
 * written as computed either way.  Preparing a bf16 layer also records (c)
 * whether a weight of W_in or W_O lies beyond fp16's range (it is inf in the
 * layer's fp16 copy); W_out is used in bf16 and not checked.
 * hymba_layer_check synchronises `stream`, reads the record, clears (a) and
 * (b) (the weight record stays), and returns HYMBA_ERR_RANGE (with a message)
 * if anything is recorded, else HYMBA_OK.  A global
 * layer's decode at pos >= cache_len is not an error: it attends to the last
 * cache_len real tokens (exact global attention needs cache_len >= pos + 1). */
int32_t hymba_layer_check(hymba_layer* layer, void* stream);

/* Prefill schedule.  enable = 1 (the default): the SSM branch (the selective
 * scan) runs on the layer's second stream, beside attention and W_O.
 * enable = 0: every kernel of a prefill runs in order on the call's stream,
 * so stage timings measure each kernel alone.  Results are identical either
 * way.  Host only. */
int32_t hymba_layer_set_overlap(hymba_layer* layer, int32_t enable);
/* Prefill projections of a bf16 layer (more than 256 rows).
 * HYMBA_GEMM_LIBRARY (0, the default): hipBLASLt on fp16 copies, x converted
 * by a separate pass that also computes the fp32 B/C columns.
 * HYMBA_GEMM_TILED (1): the hand-written tiled matrix-core GEMM of
 * hymba_kernel_gemm_tiles, which multiplies the bf16 x and W_in directly and
 * writes the fp32 B/C columns from its accumulator (no conversion pass).
 * Both round the same exact products' fp32 sums; results differ only in
 * summation order.  The library is the default because it is faster on
 * every prefill shape measured (8K input projection 3.5 ms against 4.4 ms).
 * Host only; returns HYMBA_ERR_INVALID_ARG for other values. */
#define HYMBA_GEMM_LIBRARY 0
#define HYMBA_GEMM_TILED 1
int32_t hymba_layer_set_gemm(hymba_layer* layer, int32_t backend);
int32_t hymba_layer_profile(hymba_layer* layer, int32_t enable);
int32_t hymba_layer_profile_read(hymba_layer* layer, float* stage_ms, int32_t n);
const char* hymba_stage_name(int32_t stage);

/* ---- per-kernel entry points (parity tests and profiling) -----------------
 * Each runs one kernel of the path on caller buffers, with the same layouts
 * the layer uses internally.  dtype names the element type of the 16/32-bit
 * operands: HYMBA_F32 or HYMBA_F16 (what bf16 layers use inside).  The
 * attention entry returns HYMBA_ERR_UNSUPPORTED for HYMBA_BF16: bf16
 * probabilities would round the P.V operand to 8 significand bits, which
 * misses the 2e-2 RMS bar of a bf16 layer, so bf16 layers attend in fp16.   */

/* Prefill attention.  q: rows (b*T + t), ld_q; head h at column h*hd.
 * k/v: row t of sequence b at k + b*kv_seq_stride + t*ld_kv, KV head g at
 * column g*hd.  k_meta/v_meta: [M, Hkv, hd].  o: rows (b*T + t), ld_o. */
int32_t hymba_kernel_attention(int32_t dtype, const void* q, int64_t ld_q, const void* k,
                               const void* v, int64_t ld_kv, int64_t kv_seq_stride,
                               const void* k_meta, const void* v_meta, int32_t n_meta, void* o,
                               int64_t ld_o, int32_t B, int32_t T, int32_t n_heads,
                               int32_t n_kv_heads, int32_t head_dim, int32_t window, void* stream);

/* Selective scan over B sequences of T rows.  u, dt: [B*T, E] slices with
 * row stride ld (HYMBA_F32 or HYMBA_F16); bc: fp32 rows with B_t at
 * bc[0..N) and C_t at bc[N..2N) (row stride ld_bc, a multiple of 4 and
 * >= 2N; bc 16-byte aligned; ld, ldy >= E).  A [E, N], D, dt_bias [E]
 * fp32 (A is the decay rate, not scaled).  h0 [E, N] fp32 shared initial
 * state or NULL (zero).  y [B*T, E] (row stride ldy) receives the ungated
 * output; h_out [B, E, N] fp32 the final state (may be NULL).
 * workspace: >= E*N*4 bytes, 256-byte aligned.  With
 * hymba_kernel_selective_scan_workspace(B, T, E, N) bytes, few long
 * sequences (too few channel groups to fill the GPU) are cut into time
 * segments: a first launch keeps each segment's end state from zero and its
 * summed step, and the scan starts every segment from the state the
 * recurrence carries into it (the product of a segment's decays is
 * exp(A * the sum of its steps)).  With less, one pass.  Either way the same
 * recurrence, to fp32 rounding.  B <= 65535. */
int32_t hymba_kernel_selective_scan(int32_t dtype, const void* u, const void* dt, int64_t ld,
                                    const float* bc, int64_t ld_bc, const float* A, const float* D,
                                    const float* dt_bias, const float* h0, void* y, int64_t ldy,
                                    float* h_out, int32_t B, int32_t T, int32_t E, int32_t N,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Fused epilogue over `rows` tokens: F = beta1*rms(ao) + beta2*rms(y*SiLU(z)).
 * dtype HYMBA_F32: everything fp32.  HYMBA_F16: ao, y, z fp16 and F bf16 (as
 * in bf16 layers, whose output projection takes F in bf16).  Row strides are
 * >= E and multiples of 8 elements (4 for fp32); pointers 16-byte aligned. */
int32_t hymba_kernel_epilogue(int32_t dtype, const void* ao, int64_t ld_ao, const void* y,
                              int64_t ld_y, const void* z, int64_t ld_z, const float* beta1,
                              const float* beta2, void* f, int64_t ld_f, int64_t rows, int32_t E,
                              float eps, void* stream);

/* Few-row projection, the weight-streaming GEMM the layer calls for up to 256
 * rows (decode batches): y[M, N] = x[M, K] . w[N, K]^T with fp32 accumulation
 * ([H] §2.1 Eq. 3: the shared input projection, W_O and the output
 * projection).  Types (w, x, y): (HYMBA_F16, HYMBA_F16, HYMBA_F16),
 * (HYMBA_F16, HYMBA_BF16, HYMBA_F16) (x converted to fp16 on its way in),
 * (HYMBA_F16, HYMBA_F16, HYMBA_BF16) and (HYMBA_BF16, HYMBA_BF16, HYMBA_BF16).
 * Row-major, 16-byte aligned pointers; ldw, ldx multiples of 8 and >= K; ldy
 * a multiple of 4 and >= N; N % 4 == 0, K % 8 == 0; M >= 0 (any number of
 * rows works; the kernel is meant for few).  y32 (fp32, row stride ldy32, a
 * multiple of 4) or NULL: also receives the columns [c0, c1) of y
 * (multiples of 4) as y32[m, c - c0].  workspace: device memory of at least
 * hymba_kernel_gemm_rows_workspace(M, N, K) bytes, 16-byte aligned (may be
 * NULL when that is 0, which it is for every shape with the current kernel).
 * Deterministic: the sum over K is taken in a fixed order. */
int32_t hymba_kernel_gemm_rows(int32_t w_dtype, int32_t x_dtype, int32_t y_dtype, const void* w,
                               int64_t ldw, const void* x, int64_t ldx, void* y, int64_t ldy,
                               float* y32, int64_t ldy32, int32_t c0, int32_t c1, int32_t M,
                               int32_t N, int32_t K, void* workspace, size_t workspace_bytes,
                               void* stream);

/* Many-row projection, the tiled matrix-core GEMM bf16 layers use for more
 * than 256 rows (prefill): y[M, N] = x[M, K] . w[N, K]^T with fp32
 * accumulation and one rounding to y's type ([H] §2.1 Eq. 3: the shared
 * input projection, W_O and the output projection; [G] §3.3: the O(T D^2)
 * linear layers).  in_dtype names x and w (both HYMBA_F16 or both
 * HYMBA_BF16: the products are taken in that type, bf16 x is not converted);
 * y_dtype is HYMBA_F16 or HYMBA_BF16.  Row-major; x, w 16-byte aligned with
 * ldx, ldw multiples of 8 and >= K; y 8-byte aligned with ldy a multiple of
 * 4 and >= N; N % 4 == 0, K % 8 == 0, M >= 0.  y32 (fp32, 16-byte aligned,
 * row stride ldy32 a multiple of 4) or NULL: also receives the columns
 * [c0, c1) (multiples of 4) as y32[m, c - c0], straight from the fp32
 * accumulator.  No workspace.  Deterministic: each output's K sum is taken
 * in one fixed order.  Asynchronous on `stream`. */
int32_t hymba_kernel_gemm_tiles(int32_t in_dtype, int32_t y_dtype, const void* w, int64_t ldw,
                                const void* x, int64_t ldx, void* y, int64_t ldy, float* y32,
                                int64_t ldy32, int32_t c0, int32_t c1, int64_t M, int32_t N,
                                int32_t K, void* stream);

/* Workspace bytes hymba_kernel_gemm_rows needs for [M, N, K]: 0, since the kernel
 * never splits K across workgroups (kept so that callers size it the same way if
 * a later kernel does). */
size_t hymba_kernel_gemm_rows_workspace(int32_t M, int32_t N, int32_t K);

/* Workspace bytes of hymba_kernel_selective_scan for B sequences of T steps
 * (E channels, N states) that let it split time; 0 for invalid sizes. */
size_t hymba_kernel_selective_scan_workspace(int32_t B, int32_t T, int32_t E, int32_t N);

#ifdef __cplusplus
}
#endif

#endif /* HYMBA_MIXER_H */
