/*
 * griffin_block.h -- C ABI of the Griffin recurrent block, the library's second
 * diagonal-recurrence workload (MI355X, gfx950).
 *
 * The block (Griffin summary, hyeon-jae.tistory.com, section 2.3 "Recurrent
 * block", section 2.4 "Real-Gated Linear Recurrent Unit (RG-LRU)", appendix A,
 * and the Hawk paragraph of section 3):
 *
 *     [u | v] = x W_in^T                          two branches of width R = d_rnn
 *     xc_t    = sum_k conv_w[k] * u_(t-k)         causal separable Conv1D, width 4, no bias
 *     r_t     = sigmoid(W_a xc_t),  i_t = sigmoid(W_x xc_t)      (W_gate = [W_a ; W_x])
 *     log a_t = c r_t log sigmoid(Lambda)         in log space
 *     h_t     = a_t h_(t-1) + sqrt(1 - a_t^2) (i_t xc_t)
 *     y       = (h * GeLU(v)) W_out^T             GeLU(v) = v Phi(v)
 *
 * No gate biases; the conv and the recurrence start from the handed state (or
 * zeros).  The state of a sequence is its last 3 branch inputs u (oldest
 * first) and h.
 *
 * Types (cfg.dtype): HYMBA_F32 -- everything fp32.  HYMBA_BF16 -- x, y and
 * the weight matrices bf16 at the boundary; inside, the GEMM operands and the
 * intermediate activations (branches u and v, conv output, gate
 * pre-activations, RG-LRU output) are fp16 with fp32 accumulation, against
 * fp16 copies of the weights made once by griffin_block_prepare; conv_w,
 * Lambda and the states fp32.  (bf16 intermediates were measured at about
 * 2.4e-2 x RMS max error on y, fp16 at about 3e-3.)  Inputs must be within
 * the fp16 range.
 *
 * Memory: all pointers are caller-owned device memory, except cfg/weights
 * structs and stage_ms (host).  Matrices are row-major [out, in].  Calls are
 * asynchronous on `stream` unless stage_ms is given.  Errors: HYMBA_* status
 * codes of hymba_mixer.h, text through hymba_last_error().  No allocation in
 * a call (the GEMM library creates its per-device handle once).
 */
#ifndef GRIFFIN_BLOCK_H
#define GRIFFIN_BLOCK_H

#include <stddef.h>
#include <stdint.h>

#include "hymba_mixer.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct griffin_block_cfg {
  int32_t d_model; /* D (multiple of 8)                                              */
  int32_t d_rnn;   /* R (multiple of 8)                                              */
  int32_t dtype;   /* HYMBA_F32 or HYMBA_BF16                                        */
  float c;         /* the recurrence-gate exponent scale (8 in the summary)          */
} griffin_block_cfg;

typedef struct griffin_block_weights {
  const void* w_in;     /* [2R, D]: rows [0, R) the recurrent branch u, [R, 2R) v  */
  const float* conv_w;  /* [4, R]: tap k multiplies the input k steps back         */
  const void* w_gate;   /* [2R, R]: rows [0, R) W_a, [R, 2R) W_x                    */
  const float* lam;     /* [R] Lambda: a = sigmoid(Lambda)                          */
  const void* w_out;    /* [D, R]                                                   */
} griffin_block_weights;

#define GRIFFIN_N_STAGES 5 /* in_proj, conv, gate_proj, rglru, out_proj */

/* Bytes of the persistent buffer of a block (the fp16 weight copies of a bf16
 * block, 0 for fp32), 0 for an invalid cfg. */
size_t griffin_block_persistent_bytes(const griffin_block_cfg* cfg);

/* Writes the fp16 copies of w's matrices into `persistent` (256-byte aligned,
 * griffin_block_persistent_bytes long), asynchronously on `stream`.  Run again
 * whenever the weights change: prefill and decode read the copies, not w's
 * matrices.  A no-op for fp32 blocks. */
int32_t griffin_block_prepare(const griffin_block_cfg* cfg, const griffin_block_weights* w, void* persistent,
                              size_t persistent_bytes, void* stream);

/* Workspace bytes for a prefill of [batch, seq] (seq = 1: a decode step). */
size_t griffin_workspace_bytes(const griffin_block_cfg* cfg, int32_t batch, int32_t seq);

/* Prefill of B sequences of T tokens: x [B, T, D] -> y [B, T, D].
 * persistent: the buffer griffin_block_prepare filled (NULL for fp32 blocks).
 * conv_state [B, 3, R] fp32 and h [B, R] fp32: the state to continue from
 * (NULL: zeros); conv_state_out / h_out receive the final state (NULL: not
 * written); conv_state_out may alias conv_state only when T == 1; h_out may
 * alias h.  stage_ms (host, GRIFFIN_N_STAGES floats) or NULL: with it the
 * call times each stage with events and returns only after the work has
 * finished (measurement only). */
int32_t griffin_block_prefill(const griffin_block_cfg* cfg, const griffin_block_weights* w,
                              const void* persistent, const void* x, int32_t B, int32_t T, void* y,
                              const float* conv_state, const float* h, float* conv_state_out,
                              float* h_out, void* workspace, size_t workspace_bytes, void* stream,
                              float* stage_ms);

/* One token per sequence: x_t [B, D] -> y_t [B, D]; conv_state [B, 3, R] and
 * h [B, R] (fp32) are read and updated in place. */
int32_t griffin_block_decode(const griffin_block_cfg* cfg, const griffin_block_weights* w,
                             const void* persistent, const void* x_t, int32_t B, void* y_t, float* conv_state, float* h,
                             void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif
