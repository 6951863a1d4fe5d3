"""fp64 CPU oracle of the Griffin recurrent block.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may import, call or
execute this module; the HIP library shares no code with it.  Inputs come from
``hymba_synth.griffin``.

Source: the Griffin summary (hyeon-jae.tistory.com), section 2.3 "Recurrent block", section 2.4
"Real-Gated Linear Recurrent Unit (RG-LRU)", appendix A "RG-LRU Recurrence Gate", and the Hawk
paragraph of section 3, which gives the recurrence weights alpha(r_t) = a_t = a^(c r_t) and
beta(r_t) = sqrt(1 - alpha(r_t)^2).  The summary's displayed equations were lost in extraction;
their content as stated in the text:

  [u | v]  = x W_in^T                       two branches of width D_RNN
  xc_t     = sum_k conv_w[k] * u_(t-k)      separable causal Conv1D, width 4, no bias (4 D_RNN params)
  r_t      = sigmoid(W_a xc_t)              recurrence gate (no h_(t-1) in any gate)
  i_t      = sigmoid(W_x xc_t)              input gate
  log a_t  = c r_t log sigmoid(Lambda)      computed in log space, c = 8
  h_t      = a_t h_(t-1) + sqrt(1 - a_t^2) (i_t xc_t),   y_t = h_t
  out      = (y * GeLU(v)) W_out^T          GeLU branch merged by elementwise product

Readings where the text is silent: no biases in the gates (only W_a, W_x are named); GeLU is
the exact form x * Phi(x); the conv and the recurrence start from zeros before a sequence; the
state handed to a decode step is the last (width - 1) branch inputs u and h.

Parity: the conv, the recurrence and GeLU are pinned by closed forms (impulse response,
geometric series, the normal CDF at 1); the block's composition (which branch is convolved and
recurs, where GeLU sits, what the gates read) by a hand-worked d = 1, D_RNN = 1, T = 2 case
whose every value has a closed form (tests/golden/handworked.json), which swapped branches,
a moved GeLU or gates fed the wrong input all fail; and by the prefill -> decode continuation.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

F64 = np.float64


def sigmoid(x):
    return 0.5 * (1.0 + np.tanh(0.5 * np.asarray(x, F64)))


def softplus(x):
    return np.logaddexp(0.0, np.asarray(x, F64))


def gelu(x):
    """x * Phi(x) with Phi the standard normal CDF."""
    x = np.asarray(x, F64)
    erf = np.vectorize(math.erf, otypes=[F64])
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def causal_conv(u, conv_w, history=None):
    """u: [T, R]; conv_w: [width, R]; history: [width - 1, R] inputs before t = 0 (oldest first),
    zeros when None.  xc_t = sum_k conv_w[k] * u_(t-k)."""
    u = np.asarray(u, F64)
    W = conv_w.shape[0]
    hist = np.zeros((W - 1, u.shape[1])) if history is None else np.asarray(history, F64)
    ext = np.concatenate([hist, u], axis=0)
    T = u.shape[0]
    out = np.zeros_like(u)
    for k in range(W):
        out += np.asarray(conv_w[k], F64)[None, :] * ext[W - 1 - k: W - 1 - k + T]
    return out


def rglru(xc, rho, iota, lam, c, h0=None):
    """The recurrence over [T, R] pre-gate values rho, iota; returns (h [T, R], h_T [R])."""
    xc, rho, iota = (np.asarray(a, F64) for a in (xc, rho, iota))
    r, i = sigmoid(rho), sigmoid(iota)
    log_a = -c * r * softplus(-np.asarray(lam, F64))[None, :]      # c r_t log sigmoid(lambda)
    a = np.exp(log_a)
    beta = np.sqrt(-np.expm1(2.0 * log_a))                        # sqrt(1 - a^2)
    h = np.zeros(xc.shape[1]) if h0 is None else np.asarray(h0, F64).copy()
    out = np.empty_like(xc)
    for t in range(xc.shape[0]):
        h = a[t] * h + beta[t] * (i[t] * xc[t])
        out[t] = h
    return out, h


@dataclass
class GriffinOut:
    Y: np.ndarray         # [T, D]
    u: np.ndarray         # [T, R] recurrent-branch input
    v: np.ndarray         # [T, R] GeLU-branch input
    xc: np.ndarray        # [T, R] conv output
    h: np.ndarray         # [T, R] recurrence output
    h_T: np.ndarray       # [R] final recurrence state
    conv_state: np.ndarray  # [width - 1, R] the last branch inputs u (oldest first)


def griffin_block(p, x, conv_state=None, h0=None):
    """The recurrent block on one sequence x [T, D] (optionally continuing from a state)."""
    s = p.shape
    R = s.d_rnn
    P = np.asarray(x, F64) @ np.asarray(p.w_in, F64).T
    u, v = P[:, :R], P[:, R:]
    xc = causal_conv(u, p.conv_w, conv_state)
    G = xc @ np.asarray(p.w_gate, F64).T
    h, h_T = rglru(xc, G[:, :R], G[:, R:], p.lam, s.c, h0)
    Y = (h * gelu(v)) @ np.asarray(p.w_out, F64).T
    W = s.conv_width
    hist = np.zeros((W - 1, R)) if conv_state is None else np.asarray(conv_state, F64)
    new_state = np.concatenate([hist, u], axis=0)[-(W - 1):]
    return GriffinOut(Y, u, v, xc, h, h_T, new_state)
