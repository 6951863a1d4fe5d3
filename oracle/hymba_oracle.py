"""fp64 CPU oracle of the Hymba hybrid-head mixer.  TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute this module.  The product path (the
HIP library and its Python binding) never touches it, and it shares no code,
constants or helpers with that path: its inputs come from ``hymba_synth``.

Everything is computed per sequence, in float64, as the plain definition:
the meta-token prefix is prepended and processed like any other rows (no
offline prefix shortcut), and attention is an explicitly masked softmax over
the visible key set (no online / blockwise softmax).  Row blocks of queries are
evaluated one after another only to bound memory; rows are independent.

Sources (the pages):
  [H] Hymba summary (greeksharifa.github.io):
      section 2.1 "A Fused Hybrid-Head Module", Eq. (3): Y = W_out_proj(beta1 *
      norm(M_attn X~) + beta2 * norm(M_ssm X~)), one shared input projection
      giving Q, K, V, the SSM features and the output gate;
      section 2.2 "KV Cache Optimization": sliding-window attention in most
      layers, global attention in first/middle/last, K/V shared by
      consecutive layers;
      section 2.3 "Meta Tokens": 128 learned, input-independent rows
      prepended to every sequence; their products can be precomputed;
      section 2.4 "Hymba Attention Map": the SSM seen as an implicit
      token-to-token matrix.
  [G] Griffin summary (hyeon-jae.tistory.com), section 2.3 "Local sliding
      window attention": each token attends only to a fixed window of past
      tokens.
  [N] NVIDIA technical blog on Hymba (open-lab.net mirror), the "KV cache
      sharing" bullet: grouped KV heads shared across layers.

Readings where the pages are silent (each is a named decision, applied the
same way by the GPU path):
  D1  attention ends in its own W_O (H*hd -> E); the fused width is E.
  D2  Eq. (3) is a plain sum (no 1/2).
  D3  norm = RMSNorm over the E channels of a token, eps inside the sqrt, no
      weight of its own (beta is the weight).
  D4  gate: g = y * SiLU(z), z from the shared projection, before the norm.
  D5  SSM: diagonal selective scan, A in R^{E x N}, B_t, C_t in R^N shared by
      all channels, dA = exp(dt*A), dB = dt*B, skip term D*u.
  D6  no convolution before the scan.
  D7  dt = softplus(dt_raw + dt_bias), dt_raw a full-width projection block.
  D8  SWA window = the W most recent real positions including self; meta
      keys are always visible and not counted in W.
  D9  meta rows attend causally among themselves.
  D10 scale 1/sqrt(hd); head h uses KV head floor(h*Hkv/H); no RoPE.
  D11 decode index p counts real tokens; K/V of real token r live in cache
      slot r mod C.
  D12 a KV consumer uses its producer's K/V for every position, meta included.
  D17 rotary position encoding (when rope_base > 0): the pages (Hymba summary
      section 2.5 "Hymba Model Family" on the 8K-context stage; Griffin summary
      section 2.3 "Temporal-mixing blocks") name RoPE and a changeable base but
      print no formula, so the RoFormer
      definition is used: consecutive pairs (x[2i], x[2i+1]) of every q and k
      head vector are rotated by the angle pos * base^(-2i/hd); the meta rows
      sit at positions 0..M-1 and real token t at M + t; K is rotated before it
      is cached or handed to a consumer, which uses it as given (D12).

Parity status: the attention mask, GQA grouping, scan, gate/norm/fusion and
KV-sharing are pinned by closed forms, library routines and brute force in
tests/test_oracle_pins.py.  The readings D1, D3-D7 and D10 themselves cannot
be checked against the pages (they print no worked example): as a model of
real Hymba the whole layer is "parity unpinned".
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

F64 = np.float64


# --- elementwise pieces -------------------------------------------------------

def softplus(x):
    """ln(1 + e^x), evaluated stably (D7)."""
    return np.logaddexp(0.0, x)


def sigmoid(x):
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def silu(x):
    """z * sigmoid(z), the gate activation of reading D4."""
    return x * sigmoid(x)


def rms_normalize(x, eps):
    """x / sqrt(mean(x^2) + eps) over the last axis (reading D3)."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


# --- shared input projection [H] section 2.1 ------------------------------------

def split_projection(P, s):
    """Split the shared projection's columns: [Q | K | V | U | Z | dt | B | C] (no K, V for a consumer)."""
    widths = [("q", s.n_heads * s.head_dim)]
    if s.own_kv:
        widths += [("k", s.n_kv_heads * s.head_dim), ("v", s.n_kv_heads * s.head_dim)]
    widths += [("u", s.d_inner), ("z", s.d_inner), ("dt", s.d_inner),
               ("b", s.d_state), ("c", s.d_state)]
    out, c0 = {}, 0
    for name, w in widths:
        out[name] = P[..., c0:c0 + w]
        c0 += w
    assert c0 == P.shape[-1]
    return out


# --- attention [H] sections 2.2-2.3, [G] section 2.3 ------------------------------

def rope(x, positions, base):
    """Rotary position encoding of head vectors x [L, heads, hd] at positions [L] (reading D17):
    each consecutive pair (x[..., 2i], x[..., 2i+1]) turns by positions * base**(-2i/hd).
    base <= 0 leaves x unchanged."""
    x = np.asarray(x, F64)
    if not base or base <= 0:
        return x
    hd = x.shape[-1]
    theta = float(base) ** (-2.0 * np.arange(hd // 2) / hd)
    ang = np.asarray(positions, F64)[:, None] * theta[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    out[..., 1::2] = x[..., 0::2] * s + x[..., 1::2] * c
    return out


def visible(i, j, n_meta, window):
    """Key position j is visible to query position i (positions count meta rows first).

    Causal (j <= i); for a sliding window (window > 0) additionally either j is a
    meta row (j < n_meta) or j is among the `window` most recent positions
    (j > i - window).  window <= 0 means global causal attention.
    """
    causal = j <= i
    if window <= 0:
        return causal
    return causal & ((j < n_meta) | (j > i - window))


def attention(Q, K, V, n_meta, window, row_block=256):
    """Masked softmax attention over the visible set.

    Q, K: [L, H, hd] and [L, Hkv, hd]; V: [L, Hkv, dv] (row index = position).
    Returns [L, H*dv].
    """
    Q = np.asarray(Q, F64)
    K = np.asarray(K, F64)
    V = np.asarray(V, F64)
    L, H, hd = Q.shape
    Hkv, dv = K.shape[1], V.shape[2]
    assert H % Hkv == 0
    group = H // Hkv
    scale = 1.0 / np.sqrt(hd)
    out = np.zeros((L, H, dv), F64)
    for i0 in range(0, L, row_block):
        i1 = min(L, i0 + row_block)
        rows = np.arange(i0, i1)
        # columns that can be visible to any row of this block (others are masked anyway)
        lo = 0 if window <= 0 else max(0, i0 - window + 1)
        cols = np.union1d(np.arange(min(n_meta, i1)), np.arange(lo, i1))
        mask = visible(rows[:, None], cols[None, :], n_meta, window)
        for h in range(H):
            g = h // group
            s = (Q[rows, h, :] @ K[cols, g, :].T) * scale
            s = np.where(mask, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[rows, h, :] = p @ V[cols, g, :]
    return out.reshape(L, H * dv)


# --- selective scan (reading D5) ------------------------------------------------

def selective_scan(U, dt_raw, Bm, Cm, A, D, dt_bias, h0):
    """Sequential diagonal selective scan.

    U, dt_raw: [L, E]; Bm, Cm: [L, N]; A: [E, N]; D, dt_bias: [E]; h0: [E, N].
      dt_i = softplus(dt_raw_i + dt_bias)
      h_i  = exp(dt_i * A) * h_{i-1} + (dt_i * U_i) outer B_i
      y_i  = h_i @ C_i + D * U_i
    Returns (y [L, E], h_last [E, N]).
    """
    U = np.asarray(U, F64)
    delta = softplus(np.asarray(dt_raw, F64) + np.asarray(dt_bias, F64))
    Bm = np.asarray(Bm, F64)
    Cm = np.asarray(Cm, F64)
    A = np.asarray(A, F64)
    D = np.asarray(D, F64)
    h = np.array(h0, F64, copy=True)
    L, E = U.shape
    y = np.empty((L, E), F64)
    for i in range(L):
        h = np.exp(delta[i][:, None] * A) * h + (delta[i] * U[i])[:, None] * Bm[i][None, :]
        y[i] = h @ Cm[i] + D * U[i]
    return y, h


def fuse(Ao, g, beta1, beta2, eps):
    """Eq. (3) before the output projection: beta1*norm(attn) + beta2*norm(ssm), a plain sum (D2)."""
    return np.asarray(beta1, F64) * rms_normalize(Ao, eps) + np.asarray(beta2, F64) * rms_normalize(g, eps)


# --- one layer over one sequence --------------------------------------------------

@dataclass
class LayerOut:
    Y: np.ndarray         # [T, d]   outputs of the real rows
    Y_meta: np.ndarray    # [M, d]   outputs of the meta rows
    O: np.ndarray         # [M+T, H*hd] attention heads (before W_O)
    Ao: np.ndarray        # [M+T, E]  attention branch after W_O
    y: np.ndarray         # [M+T, E]  SSM branch before the gate
    g: np.ndarray         # [M+T, E]  gated SSM branch
    F: np.ndarray         # [M+T, E]  fused (Eq. 3 before W_out_proj)
    K: np.ndarray         # [M+T, Hkv, hd]  keys used (own or handed)
    V: np.ndarray
    h_meta: np.ndarray    # [E, N] SSM state after the meta rows
    h_final: np.ndarray   # [E, N] SSM state after the last row


def meta_kv(p):
    """K/V of a producer's meta rows: the shared projection applied to them (no prefix shortcut)."""
    s = p.shape
    P = np.asarray(p.meta, F64) @ np.asarray(p.w_in, F64).T
    parts = split_projection(P, s)
    k = rope(parts["k"].reshape(s.n_meta, s.n_kv_heads, s.head_dim), np.arange(s.n_meta), s.rope_base)
    v = parts["v"].reshape(s.n_meta, s.n_kv_heads, s.head_dim)
    return k, v


def layer_forward(p, x, k_meta=None, v_meta=None, k=None, v=None, h_init=None):
    """The mixer on one sequence: X~ = [meta rows; x] -> Eq. (3) -> W_out_proj.

    x: [T, d].  A consumer (p.shape.own_kv False) takes k_meta/v_meta [M, Hkv, hd]
    and k/v [T, Hkv, hd] from its producer (D12).  h_init, if given, replaces
    the zero state the scan starts from before the meta rows.
    """
    s = p.shape
    M, T = s.n_meta, x.shape[0]
    L = M + T
    xt = np.concatenate([np.asarray(p.meta, F64), np.asarray(x, F64)], axis=0)
    P = xt @ np.asarray(p.w_in, F64).T
    parts = split_projection(P, s)
    Q = rope(parts["q"].reshape(L, s.n_heads, s.head_dim), np.arange(L), s.rope_base)
    if s.own_kv:
        K = rope(parts["k"].reshape(L, s.n_kv_heads, s.head_dim), np.arange(L), s.rope_base)
        V = parts["v"].reshape(L, s.n_kv_heads, s.head_dim)
    else:
        K = np.concatenate([np.asarray(k_meta, F64), np.asarray(k, F64)], axis=0)
        V = np.concatenate([np.asarray(v_meta, F64), np.asarray(v, F64)], axis=0)
    O = attention(Q, K, V, M, s.window)
    Ao = O @ np.asarray(p.w_o, F64).T
    h0 = np.zeros((s.d_inner, s.d_state), F64) if h_init is None else np.asarray(h_init, F64)
    args = (p.A, p.D, p.dt_bias)
    y_m, h_meta = selective_scan(parts["u"][:M], parts["dt"][:M], parts["b"][:M], parts["c"][:M],
                                 *args, h0)
    y_r, h_fin = selective_scan(parts["u"][M:], parts["dt"][M:], parts["b"][M:], parts["c"][M:],
                                *args, h_meta)
    y = np.concatenate([y_m, y_r], axis=0)
    g = y * silu(parts["z"])
    F = fuse(Ao, g, p.beta1, p.beta2, s.rms_eps)
    Yall = F @ np.asarray(p.w_out, F64).T
    return LayerOut(Yall[M:], Yall[:M], O, Ao, y, g, F, K, V, h_meta, h_fin)


# --- one decode step (reading D11) -------------------------------------------------

@dataclass
class DecodeOut:
    Y: np.ndarray         # [d]
    h: np.ndarray         # [E, N] updated state
    k_cache: np.ndarray   # [Hkv, C, hd] cache after the step (a producer writes its slot)
    v_cache: np.ndarray
    O: np.ndarray         # [H*hd]
    Ao: np.ndarray        # [E]
    y: np.ndarray         # [E]
    F: np.ndarray         # [E]


def decode_step(p, x, pos, k_cache, v_cache, h, k_meta, v_meta):
    """One new token at real index `pos` for one sequence.

    x: [d]; k_cache, v_cache: [Hkv, C, hd] with real token r in slot r mod C;
    h: [E, N] state after the previous token; k_meta, v_meta: [M, Hkv, hd].
    A producer writes its new k, v to slot pos mod C first; a consumer only
    reads (its producer has written the slot).  Keys: all meta rows plus real
    tokens max(0, pos-W+1)..pos (global: 0..pos, which needs pos < C).
    """
    s = p.shape
    M, C = s.n_meta, k_cache.shape[1]
    Pr = np.asarray(x, F64) @ np.asarray(p.w_in, F64).T
    parts = split_projection(Pr, s)
    kc = np.array(k_cache, F64, copy=True)
    vc = np.array(v_cache, F64, copy=True)
    if s.own_kv:
        kc[:, pos % C, :] = rope(parts["k"].reshape(1, s.n_kv_heads, s.head_dim), [M + pos], s.rope_base)[0]
        vc[:, pos % C, :] = parts["v"].reshape(s.n_kv_heads, s.head_dim)
    lo = max(0, pos - s.window + 1) if s.window > 0 else 0
    if s.window <= 0:
        assert pos < C, "a global cache must hold every real token"
    reals = np.arange(lo, pos + 1)
    Kk = np.concatenate([np.asarray(k_meta, F64), kc[:, reals % C, :].transpose(1, 0, 2)], axis=0)
    Vv = np.concatenate([np.asarray(v_meta, F64), vc[:, reals % C, :].transpose(1, 0, 2)], axis=0)
    q = rope(parts["q"].reshape(1, s.n_heads, s.head_dim), [M + pos], s.rope_base)[0]
    group = s.n_heads // s.n_kv_heads
    O = np.empty((s.n_heads, s.head_dim), F64)
    for hh in range(s.n_heads):
        gk = hh // group
        sc = Kk[:, gk, :] @ q[hh] / np.sqrt(s.head_dim)
        w = np.exp(sc - sc.max())
        O[hh] = (w / w.sum()) @ Vv[:, gk, :]
    O = O.reshape(-1)
    Ao = O @ np.asarray(p.w_o, F64).T
    y, h_new = selective_scan(parts["u"][None], parts["dt"][None], parts["b"][None], parts["c"][None],
                              p.A, p.D, p.dt_bias, h)
    y = y[0]
    g = y * silu(parts["z"])
    F = fuse(Ao, g, p.beta1, p.beta2, s.rms_eps)
    Y = F @ np.asarray(p.w_out, F64).T
    return DecodeOut(Y, h_new, kc, vc, O, Ao, y, F)


# --- batched conveniences ---------------------------------------------------------

def prefill_batch(case, seqs=None):
    """layer_forward for the chosen sequences of a hymba_synth PrefillCase."""
    seqs = range(case.batch) if seqs is None else seqs
    outs = {}
    for b in seqs:
        if case.shape.own_kv:
            outs[b] = layer_forward(case.params, case.x[b])
        else:
            outs[b] = layer_forward(case.params, case.x[b], case.k_meta, case.v_meta,
                                    case.k[b], case.v[b])
    return outs
