"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every check here compares the oracle with something other than itself: a
library routine (torch SDPA, numpy.cumsum), a closed form, a hand-worked
example (tests/golden/handworked.json), or a brute-force loop over an
explicitly enumerated index set.  Each is chosen so that a plausible slip in
the oracle (window off by one, a hidden meta key, a wrong head grouping, a
dropped term of the recurrence, a norm over the wrong axis, a mis-split
projection) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from hymba_synth import LayerShape, make_layer_params, make_prefill_case
from oracle import hymba_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "handworked.json")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _expr(s):
    return float(eval(str(s), {"__builtins__": {}}, {"exp": math.exp, "log": math.log, "ln2": math.log(2.0)}))


def _sdpa(Q, K, V, mask=None, causal=False):
    """torch's fp64 scaled_dot_product_attention with K/V heads repeated in contiguous groups."""
    L, H, hd = Q.shape
    G = H // K.shape[1]
    q = torch.from_numpy(np.ascontiguousarray(Q.transpose(1, 0, 2)))
    k = torch.from_numpy(np.ascontiguousarray(np.repeat(K, G, axis=1).transpose(1, 0, 2)))
    v = torch.from_numpy(np.ascontiguousarray(np.repeat(V, G, axis=1).transpose(1, 0, 2)))
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m, is_causal=causal)
    return o.numpy().transpose(1, 0, 2).reshape(L, H * hd)


def _brute_visible_set(i, n_meta, window):
    """Keys for query position i written out as sets: meta rows up to i, plus the
    `window` most recent positions counting back from i itself (all of 0..i if global)."""
    meta = set(range(min(n_meta, i + 1)))
    if window <= 0:
        recent = set(range(i + 1))
    else:
        recent = {i - k for k in range(window) if i - k >= 0}
    return sorted(meta | recent)


def _brute_mask(L, n_meta, window):
    m = np.zeros((L, L), dtype=bool)
    for i in range(L):
        m[i, _brute_visible_set(i, n_meta, window)] = True
    return m


def _qkv(L, H, Hkv, hd, seed):
    r = _rng(seed)
    return (r.standard_normal((L, H, hd)), r.standard_normal((L, Hkv, hd)),
            r.standard_normal((L, Hkv, hd)))


# --- attention ---------------------------------------------------------------------

@pytest.mark.parametrize("M,T,W", [(4, 20, 24), (4, 20, 100), (0, 17, 17), (8, 9, 17)])
def test_window_covering_sequence_equals_causal_sdpa(M, T, W):
    """North-star check 1: with W >= M+T sliding-window attention is full causal attention."""
    Q, K, V = _qkv(M + T, 6, 2, 8, 1)
    got = orc.attention(Q, K, V, M, W)
    ref = _sdpa(Q, K, V, causal=True)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(orc.attention(Q, K, V, M, 0), ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("M,T,W", [(3, 13, 4), (0, 11, 3), (5, 7, 1), (2, 30, 8)])
def test_sliding_window_against_enumerated_sets(M, T, W):
    """Brute force: per query a scalar-loop softmax over the enumerated visible set."""
    L, H, Hkv, hd = M + T, 4, 2, 3
    Q, K, V = _qkv(L, H, Hkv, hd, 2)
    got = orc.attention(Q, K, V, M, W).reshape(L, H, hd)
    for i in range(L):
        keys = _brute_visible_set(i, M, W)
        for h in range(H):
            g = h // (H // Hkv)
            sc = [sum(Q[i, h, e] * K[j, g, e] for e in range(hd)) / math.sqrt(hd) for j in keys]
            mx = max(sc)
            w = [math.exp(x - mx) for x in sc]
            tot = sum(w)
            for e in range(hd):
                ref = sum(w[a] * V[j, g, e] for a, j in enumerate(keys)) / tot
                assert abs(got[i, h, e] - ref) < 1e-12


def test_swa_matches_sdpa_with_enumerated_mask():
    Q, K, V = _qkv(48, 4, 1, 16, 3)
    mask = _brute_mask(48, 8, 10)
    np.testing.assert_allclose(orc.attention(Q, K, V, 8, 10), _sdpa(Q, K, V, mask=mask),
                               rtol=1e-12, atol=1e-12)


def test_meta_tokens_visible_to_every_query():
    """North-star check 2: with W=1 each real query sees exactly the M meta keys and itself,
    with the closed-form softmax weights, every meta weight > 0."""
    M, T, hd = 5, 12, 4
    L = M + T
    r = _rng(4)
    Q = r.standard_normal((L, 1, hd)) * 2.0
    K = r.standard_normal((L, 1, hd)) * 2.0
    # V = one-hot of the position, so the output row is the attention weight vector
    V = np.eye(L)[:, None, :]
    got = orc.attention(Q, K, V, M, 1)  # [L, L] weights
    for i in range(M, L):
        support = np.nonzero(got[i] > 0)[0].tolist()
        assert support == list(range(M)) + [i]
        keys = list(range(M)) + [i]
        sc = np.array([Q[i, 0] @ K[j, 0] / math.sqrt(hd) for j in keys])
        ref = np.exp(sc - sc.max())
        ref /= ref.sum()
        np.testing.assert_allclose(got[i, keys], ref, rtol=1e-12)
        assert np.all(got[i, :M] > 0)


def test_single_token_without_meta_returns_its_value():
    Q, K, V = _qkv(1, 3, 1, 5, 5)
    np.testing.assert_allclose(orc.attention(Q, K, V, 0, 4).reshape(3, 5), np.repeat(V[0], 3, axis=0),
                               rtol=1e-14)


def test_grouped_kv_equals_mha_with_repeated_heads():
    """GQA (grouped KV heads, NVIDIA blog's KV bullet) == MHA with each KV head repeated for its group."""
    Q, K, V = _qkv(40, 10, 2, 8, 6)
    got = orc.attention(Q, K, V, 6, 9)
    ref = orc.attention(Q, np.repeat(K, 5, axis=1), np.repeat(V, 5, axis=1), 6, 9)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)
    # and a wrong grouping (h % Hkv) would differ
    wrong = orc.attention(Q, np.tile(K, (1, 5, 1)), np.tile(V, (1, 5, 1)), 6, 9)
    assert np.abs(wrong - got).max() > 1e-3


def test_handworked_attention():
    g = json.load(open(GOLDEN))["attention_window"]
    q = np.array([_expr(x) for x in g["q"]])[:, None, None]
    k = np.array([_expr(x) for x in g["k"]])[:, None, None]
    v = np.array([_expr(x) for x in g["v"]])[:, None, None]
    for w, exp in g["expected"].items():
        got = orc.attention(q, k, v, g["n_meta"], int(w)).reshape(-1)
        np.testing.assert_allclose(got, [_expr(e) for e in exp], rtol=1e-13)


# --- selective scan ------------------------------------------------------------------

def _scan_inputs(L, E, N, seed, h0_scale=0.0):
    r = _rng(seed)
    U = r.standard_normal((L, E))
    dt = r.standard_normal((L, E))
    Bm = r.standard_normal((L, N))
    Cm = r.standard_normal((L, N))
    A = -np.exp(r.uniform(0, np.log(8), (E, N)))
    D = r.standard_normal(E)
    bias = np.full(E, -2.0)
    h0 = r.standard_normal((E, N)) * h0_scale
    return U, dt, Bm, Cm, A, D, bias, h0


def test_scan_reduces_to_cumsum():
    """North-star check 3: A=0 and dt=1 make the state a cumulative sum of B_t*u_t."""
    L, E, N = 37, 5, 4
    U, _, Bm, Cm, _, D, _, _ = _scan_inputs(L, E, N, 7)
    A = np.zeros((E, N))
    bias = np.full(E, math.log(math.e - 1.0))   # softplus(bias) = 1
    dt_raw = np.zeros((L, E))
    y, hT = orc.selective_scan(U, dt_raw, Bm, Cm, A, D, bias, np.zeros((E, N)))
    H = np.cumsum(U[:, :, None] * Bm[:, None, :], axis=0)   # [L, E, N]
    np.testing.assert_allclose(hT, H[-1], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y, np.einsum("ten,tn->te", H, Cm) + D * U, rtol=1e-11, atol=1e-11)


def test_scan_equals_implicit_attention_matrix():
    """The recurrence written as the materialised token-to-token matrix (Hymba summary section 2.4):
    y_t = sum_{s<=t} sum_n C_t[n] exp(A[n] * sum_{r=s+1..t} dt_r) dt_s B_s[n] u_s
          + sum_n C_t[n] exp(A[n] * sum_{r=0..t} dt_r) h0[n] + D u_t   (brute-force loops)."""
    L, E, N = 9, 3, 4
    U, dtr, Bm, Cm, A, D, bias, h0 = _scan_inputs(L, E, N, 8, h0_scale=1.0)
    y, _ = orc.selective_scan(U, dtr, Bm, Cm, A, D, bias, h0)
    for c in range(E):
        dts = [math.log1p(math.exp(dtr[t, c] + bias[c])) for t in range(L)]
        for t in range(L):
            acc = D[c] * U[t, c]
            for n in range(N):
                acc += Cm[t, n] * math.exp(A[c, n] * sum(dts[0:t + 1])) * h0[c, n]
                for s in range(t + 1):
                    decay = math.exp(A[c, n] * sum(dts[s + 1:t + 1]))
                    acc += Cm[t, n] * decay * dts[s] * Bm[s, n] * U[s, c]
            assert abs(y[t, c] - acc) < 1e-11 * max(1.0, abs(acc))


def test_scan_zero_input_is_pure_decay():
    L, E, N = 15, 4, 3
    _, dtr, Bm, Cm, A, D, bias, h0 = _scan_inputs(L, E, N, 9, h0_scale=1.0)
    U = np.zeros((L, E))
    y, hT = orc.selective_scan(U, dtr, Bm, Cm, A, D, bias, h0)
    cum = np.cumsum(np.log1p(np.exp(dtr + bias)), axis=0)
    np.testing.assert_allclose(hT, np.exp(A * cum[-1][:, None]) * h0, rtol=1e-12)
    ref_y = np.einsum("ten,tn->te", np.exp(A[None] * cum[:, :, None]) * h0[None], Cm)
    np.testing.assert_allclose(y, ref_y, rtol=1e-11, atol=1e-13)


def test_scan_tiny_step_freezes_state():
    L, E, N = 6, 3, 2
    U, _, Bm, Cm, A, D, bias, h0 = _scan_inputs(L, E, N, 10, h0_scale=1.0)
    dtr = np.full((L, E), -60.0)   # dt = softplus(-62) ~ 1e-27
    y, hT = orc.selective_scan(U, dtr, Bm, Cm, A, D, bias, h0)
    np.testing.assert_allclose(hT, h0, rtol=1e-20, atol=1e-24)
    np.testing.assert_allclose(y, (h0 @ Cm.T).T + D * U, rtol=1e-13)


def test_handworked_scan():
    g = json.load(open(GOLDEN))["scan"]
    arr = lambda key: np.array(g[key], dtype=np.float64)
    y, hT = orc.selective_scan(arr("u"), arr("dt_raw"), arr("B"), arr("C"), arr("A"), arr("D"),
                               arr("dt_bias"), arr("h0"))
    np.testing.assert_allclose(y[:, 0], [_expr(e) for e in g["expected_y"]], rtol=1e-13)
    np.testing.assert_allclose(hT[0], [_expr(e) for e in g["expected_h_final"]], rtol=1e-13)


# --- elementwise pieces ----------------------------------------------------------------

def test_elementwise_special_values():
    assert orc.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-15)
    assert orc.softplus(-40.0) == pytest.approx(math.exp(-40.0), rel=1e-12)
    assert orc.softplus(50.0) == pytest.approx(50.0, rel=1e-15)
    assert orc.silu(0.0) == 0.0
    assert orc.silu(40.0) == pytest.approx(40.0, rel=1e-15)
    assert abs(orc.silu(-40.0)) < 1e-15
    assert orc.silu(1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    x = np.full((2, 7), -3.0)
    np.testing.assert_allclose(orc.rms_normalize(x, 1e-6), -1.0 / math.sqrt(1.0 + 1e-6 / 9.0), rtol=1e-15)
    # per-row, not per-column
    x = np.array([[1.0, 1.0], [10.0, 10.0]])
    np.testing.assert_allclose(orc.rms_normalize(x, 0.0), np.ones((2, 2)), rtol=1e-15)


# --- whole layer -----------------------------------------------------------------------

SMALL = LayerShape(d_model=24, n_heads=4, head_dim=8, n_kv_heads=2, d_inner=16, d_state=4,
                   n_meta=3, window=5, own_kv=True, dtype="f32")


def _attention_branch_independent(p, x):
    """Attention branch through torch SDPA with an enumerated mask, then W_O."""
    s = p.shape
    xt = np.concatenate([p.meta, x]).astype(np.float64)
    L = xt.shape[0]
    Wq = p.w_in[:s.q_width].astype(np.float64)
    Wk = p.w_in[s.q_width:s.q_width + s.kv_width].astype(np.float64)
    Wv = p.w_in[s.q_width + s.kv_width:s.q_width + 2 * s.kv_width].astype(np.float64)
    Q = (xt @ Wq.T).reshape(L, s.n_heads, s.head_dim)
    K = (xt @ Wk.T).reshape(L, s.n_kv_heads, s.head_dim)
    V = (xt @ Wv.T).reshape(L, s.n_kv_heads, s.head_dim)
    O = _sdpa(Q, K, V, mask=_brute_mask(L, s.n_meta, s.window))
    return O @ p.w_o.astype(np.float64).T


def test_beta2_zero_leaves_attention_branch_only():
    """North-star check 4: beta2 = 0 -> Y = W_out(beta1 * rms(attention branch))."""
    r = _rng(11)
    p = make_layer_params(r, SMALL)
    p.beta2[:] = 0.0
    x = r.standard_normal((13, SMALL.d_model)).astype(np.float32)
    out = orc.layer_forward(p, x)
    Ao = _attention_branch_independent(p, x)
    ms = np.mean(Ao * Ao, axis=1, keepdims=True)
    ref = (p.beta1 * Ao / np.sqrt(ms + SMALL.rms_eps)) @ p.w_out.astype(np.float64).T
    np.testing.assert_allclose(out.Y, ref[SMALL.n_meta:], rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(out.Y_meta, ref[:SMALL.n_meta], rtol=1e-10, atol=1e-10)


def test_beta1_zero_leaves_gated_ssm_branch_only():
    r = _rng(12)
    s = SMALL
    p = make_layer_params(r, s)
    p.beta1[:] = 0.0
    x = r.standard_normal((10, s.d_model)).astype(np.float32)
    out = orc.layer_forward(p, x)
    xt = np.concatenate([p.meta, x]).astype(np.float64)
    c0 = s.q_width + 2 * s.kv_width
    W = p.w_in.astype(np.float64)
    U = xt @ W[c0:c0 + s.d_inner].T
    Z = xt @ W[c0 + s.d_inner:c0 + 2 * s.d_inner].T
    dtr = xt @ W[c0 + 2 * s.d_inner:c0 + 3 * s.d_inner].T
    Bm = xt @ W[c0 + 3 * s.d_inner:c0 + 3 * s.d_inner + s.d_state].T
    Cm = xt @ W[c0 + 3 * s.d_inner + s.d_state:].T
    # torch's cumulative product path: h_t = sum_s prod_{r=s+1..t} a_r * b_s (vectorised, not a loop)
    dt = torch.nn.functional.softplus(torch.from_numpy(dtr + p.dt_bias.astype(np.float64)))
    a = torch.exp(dt[:, :, None] * torch.from_numpy(p.A.astype(np.float64))[None])      # [L, E, N]
    b = (dt * torch.from_numpy(U))[:, :, None] * torch.from_numpy(Bm)[:, None, :]
    logcum = torch.cumsum(torch.log(a), dim=0)                                          # [L, E, N]
    L = xt.shape[0]
    H = torch.zeros_like(a)
    for t in range(L):
        H[t] = (torch.exp(logcum[t][None] - logcum[:t + 1]) * b[:t + 1]).sum(0)
    y = torch.einsum("ten,tn->te", H, torch.from_numpy(Cm)) + torch.from_numpy(p.D.astype(np.float64)) * torch.from_numpy(U)
    g = y * torch.nn.functional.silu(torch.from_numpy(Z))
    g = g.numpy()
    ref = (p.beta2 * g / np.sqrt(np.mean(g * g, axis=1, keepdims=True) + s.rms_eps)) @ p.w_out.astype(np.float64).T
    np.testing.assert_allclose(out.Y, ref[s.n_meta:], rtol=1e-9, atol=1e-9)


def test_rms_norm_makes_branch_scale_irrelevant():
    """Per-branch RMS norm (Eq. 3's norm): scaling W_O by c > 0 leaves Y unchanged up to eps."""
    r = _rng(13)
    p = make_layer_params(r, SMALL)
    x = r.standard_normal((9, SMALL.d_model)).astype(np.float32)
    y1 = orc.layer_forward(p, x).Y
    p.w_o *= 7.0
    y2 = orc.layer_forward(p, x).Y
    np.testing.assert_allclose(y1, y2, rtol=1e-3, atol=1e-5)   # eps/mean(Ao^2) effects only
    p.w_o *= -1.0   # a negative scale flips the attention branch's sign: must change Y
    y3 = orc.layer_forward(p, x).Y
    assert np.abs(y3 - y1).max() > 1e-2


def test_kv_sharing_equals_handed_kv():
    """North-star check 5: a consumer handed the producer's K/V == a layer computing that K/V itself.

    The second layer owns its K/V projection with the producer's K/V rows spliced in and the
    producer's meta rows, so it computes exactly the producer's K/V itself."""
    r = _rng(14)
    prod = make_layer_params(r, SMALL)
    cons_shape = SMALL.with_(own_kv=False)
    cons = make_layer_params(r, cons_shape)
    cons.meta = prod.meta.copy()
    x = r.standard_normal((11, SMALL.d_model)).astype(np.float32)
    P = orc.layer_forward(prod, x)
    M = SMALL.n_meta
    y_handed = orc.layer_forward(cons, x, P.K[:M], P.V[:M], P.K[M:], P.V[M:]).Y
    spliced = make_layer_params(_rng(99), SMALL)
    qw, kvw = SMALL.q_width, SMALL.kv_width
    spliced.w_in = np.concatenate([cons.w_in[:qw], prod.w_in[qw:qw + 2 * kvw], cons.w_in[qw:]])
    for f in ("meta", "w_o", "w_out", "A", "D", "dt_bias", "beta1", "beta2"):
        setattr(spliced, f, getattr(cons, f))
    y_own = orc.layer_forward(spliced, x).Y
    np.testing.assert_allclose(y_handed, y_own, rtol=1e-11, atol=1e-11)


def _ring_from_prefill(K, V, M, T, C):
    """Cache [Hkv, C, hd] holding real token t in slot t mod C (the last C tokens survive)."""
    Hkv, hd = K.shape[1], K.shape[2]
    kc = np.zeros((Hkv, C, hd))
    vc = np.zeros((Hkv, C, hd))
    for t in range(max(0, T - C), T):
        kc[:, t % C] = K[M + t]
        vc[:, t % C] = V[M + t]
    return kc, vc


@pytest.mark.parametrize("window,T", [(5, 3), (5, 5), (5, 12), (0, 9)])
def test_prefill_then_decode_equals_longer_prefill(window, T):
    """The decode step continues a prefill exactly (ring wrap-around when T >= W)."""
    s = SMALL.with_(window=window)
    r = _rng(15)
    p = make_layer_params(r, s)
    x = r.standard_normal((T + 1, s.d_model)).astype(np.float32)
    full = orc.layer_forward(p, x)
    pre = orc.layer_forward(p, x[:T])
    C = window if window > 0 else T + 4
    kc, vc = _ring_from_prefill(pre.K, pre.V, s.n_meta, T, C)
    M = s.n_meta
    d = orc.decode_step(p, x[T], T, kc, vc, pre.h_final, pre.K[:M], pre.V[:M])
    np.testing.assert_allclose(d.Y, full.Y[T], rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(d.h, full.h_final, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(d.k_cache[:, T % C], full.K[M + T], rtol=1e-13)


def test_consumer_decode_equals_longer_consumer_prefill():
    s = SMALL
    r = _rng(16)
    prod = make_layer_params(r, s)
    cons = make_layer_params(r, s.with_(own_kv=False))
    T = 8
    x = r.standard_normal((T + 1, s.d_model)).astype(np.float32)
    xc = r.standard_normal((T + 1, s.d_model)).astype(np.float32)
    M = s.n_meta
    Pfull = orc.layer_forward(prod, x)
    full = orc.layer_forward(cons, xc, Pfull.K[:M], Pfull.V[:M], Pfull.K[M:], Pfull.V[M:])
    pre = orc.layer_forward(cons, xc[:T], Pfull.K[:M], Pfull.V[:M], Pfull.K[M:M + T], Pfull.V[M:M + T])
    kc, vc = _ring_from_prefill(Pfull.K, Pfull.V, M, T + 1, s.window)   # producer already wrote token T
    d = orc.decode_step(cons, xc[T], T, kc, vc, pre.h_final, Pfull.K[:M], Pfull.V[:M])
    np.testing.assert_allclose(d.Y, full.Y[T], rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("window", [4, 0])
def test_meta_prefix_precompute_equals_plain_prefix(window):
    """The meta rows' K/V and SSM state can be computed once, offline (Hymba summary section 2.3):
    meta-only run, then token-by-token decode from it, reproduces the plain [meta; X] run."""
    s = SMALL.with_(window=window)
    r = _rng(17)
    p = make_layer_params(r, s)
    T = 10
    x = r.standard_normal((T, s.d_model)).astype(np.float32)
    plain = orc.layer_forward(p, x)
    pre = orc.layer_forward(p, x[:0])          # the meta prefix alone
    kmeta, vmeta = orc.meta_kv(p)
    np.testing.assert_allclose(pre.K, kmeta, rtol=1e-12)
    np.testing.assert_allclose(pre.Y_meta, plain.Y_meta, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(pre.h_final, plain.h_meta, rtol=1e-12, atol=1e-12)
    C = window if window > 0 else T
    kc = np.zeros((s.n_kv_heads, C, s.head_dim))
    vc = np.zeros_like(kc)
    h = pre.h_final
    for t in range(T):
        d = orc.decode_step(p, x[t], t, kc, vc, h, kmeta, vmeta)
        kc, vc, h = d.k_cache, d.v_cache, d.h
        np.testing.assert_allclose(d.Y, plain.Y[t], rtol=1e-10, atol=1e-10)


def test_prefill_case_shapes_and_split():
    """The projection split covers every column exactly once, for producer and consumer layouts."""
    for own in (True, False):
        s = SMALL.with_(own_kv=own)
        case = make_prefill_case(s, 2, 5, 3)
        P = np.zeros((7, s.n_in))
        parts = orc.split_projection(P, s)
        assert sum(v.shape[-1] for v in parts.values()) == s.n_in
        assert ("k" in parts) == own
        outs = orc.prefill_batch(case)
        assert outs[1].Y.shape == (5, s.d_model)


# --- rotary position encoding (reading D17) --------------------------------------------

def test_rope_two_dims_is_a_plane_rotation():
    """hd = 2: the single pair turns by the position itself (base**0 = 1), counter-clockwise."""
    for p in (0.0, 1.0, 3.0, 1000.0):
        out = orc.rope(np.array([[[1.0, 0.0]], [[0.0, 1.0]]]), [p, p], 10000.0)
        assert np.allclose(out[0, 0], [math.cos(p), math.sin(p)], atol=1e-12)
        assert np.allclose(out[1, 0], [-math.sin(p), math.cos(p)], atol=1e-12)


def test_rope_pairs_and_frequencies():
    """hd = 4: dims (0, 1) turn at frequency 1, dims (2, 3) at base**-0.5; no mixing across pairs."""
    base, p = 100.0, 2.5
    e = np.eye(4)[:, None, :]                      # four unit vectors, one head each
    out = orc.rope(e, [p] * 4, base)
    w1 = base ** -0.5
    assert np.allclose(out[0, 0], [math.cos(p), math.sin(p), 0, 0], atol=1e-12)
    assert np.allclose(out[2, 0], [0, 0, math.cos(p * w1), math.sin(p * w1)], atol=1e-12)
    assert np.allclose(out[3, 0], [0, 0, -math.sin(p * w1), math.cos(p * w1)], atol=1e-12)


def test_rope_scores_depend_only_on_relative_position():
    r = np.random.Generator(np.random.PCG64(5))
    q = r.standard_normal((1, 3, 16))
    k = r.standard_normal((1, 3, 16))
    def score(i, j):
        return np.sum(orc.rope(q, [i], 500.0) * orc.rope(k, [j], 500.0), axis=-1)
    assert np.allclose(score(7, 3), score(107, 103), atol=1e-10)
    assert np.allclose(score(0, 0), np.sum(q * k, axis=-1), atol=1e-12)   # no offset: plain dot
    assert not np.allclose(score(7, 3), score(7, 4))
    # rotations keep every vector's norm
    assert np.allclose(np.linalg.norm(orc.rope(q, [12345], 500.0), axis=-1), np.linalg.norm(q, axis=-1))


def test_rope_prefill_then_decode_uses_the_same_positions():
    """With RoPE, decode at real index T (position M + T) continues prefill(T) exactly as row T of
    prefill(T+1): meta at positions 0..M-1, real token t at M + t, K rotated before caching."""
    s = SMALL.with_(window=5, rope_base=50.0)
    case = make_prefill_case(s, 1, 12, seed=91)
    T = 11
    full = orc.layer_forward(case.params, case.x[0])
    pre = orc.layer_forward(case.params, case.x[0, :T])
    C = 5
    kc = np.zeros((s.n_kv_heads, C, s.head_dim))
    vc = np.zeros_like(kc)
    for t in range(T - C, T):
        kc[:, t % C] = pre.K[s.n_meta + t]
        vc[:, t % C] = pre.V[s.n_meta + t]
    km, vm = orc.meta_kv(case.params)
    assert np.allclose(km, full.K[:s.n_meta], atol=1e-12)
    d = orc.decode_step(case.params, case.x[0, T], T, kc, vc, pre.h_final, km, vm)
    assert np.allclose(d.Y, full.Y[T], rtol=1e-10, atol=1e-12)
    # and RoPE changes the result (the base is not silently ignored)
    plain = orc.layer_forward(make_prefill_case(s.with_(rope_base=0.0), 1, 12, seed=91).params, case.x[0])
    assert not np.allclose(plain.Y, full.Y)
