"""Pins of the Griffin recurrent-block oracle against closed forms (CPU)."""
import math

import numpy as np
import pytest

from hymba_synth.griffin import GRIFFIN_SMALL, make_griffin_case, make_griffin_params
from oracle import griffin_oracle as go


def test_gelu_matches_the_normal_cdf_at_known_points():
    # Phi(1) = 0.8413447460685429, Phi(-1) = 1 - Phi(1) (standard normal table values)
    assert go.gelu(1.0) == pytest.approx(0.8413447460685429, abs=1e-15)
    assert go.gelu(-1.0) == pytest.approx(-(1 - 0.8413447460685429), abs=1e-15)
    assert go.gelu(0.0) == 0.0
    assert go.gelu(8.0) == pytest.approx(8.0, abs=1e-12)
    assert abs(go.gelu(-8.0)) < 1e-12


def test_conv_impulse_response_and_causality():
    R, W = 3, 4
    w = np.arange(1, W * R + 1, dtype=float).reshape(W, R)
    u = np.zeros((7, R))
    u[2] = 1.0
    out = go.causal_conv(u, w)
    assert np.allclose(out[:2], 0.0)                 # nothing before the impulse
    for k in range(W):
        assert np.allclose(out[2 + k], w[k])         # tap k shows k steps later
    assert np.allclose(out[2 + W:], 0.0)
    hist = np.array([[5.0] * R, [0.0] * R, [0.0] * R])  # oldest first: 3 steps before t = 0
    out2 = go.causal_conv(np.zeros((2, R)), w, hist)
    assert np.allclose(out2[0], 5.0 * w[3]) and np.allclose(out2[1], 0.0)


def test_rglru_constant_inputs_follow_the_geometric_series():
    """sigmoid(lam) = 1/2, c = 8, r = 1/2 -> a = (1/2)^4; h_t = b (1 - a^t) / (1 - a)."""
    T, R = 12, 2
    lam = np.zeros(R)                                 # sigmoid(0) = 1/2
    rho = np.zeros((T, R))                            # r = 1/2
    iota = np.full((T, R), math.log(3.0))             # i = 3/4
    xc = np.full((T, R), 2.0)
    h, hT = go.rglru(xc, rho, iota, lam, 8.0)
    a = 0.5 ** 4
    b = math.sqrt(1 - a * a) * 0.75 * 2.0
    for t in range(T):
        assert h[t, 0] == pytest.approx(b * (1 - a ** (t + 1)) / (1 - a), rel=1e-13)
    assert np.allclose(hT, h[-1])


def test_rglru_closed_gate_keeps_the_state():
    """r -> 0: a -> 1 and sqrt(1 - a^2) -> 0, so the state passes through unchanged."""
    T, R = 5, 3
    h0 = np.array([1.0, -2.0, 0.5])
    h, _ = go.rglru(np.ones((T, R)), np.full((T, R), -80.0), np.zeros((T, R)), np.zeros(R), 8.0, h0)
    assert np.allclose(h, h0[None, :], atol=1e-12)


def test_block_prefill_then_decode_continues():
    """The block on T + 1 tokens equals the block on T tokens followed by one more token from the
    handed state (the last width - 1 branch inputs and h)."""
    case = make_griffin_case(GRIFFIN_SMALL, 1, 21, seed=3)
    x = case.x[0]
    full = go.griffin_block(case.params, x)
    head = go.griffin_block(case.params, x[:20])
    tail = go.griffin_block(case.params, x[20:], head.conv_state, head.h_T)
    assert np.allclose(tail.Y[0], full.Y[20], rtol=1e-12, atol=1e-12)
    assert np.allclose(tail.h_T, full.h_T, rtol=1e-12, atol=1e-12)


def test_lambda_init_puts_a_power_c_in_range():
    p = make_griffin_params(np.random.Generator(np.random.PCG64(1)), GRIFFIN_SMALL)
    ac = go.sigmoid(p.lam) ** GRIFFIN_SMALL.c
    assert np.all(ac > 0.9 - 1e-6) and np.all(ac < 0.999 + 1e-6)


# ---- the block's composition, pinned by a hand-worked case (tests/golden/handworked.json) ----

import json
import os

from hymba_synth.griffin import GriffinParams, GriffinShape

_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "handworked.json")


def _golden_block():
    g = json.load(open(_GOLDEN))["griffin_block"]
    ev = lambda s: float(eval(str(s), {"__builtins__": {}}, {"log": math.log, "sqrt": math.sqrt,   # noqa: E731
                                                               "Phi1": g["Phi1"]}))
    arr = lambda a: np.array([[ev(v) for v in row] for row in a], dtype=float)   # noqa: E731
    shape = GriffinShape(d_model=g["d_model"], d_rnn=g["d_rnn"], dtype="f32", c=g["c"])
    p = GriffinParams(shape, arr(g["w_in"]), arr(g["conv_w"]), arr(g["w_gate"]), np.array(g["lam"], float),
                      arr(g["w_out"]))
    x = arr(g["x"])
    return p, x, np.array([ev(s) for s in g["expected_h"]]), np.array([ev(s) for s in g["expected_Y"]])


def test_block_matches_the_handworked_case():
    p, x, h_ref, y_ref = _golden_block()
    out = go.griffin_block(p, x)
    assert np.allclose(out.h[:, 0], h_ref, rtol=1e-13, atol=1e-15)
    assert np.allclose(out.Y[:, 0], y_ref, rtol=1e-13, atol=1e-15)
    assert np.allclose(out.xc[:, 0], [1.0, -0.5], rtol=0, atol=1e-15)


def _composed(p, x, recur_in="u", gate_src="xc", gelu_on="v", conv_on="u"):
    """The block assembled from the oracle's pieces with one part moved (a planted mistake)."""
    R = p.shape.d_rnn
    P = np.asarray(x, float) @ np.asarray(p.w_in, float).T
    br = {"u": P[:, :R], "v": P[:, R:]}
    xc = go.causal_conv(br[conv_on], p.conv_w)
    src = {"xc": xc, "x": np.asarray(x, float), "u": br["u"]}[gate_src]
    G = src @ np.asarray(p.w_gate, float).T
    h, _ = go.rglru(xc if recur_in == "u" else br["v"], G[:, :R], G[:, R:], p.lam, p.shape.c)
    other = br["v"] if gelu_on == "v" else br["u"]
    Y = (h * go.gelu(other)) if gelu_on != "h" else (go.gelu(h) * br["v"])
    return Y @ np.asarray(p.w_out, float).T


@pytest.mark.parametrize("mistake", [
    dict(conv_on="v", gelu_on="u"),     # branches swapped
    dict(gelu_on="h"),                  # GeLU on the recurrent branch instead of the other one
    dict(conv_on="v"),                  # the conv applied to the GeLU branch's input
    dict(gate_src="x"),                 # gates fed the block input instead of the conv output
    dict(gate_src="u"),                 # gates fed the branch input before the conv
])
def test_planted_composition_mistakes_fail_the_handworked_case(mistake):
    p, x, _, y_ref = _golden_block()
    assert np.allclose(_composed(p, x)[:, 0], y_ref, rtol=1e-13)        # the unchanged assembly passes
    bad = _composed(p, x, **mistake)[:, 0]
    assert np.max(np.abs(bad - y_ref)) > 1e-3 * np.max(np.abs(y_ref)), mistake
