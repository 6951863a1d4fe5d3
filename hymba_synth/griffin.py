"""Seeded synthetic inputs for the Griffin recurrent block (no arithmetic of the method here).

Shapes follow the Griffin summary (hyeon-jae.tistory.com), section 2.3 "Recurrent block" and
section 2.4 "Real-Gated Linear Recurrent Unit": two linear branches D -> D_RNN, a separable
Conv1D of temporal width 4 (4 * D_RNN parameters), the RG-LRU with recurrence weight
a = sigmoid(Lambda) and the constant c = 8, and an output projection D_RNN -> D.
Initialisation as the summary states it: W_a, W_x (and the other linear layers) LeCun,
N(0, 1/fan_in); Lambda such that a^c is uniform on [0.9, 0.999]; Hawk's width D_RNN ~ 4D/3.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import numpy as np

from .generate import _store, draw_normal


@dataclass(frozen=True)
class GriffinShape:
    d_model: int
    d_rnn: int
    dtype: str            # "f32" or "bf16" (storage of x, y and the weight matrices)
    conv_width: int = 4
    c: float = 8.0

    def with_(self, **kw) -> "GriffinShape":
        return replace(self, **kw)


@dataclass
class GriffinParams:
    shape: GriffinShape
    w_in: np.ndarray      # [2 R, D]: rows [0, R) the recurrent branch, [R, 2R) the GeLU branch
    conv_w: np.ndarray    # [width, R]: tap k multiplies the input k steps back
    w_gate: np.ndarray    # [2 R, R]: rows [0, R) W_a (recurrence gate), [R, 2R) W_x (input gate)
    lam: np.ndarray       # [R] Lambda
    w_out: np.ndarray     # [D, R]


def make_griffin_params(rng: np.random.Generator, s: GriffinShape) -> GriffinParams:
    """Draw order: W_in, conv, W_gate, Lambda, W_out."""
    D, R = s.d_model, s.d_rnn
    w_in = _store(draw_normal(rng, (2 * R, D), 1.0 / np.sqrt(D)), s.dtype)
    conv_w = draw_normal(rng, (s.conv_width, R), 1.0 / np.sqrt(s.conv_width)).astype(np.float32)
    w_gate = _store(draw_normal(rng, (2 * R, R), 1.0 / np.sqrt(R)), s.dtype)
    ac = rng.uniform(0.9, 0.999, R)                      # a^c
    a = ac ** (1.0 / s.c)
    lam = np.log(a / (1.0 - a)).astype(np.float32)       # sigmoid(lam) = a
    w_out = _store(draw_normal(rng, (D, R), 1.0 / np.sqrt(R)), s.dtype)
    return GriffinParams(s, w_in, conv_w, w_gate, lam, w_out)


@dataclass
class GriffinCase:
    shape: GriffinShape
    batch: int
    seq: int
    x: np.ndarray         # [B, T, D]
    params: GriffinParams


def make_griffin_case(shape: GriffinShape, batch: int, seq: int, seed: int,
                      params: Optional[GriffinParams] = None) -> GriffinCase:
    rng = np.random.Generator(np.random.PCG64(seed))
    p = params if params is not None else make_griffin_params(rng, shape)
    x = _store(draw_normal(rng, (batch, seq, shape.d_model)), shape.dtype)
    return GriffinCase(shape, batch, seq, x, p)


# the block at the 1.5B mixer's scale (D_RNN = 4D/3) and a tiny fp32 case
GRIFFIN_SMALL = GriffinShape(d_model=64, d_rnn=96, dtype="f32")
GRIFFIN_8K = GriffinShape(d_model=1536, d_rnn=2048, dtype="bf16")
