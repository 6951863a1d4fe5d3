"""Seeded generators for mixer inputs and parameters.

Recipe (the same for every workload):
  * generator: numpy PCG64 seeded with 1000 + workload id (tests pass their own seed);
  * draw order: X, meta rows R, W_in, W_O, W_out, A, D, beta1, beta2, then workload extras;
  * activations X and meta rows R ~ N(0, 1);
  * weights ~ N(0, 1/fan_in), stored [out_features, in_features];
  * dt bias = -2, so a unit-variance projection gives dt = softplus(N(0,1) - 2);
  * A[c, n] = -exp(u), u ~ U[ln 1, ln 8];  D ~ N(0, 1);  beta1, beta2 ~ U[0.5, 1.5];
  * bf16 workloads round X, R and the three weight matrices (and any handed K/V)
    to bf16 once (round-to-nearest-even); A, D, dt bias, beta and SSM states stay fp32.
All arrays are returned as float32 numpy arrays holding exactly the stored values.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import Config, LayerShape, workload

DT_BIAS = -2.0


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
    out = ((bits + bias) & np.uint32(0xFFFF0000)).view(np.float32)
    return out


def draw_normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_round(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


@dataclass
class LayerParams:
    shape: LayerShape
    meta: np.ndarray      # [M, d]
    w_in: np.ndarray      # [n_in, d]
    w_o: np.ndarray       # [E, H*hd]
    w_out: np.ndarray     # [d, E]
    A: np.ndarray         # [E, N] fp32
    D: np.ndarray         # [E] fp32
    dt_bias: np.ndarray   # [E] fp32
    beta1: np.ndarray     # [E] fp32
    beta2: np.ndarray     # [E] fp32


def make_layer_params(rng: np.random.Generator, s: LayerShape) -> LayerParams:
    """Draw one layer's parameters in the documented order (R, W_in, W_O, W_out, A, D, beta1, beta2)."""
    meta = _store(draw_normal(rng, (s.n_meta, s.d_model)), s.dtype)
    w_in = _store(draw_normal(rng, (s.n_in, s.d_model), 1.0 / np.sqrt(s.d_model)), s.dtype)
    w_o = _store(draw_normal(rng, (s.d_inner, s.q_width), 1.0 / np.sqrt(s.q_width)), s.dtype)
    w_out = _store(draw_normal(rng, (s.d_model, s.d_inner), 1.0 / np.sqrt(s.d_inner)), s.dtype)
    u = rng.uniform(np.log(1.0), np.log(8.0), size=(s.d_inner, s.d_state))
    A = (-np.exp(u)).astype(np.float32)
    D = draw_normal(rng, (s.d_inner,))
    beta1 = rng.uniform(0.5, 1.5, size=s.d_inner).astype(np.float32)
    beta2 = rng.uniform(0.5, 1.5, size=s.d_inner).astype(np.float32)
    dt_bias = np.full(s.d_inner, DT_BIAS, dtype=np.float32)
    return LayerParams(s, meta, w_in, w_o, w_out, A, D, dt_bias, beta1, beta2)


@dataclass
class PrefillCase:
    shape: LayerShape
    batch: int
    seq: int
    x: np.ndarray                          # [B, T, d]
    params: LayerParams
    # handed K/V for a consumer layer (None for a layer that owns its K/V)
    k_meta: Optional[np.ndarray] = None    # [M, Hkv, hd]
    v_meta: Optional[np.ndarray] = None
    k: Optional[np.ndarray] = None         # [B, T, Hkv, hd]
    v: Optional[np.ndarray] = None


def make_prefill_case(shape: LayerShape, batch: int, seq: int, seed: int) -> PrefillCase:
    rng = np.random.Generator(np.random.PCG64(seed))
    x = _store(draw_normal(rng, (batch, seq, shape.d_model)), shape.dtype)
    params = make_layer_params(rng, shape)
    case = PrefillCase(shape, batch, seq, x, params)
    if not shape.own_kv:
        hk = (shape.n_kv_heads, shape.head_dim)
        case.k_meta = _store(draw_normal(rng, (shape.n_meta,) + hk), shape.dtype)
        case.v_meta = _store(draw_normal(rng, (shape.n_meta,) + hk), shape.dtype)
        case.k = _store(draw_normal(rng, (batch, seq) + hk), shape.dtype)
        case.v = _store(draw_normal(rng, (batch, seq) + hk), shape.dtype)
    return case


@dataclass
class DecodeCase:
    shape: LayerShape                # producer (owns K/V)
    consumer_shape: LayerShape       # consumer (reads the producer's K/V)
    batch: int
    x: np.ndarray                    # [B, d] input of the producer layer
    pos: np.ndarray                  # [B] int64 real-token index of the new token
    producer: LayerParams
    consumer: LayerParams
    k_cache: np.ndarray              # [B, Hkv, C, hd] ring (C = window) shared by the pair
    v_cache: np.ndarray
    state_p: np.ndarray              # [B, E, N] fp32 SSM state of the producer
    state_c: np.ndarray              # [B, E, N] fp32 SSM state of the consumer
    x_c: np.ndarray                  # [B, d] input of the consumer layer


def make_decode_case(shape: LayerShape, consumer_shape: LayerShape, batch: int, pos: int,
                     seed: int, cache_len: Optional[int] = None) -> DecodeCase:
    rng = np.random.Generator(np.random.PCG64(seed))
    x = _store(draw_normal(rng, (batch, shape.d_model)), shape.dtype)
    prod = make_layer_params(rng, shape)
    cons = make_layer_params(rng, consumer_shape)
    C = cache_len if cache_len is not None else shape.window
    hk = (batch, shape.n_kv_heads, C, shape.head_dim)
    k_cache = _store(draw_normal(rng, hk), shape.dtype)
    v_cache = _store(draw_normal(rng, hk), shape.dtype)
    state_p = draw_normal(rng, (batch, shape.d_inner, shape.d_state))
    state_c = draw_normal(rng, (batch, consumer_shape.d_inner, consumer_shape.d_state))
    x_c = _store(draw_normal(rng, (batch, consumer_shape.d_model)), shape.dtype)
    posv = np.full(batch, pos, dtype=np.int64)
    return DecodeCase(shape, consumer_shape, batch, x, posv, prod, cons, k_cache, v_cache,
                      state_p, state_c, x_c)


def make_config_case(name: str):
    """The named workload's inputs, seeded with its base seed."""
    cfg: Config = workload(name)
    seed = cfg.seed
    if cfg.kind == "prefill":
        return make_prefill_case(cfg.shape, cfg.batch, cfg.seq, seed)
    return make_decode_case(cfg.shape, cfg.consumer_shape, cfg.batch, cfg.seq, seed)
