"""Convenience wrapper over the C-ABI: device memory (torch) and streams around one layer.

Every computation runs in libhymba_mixer.so; this module only uploads
weights, owns the persistent buffer and a workspace, and passes pointers.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import _lib as L


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def torch_dtype(dtype: str) -> torch.dtype:
    """Storage type of a layer's x, y and weight matrices."""
    return {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]


def act_dtype(dtype: str) -> torch.dtype:
    """Activation type of a layer: the type of the K/V it exchanges and caches."""
    return {"bf16": torch.float16, "f32": torch.float32}[dtype]


def upload(a, dtype: torch.dtype, device) -> torch.Tensor:
    """numpy (or tensor) -> contiguous device tensor of `dtype`."""
    t = torch.as_tensor(np.ascontiguousarray(a)) if isinstance(a, np.ndarray) else a
    return t.to(device=device, dtype=dtype).contiguous()


def make_kv(k_meta=None, v_meta=None, k=None, v=None, k_cache=None, v_cache=None) -> L.hymba_kv:
    kv = L.hymba_kv()
    kv.k_meta, kv.v_meta = _ptr(k_meta), _ptr(v_meta)
    kv.k, kv.v = _ptr(k), _ptr(v)
    kv.k_cache, kv.v_cache = _ptr(k_cache), _ptr(v_cache)
    kv.cache_len = 0 if k_cache is None else int(k_cache.shape[2])
    return kv


class MixerLayer:
    """One hybrid-head mixer layer on the current GPU.

    `shape` has the fields of a layer configuration (d_model, n_heads, head_dim,
    n_kv_heads, d_inner, d_state, n_meta, window, own_kv, dtype, rms_eps and,
    optionally, rope_base);
    `params` has meta, w_in, w_o, w_out, A, D, dt_bias, beta1, beta2 arrays.
    """

    def __init__(self, shape, params, device="cuda"):
        self.shape = shape
        self.device = torch.device(device)
        self.dtype = torch_dtype(shape.dtype)
        self.act_dtype = act_dtype(shape.dtype)
        f32 = torch.float32
        self.w_in = upload(params.w_in, self.dtype, self.device)
        self.w_o = upload(params.w_o, self.dtype, self.device)
        self.w_out = upload(params.w_out, self.dtype, self.device)
        self.meta = upload(params.meta, self.dtype, self.device) if shape.n_meta > 0 else None
        self.A = upload(params.A, f32, self.device)
        self.D = upload(params.D, f32, self.device)
        self.dt_bias = upload(params.dt_bias, f32, self.device)
        self.beta1 = upload(params.beta1, f32, self.device)
        self.beta2 = upload(params.beta2, f32, self.device)
        cfg = L.hymba_layer_cfg()
        cfg.d_model, cfg.n_heads, cfg.n_kv_heads = shape.d_model, shape.n_heads, shape.n_kv_heads
        cfg.head_dim, cfg.d_inner, cfg.d_state = shape.head_dim, shape.d_inner, shape.d_state
        cfg.n_meta, cfg.window, cfg.own_kv = shape.n_meta, shape.window, int(shape.own_kv)
        cfg.dtype = L.HYMBA_BF16 if shape.dtype == "bf16" else L.HYMBA_F32
        cfg.rms_eps = shape.rms_eps
        cfg.rope_base = getattr(shape, "rope_base", 0.0)
        self.cfg = cfg
        w = L.hymba_layer_weights()
        w.w_in, w.w_o, w.w_out, w.meta = _ptr(self.w_in), _ptr(self.w_o), _ptr(self.w_out), _ptr(self.meta)
        w.A, w.D, w.dt_bias = _ptr(self.A), _ptr(self.D), _ptr(self.dt_bias)
        w.beta1, w.beta2 = _ptr(self.beta1), _ptr(self.beta2)
        self.weights = w
        nbytes = L.hymba_layer_persistent_bytes(cfg)
        if nbytes == 0:
            raise L.HymbaError(L.HYMBA_ERR_INVALID_ARG, L.hymba_last_error())
        self.persistent = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        base = self.persistent.data_ptr()
        self._pbase = (base + 255) // 256 * 256
        self.handle = L.hymba_layer_create(cfg, w, self._pbase, nbytes)
        self._ws: Optional[torch.Tensor] = None

    # -- memory ------------------------------------------------------------------
    def workspace(self, batch: int, seq: int) -> torch.Tensor:
        need = L.hymba_mixer_workspace_bytes(self.handle, batch, seq)
        if self._ws is None or self._ws.numel() < need:
            self._ws = None
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._ws

    @staticmethod
    def stream() -> int:
        return torch.cuda.current_stream().cuda_stream

    # -- the C-ABI calls -----------------------------------------------------------
    def bind(self, producer: Optional["MixerLayer"]) -> None:
        L.hymba_kv_share_bind(self.handle, None if producer is None else producer.handle)

    def prepare(self, kv: Optional[L.hymba_kv] = None) -> None:
        ws = self.workspace(1, 1)
        L.hymba_layer_prepare(self.handle, kv, ws.data_ptr(), ws.numel(), self.stream())

    def prefill(self, x: torch.Tensor, kv: Optional[L.hymba_kv] = None, state_out: Optional[torch.Tensor] = None,
                y: Optional[torch.Tensor] = None) -> torch.Tensor:
        B, T, d = x.shape
        assert d == self.shape.d_model and x.dtype == self.dtype and x.is_contiguous()
        if y is None:
            y = torch.empty_like(x)
        if state_out is not None:
            assert state_out.shape == (B, self.shape.d_inner, self.shape.d_state) and state_out.dtype == torch.float32
        ws = self.workspace(B, T)
        L.hymba_mixer_prefill(self.handle, x.data_ptr(), B, T, y.data_ptr(), kv, _ptr(state_out), ws.data_ptr(),
                              ws.numel(), self.stream())
        return y

    def decode(self, x: torch.Tensor, pos: torch.Tensor, kv: L.hymba_kv, state: torch.Tensor,
               y: Optional[torch.Tensor] = None) -> torch.Tensor:
        B, d = x.shape
        assert d == self.shape.d_model and x.dtype == self.dtype and x.is_contiguous()
        assert pos.dtype == torch.int64 and pos.numel() == B and pos.is_cuda
        assert state.shape == (B, self.shape.d_inner, self.shape.d_state) and state.dtype == torch.float32
        if y is None:
            y = torch.empty_like(x)
        ws = self.workspace(B, 1)
        L.hymba_mixer_decode(self.handle, x.data_ptr(), pos.data_ptr(), B, y.data_ptr(), kv, state.data_ptr(),
                             ws.data_ptr(), ws.numel(), self.stream())
        return y

    def check(self) -> None:
        """Raises HymbaError(HYMBA_ERR_RANGE) if a device-side check failed since the last check."""
        L.hymba_layer_check(self.handle, self.stream())

    def set_overlap(self, enable: bool) -> None:
        L.hymba_layer_set_overlap(self.handle, enable)

    def set_gemm(self, backend: int) -> None:
        """bf16 prefill projections: HYMBA_GEMM_LIBRARY (0, hipBLASLt, the default) or HYMBA_GEMM_TILED
        (1, the hand-written tiled matrix-core GEMM)."""
        L.hymba_layer_set_gemm(self.handle, backend)

    def meta_outputs(self):
        """(k_meta, v_meta, h_meta, y_meta) as device tensors viewing the persistent buffer."""
        s = self.shape
        kp, vp, hp, yp = L.hymba_layer_meta_outputs(self.handle)
        es = 2 if s.dtype == "bf16" else 4
        base = self.persistent.data_ptr()

        def view(ptr, nelem, dtype, shape):
            if ptr is None:
                return None
            off = ptr - base
            nbytes = nelem * (2 if dtype in (torch.bfloat16, torch.float16) else 4)
            return self.persistent[off:off + nbytes].view(dtype).view(*shape)

        M, Hkv, hd = s.n_meta, s.n_kv_heads, s.head_dim
        del es
        return (view(kp, M * Hkv * hd, self.act_dtype, (M, Hkv, hd)),
                view(vp, M * Hkv * hd, self.act_dtype, (M, Hkv, hd)),
                view(hp, s.d_inner * s.d_state, torch.float32, (s.d_inner, s.d_state)),
                view(yp, M * s.d_model, self.dtype, (M, s.d_model)))

    def close(self) -> None:
        if getattr(self, "handle", None):
            L.hymba_layer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
