"""Convenience wrapper over the Griffin block's C-ABI: device memory (torch) around one block.

Every computation runs in libhymba_mixer.so; this module uploads weights, owns a workspace and
passes pointers.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib as L
from .layer import torch_dtype, upload


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


class GriffinBlock:
    """The recurrent block of a Griffin shape (d_model, d_rnn, dtype, c) with params w_in, conv_w,
    w_gate, lam, w_out."""

    def __init__(self, shape, params, device="cuda"):
        self.shape = shape
        self.device = torch.device(device)
        self.dtype = torch_dtype(shape.dtype)
        f32 = torch.float32
        self.w_in = upload(params.w_in, self.dtype, self.device)
        self.conv_w = upload(params.conv_w, f32, self.device)
        self.w_gate = upload(params.w_gate, self.dtype, self.device)
        self.lam = upload(params.lam, f32, self.device)
        self.w_out = upload(params.w_out, self.dtype, self.device)
        self.cfg = L.griffin_block_cfg()
        self.cfg.d_model, self.cfg.d_rnn, self.cfg.c = shape.d_model, shape.d_rnn, shape.c
        self.cfg.dtype = L.HYMBA_BF16 if shape.dtype == "bf16" else L.HYMBA_F32
        self.w = L.griffin_block_weights()
        self.w.w_in, self.w.conv_w, self.w.w_gate = _ptr(self.w_in), _ptr(self.conv_w), _ptr(self.w_gate)
        self.w.lam, self.w.w_out = _ptr(self.lam), _ptr(self.w_out)
        self._ws = None
        n = L.griffin_block_persistent_bytes(self.cfg)
        self.persistent = torch.empty(max(n, 256), dtype=torch.uint8, device=self.device) if n else None
        L.griffin_block_prepare(self.cfg, self.w, _ptr(self.persistent), n, self._stream())

    def _stream(self):
        return torch.cuda.current_stream(self.device).cuda_stream

    def workspace(self, B: int, T: int) -> torch.Tensor:
        need = L.griffin_workspace_bytes(self.cfg, B, T)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
        return self._ws

    def new_state(self, B: int):
        R = self.shape.d_rnn
        return (torch.zeros(B, 3, R, dtype=torch.float32, device=self.device),
                torch.zeros(B, R, dtype=torch.float32, device=self.device))

    def prefill(self, x: torch.Tensor, conv_state=None, h=None, conv_state_out=None, h_out=None,
                y: Optional[torch.Tensor] = None, timed: bool = False):
        B, T, D = x.shape
        if y is None:
            y = torch.empty(B, T, D, dtype=self.dtype, device=self.device)
        ws = self.workspace(B, T)
        ms = L.griffin_block_prefill(self.cfg, self.w, _ptr(self.persistent), x.data_ptr(), B, T, y.data_ptr(),
                                     _ptr(conv_state), _ptr(h), _ptr(conv_state_out), _ptr(h_out), ws.data_ptr(),
                                     ws.numel(), self._stream(), timed)
        return (y, ms) if timed else y

    def decode(self, x_t: torch.Tensor, conv_state: torch.Tensor, h: torch.Tensor,
               y_t: Optional[torch.Tensor] = None) -> torch.Tensor:
        B, D = x_t.shape
        if y_t is None:
            y_t = torch.empty(B, D, dtype=self.dtype, device=self.device)
        ws = self.workspace(B, 1)
        L.griffin_block_decode(self.cfg, self.w, _ptr(self.persistent), x_t.data_ptr(), B, y_t.data_ptr(),
                               conv_state.data_ptr(), h.data_ptr(), ws.data_ptr(), ws.numel(), self._stream())
        return y_t
