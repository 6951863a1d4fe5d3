"""Layer shapes and the five workloads of the hybrid-head mixer.

Shapes follow the Hymba model family (Hymba summary, greeksharifa.github.io,
section 2.5 "Hymba Model Family" / Table 11: hidden 1600 for 1.5B, local window
1024, SSM state 16, 128 meta tokens from section 2.3) and the 300M ablation
scale (section 2 roadmap).  Head counts, head dim and SSM width are fixed here;
the pages do not give them.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional


@dataclass(frozen=True)
class LayerShape:
    d_model: int
    n_heads: int
    head_dim: int
    n_kv_heads: int
    d_inner: int
    d_state: int
    n_meta: int
    window: int          # > 0: sliding window over real tokens (incl. self); 0: global causal
    own_kv: bool         # True: the layer projects its own K/V; False: K/V come from the previous layer
    dtype: str           # "f32" or "bf16" (storage); state and accumulation are fp32 in both
    rms_eps: float = 1e-6
    rope_base: float = 0.0   # > 0: rotary position encoding of q and k with this base; 0: none

    @property
    def q_width(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_width(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def n_in(self) -> int:
        """Columns of the shared input projection: [Q|K|V|U|Z|dt|B|C] (no K,V for a consumer)."""
        kv = 2 * self.kv_width if self.own_kv else 0
        return self.q_width + kv + 3 * self.d_inner + 2 * self.d_state

    def with_(self, **kw) -> "LayerShape":
        return replace(self, **kw)


@dataclass(frozen=True)
class Config:
    seed: int                      # base seed of the workload's inputs
    name: str
    kind: str                      # "prefill" or "decode"
    batch: int
    seq: int                       # prefill: real tokens per sequence; decode: real tokens already cached
    shape: LayerShape
    consumer_shape: Optional[LayerShape] = None   # decode pair: the KV-sharing partner
    note: str = ""


_C0 = LayerShape(d_model=64, n_heads=2, head_dim=32, n_kv_heads=2, d_inner=64, d_state=8,
                 n_meta=16, window=32, own_kv=True, dtype="f32")
_C1 = LayerShape(d_model=1024, n_heads=16, head_dim=64, n_kv_heads=4, d_inner=2048, d_state=16,
                 n_meta=128, window=1024, own_kv=True, dtype="bf16")
_15B = LayerShape(d_model=1600, n_heads=25, head_dim=64, n_kv_heads=5, d_inner=3200, d_state=16,
                  n_meta=128, window=1024, own_kv=True, dtype="bf16")

WORKLOADS = [
    Config(1000, "tiny-f32", "prefill", 1, 128, _C0,
           note="tiny fp32 mixer, SWA 32, 16 meta tokens"),
    Config(1001, "300m-ablation-swa", "prefill", 8, 2048, _C1,
           note="300M-ablation-shaped SWA layer, bf16"),
    Config(1002, "1.5b-swa-8k-kvshare", "prefill", 16, 8192, _15B.with_(own_kv=False),
           note="1.5B-shaped SWA layer at 8K, K/V handed from the preceding layer"),
    Config(1003, "1.5b-global-8k", "prefill", 8, 8192, _15B.with_(window=0),
           note="1.5B-shaped global-attention layer at 8K"),
    Config(1004, "1.5b-decode-b128", "decode", 128, 8192, _15B,
           consumer_shape=_15B.with_(own_kv=False),
           note="decode step at real index 8192, SWA ring 1024 shared by a producer/consumer pair"),
]


TINY_F32 = "tiny-f32"
ABLATION_300M = "300m-ablation-swa"
SWA_8K = "1.5b-swa-8k-kvshare"
GLOBAL_8K = "1.5b-global-8k"
DECODE_B128 = "1.5b-decode-b128"


def workload(name: str) -> Config:
    """The workload of that name (KeyError for an unknown one)."""
    for c in WORKLOADS:
        if c.name == name:
            return c
    raise KeyError(name)
