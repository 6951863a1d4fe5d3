"""The prefill -> decode handoff at the 1.5B shapes and a chain of KV-sharing layer pairs.

- An 8192-token prefill of a producer/consumer pair (sliding window 1024, ring cache of 1024
  slots; and global attention over a full cache) leaves the cache and SSM states from which one
  decode step at position 8192 continues: the decode outputs equal row 8192 of the oracle run on
  all 8193 tokens, for the producer and for the consumer that reads its K/V (Hymba summary
  section 2.2: SWA in most layers, global in a few, K/V shared by consecutive layers).
- A chain global producer -> global consumer -> SWA producer -> SWA consumer (RoPE on the global
  pair) sharing caches, rings and SSM states across a prefill and one decode step, checked layer
  by layer: the oracle chain rounds each layer's output to bf16 (the activation stored between
  layers) and feeds it to the next layer; GPU layer i takes those same rows, so each layer is
  held to the single-layer bar and no value of the GPU path enters the oracle.  (A free-running
  GPU chain would carry each layer's rounding into the next, which the single-layer bar does not
  cover.)
"""
import numpy as np
import pytest
import torch

from hymba_synth import GLOBAL_8K, SWA_8K, LayerShape, bf16_round, make_layer_params, workload
from hymba_synth.generate import _store, draw_normal
from oracle import hymba_oracle as orc

from gpu_util import MixerLayer, announce, check, check_stored, dev, host, make_kv

pytestmark = pytest.mark.gpu


def _pair_params(shape, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    pp = make_layer_params(rng, shape.with_(own_kv=True))
    pc = make_layer_params(rng, shape.with_(own_kv=False))
    return rng, pp, pc


def _handoff(shape, B, T, cache_len, seed, seqs):
    sp, sc = shape.with_(own_kv=True), shape.with_(own_kv=False)
    rng, pp, pc = _pair_params(shape, seed)
    x = _store(draw_normal(rng, (B, T + 1, sp.d_model)), "bf16")
    xc = _store(draw_normal(rng, (B, T + 1, sp.d_model)), "bf16")
    prod, cons = MixerLayer(sp, pp), MixerLayer(sc, pc)
    cons.bind(prod)
    hk = (B, sp.n_kv_heads, cache_len, sp.head_dim)
    kc = torch.zeros(hk, dtype=torch.float16, device="cuda")
    vc = torch.zeros_like(kc)
    kf = torch.empty((B, T, sp.n_kv_heads, sp.head_dim), dtype=torch.float16, device="cuda")
    vf = torch.empty_like(kf)
    stp = torch.empty((B, sp.d_inner, sp.d_state), dtype=torch.float32, device="cuda")
    stc = torch.empty_like(stp)
    xd, xcd = dev(x, "bf16"), dev(xc, "bf16")
    yp_pre = prod.prefill(xd[:, :T].contiguous(), make_kv(k=kf, v=vf, k_cache=kc, v_cache=vc), stp)
    yc_pre = cons.prefill(xcd[:, :T].contiguous(), make_kv(k=kf, v=vf), stc)
    pos = torch.full((B,), T, dtype=torch.int64, device="cuda")
    ring = make_kv(k_cache=kc, v_cache=vc)
    yp = prod.decode(xd[:, T].contiguous(), pos, ring, stp)
    yc = cons.decode(xcd[:, T].contiguous(), pos, ring, stc)
    torch.cuda.synchronize()
    prod.check()
    cons.check()
    yp_pre, yc_pre, yp, yc, stp, stc = map(host, (yp_pre, yc_pre, yp, yc, stp, stc))
    M = sp.n_meta
    for b in seqs:
        rp = orc.layer_forward(pp, x[b])                                    # all T + 1 tokens
        rc = orc.layer_forward(pc, xc[b], rp.K[:M], rp.V[:M], rp.K[M:], rp.V[M:])
        check_stored(f"producer prefill Y[b={b}]", yp_pre[b], rp.Y[:T], "bf16")
        check_stored(f"consumer prefill Y[b={b}]", yc_pre[b], rc.Y[:T], "bf16")
        check_stored(f"producer decode y[b={b}] at {T}", yp[b], rp.Y[T], "bf16")
        check_stored(f"consumer decode y[b={b}] at {T}", yc[b], rc.Y[T], "bf16")
        check(f"producer state after decode [b={b}]", stp[b], rp.h_final, "bf16")
        check(f"consumer state after decode [b={b}]", stc[b], rc.h_final, "bf16")


def test_handoff_8k_swa_pair():
    announce("prefill 8192 -> decode at 8192, 1.5B SWA pair, ring of 1024")
    _handoff(workload(SWA_8K).shape, 2, 8192, 1024, seed=501, seqs=[1])


def test_handoff_8k_global_pair():
    announce("prefill 8192 -> decode at 8192, 1.5B global pair, full cache")
    _handoff(workload(GLOBAL_8K).shape, 2, 8192, 8200, seed=503, seqs=[0])


CHAIN = LayerShape(d_model=256, n_heads=8, head_dim=64, n_kv_heads=2, d_inner=512, d_state=16, n_meta=64,
                   window=48, own_kv=True, dtype="bf16")


def test_chain_of_pairs_with_a_global_pair():
    announce("chain: global producer/consumer (RoPE) -> SWA producer/consumer, prefill then one decode step")
    B, T = 2, 300
    g = CHAIN.with_(window=0, rope_base=10000.0)
    shapes = [g, g.with_(own_kv=False), CHAIN, CHAIN.with_(own_kv=False)]
    rng = np.random.Generator(np.random.PCG64(505))
    params = [make_layer_params(rng, s) for s in shapes]
    x = _store(draw_normal(rng, (B, T + 1, CHAIN.d_model)), "bf16")
    # the oracle chain: each layer on the bf16 rows the layer before it stores; a consumer on the
    # K/V of its producer
    M = CHAIN.n_meta
    ref, ins = [], []
    for b in range(B):
        cur, rb, ib = x[b], [], []
        for i, p in enumerate(params):
            ib.append(cur)
            if i % 2 == 0:
                r = orc.layer_forward(p, cur)
                kv_pair = r
            else:
                r = orc.layer_forward(p, cur, kv_pair.K[:M], kv_pair.V[:M], kv_pair.K[M:], kv_pair.V[M:])
            rb.append(r.Y)
            cur = bf16_round(r.Y)
        ref.append(rb)
        ins.append(ib)
    # the GPU chain: the same four layers sharing caches, rings and states across the prefill and
    # the decode step, layer i fed the rows the oracle chain hands to layer i
    layers = [MixerLayer(s, p) for s, p in zip(shapes, params)]
    layers[1].bind(layers[0])
    layers[3].bind(layers[2])
    hkv = (B, T, CHAIN.n_kv_heads, CHAIN.head_dim)
    kf = [torch.empty(hkv, dtype=torch.float16, device="cuda") for _ in range(2)]
    vf = [torch.empty(hkv, dtype=torch.float16, device="cuda") for _ in range(2)]
    caches = [T + 8, CHAIN.window]   # the global pair keeps every token, the SWA pair a ring
    kc = [torch.zeros((B, CHAIN.n_kv_heads, C, CHAIN.head_dim), dtype=torch.float16, device="cuda") for C in caches]
    vc = [torch.zeros_like(k) for k in kc]
    states = [torch.empty((B, s.d_inner, s.d_state), dtype=torch.float32, device="cuda") for s in shapes]
    inputs = [dev(np.stack([ins[b][i] for b in range(B)]), "bf16") for i in range(len(layers))]
    outs = []
    for i, lay in enumerate(layers):
        pair = i // 2
        kv = make_kv(k=kf[pair], v=vf[pair], k_cache=kc[pair], v_cache=vc[pair]) if i % 2 == 0 else \
            make_kv(k=kf[pair], v=vf[pair])
        outs.append(lay.prefill(inputs[i][:, :T].contiguous(), kv, states[i]))
    pos = torch.full((B,), T, dtype=torch.int64, device="cuda")
    douts = []
    for i, lay in enumerate(layers):
        pair = i // 2
        douts.append(lay.decode(inputs[i][:, T].contiguous(), pos, make_kv(k_cache=kc[pair], v_cache=vc[pair]),
                                states[i]))
    torch.cuda.synchronize()
    for lay in layers:
        lay.check()
    outs, douts = [host(o) for o in outs], [host(o) for o in douts]
    for b in range(B):
        for i in range(len(layers)):
            check_stored(f"layer {i} prefill Y[b={b}]", outs[i][b], ref[b][i][:T], "bf16")
            check_stored(f"layer {i} decode y[b={b}] at {T}", douts[i][b], ref[b][i][T], "bf16")
    for lay in reversed(layers):   # consumers before the producers they read
        lay.close()
