"""Layer-level parity of hymba_mixer_prefill / hymba_mixer_decode / hymba_kv_share_bind
against the fp64 oracle, through the C ABI.

Small layers are checked on every sequence; the four full-size workloads
(300M-ablation SWA layer, 1.5B SWA KV-consumer at 8K, 1.5B global layer at
8K, B=128 decode pair) run in the launch configuration the benchmark times and
are checked on sampled sequences (the oracle computes whole sequences).
"""
import numpy as np
import pytest
import torch

from hymba_synth import (DECODE_B128, GLOBAL_8K, ABLATION_300M, SWA_8K, TINY_F32, LayerShape, make_decode_case,
                         make_prefill_case, workload)
from hymba_synth.generate import make_config_case
from hybrid_attention_ssm_swa_amd import _lib as H
from oracle import hymba_oracle as orc

from gpu_util import MixerLayer, act, announce, check, check_stored, dev, host, make_kv

pytestmark = pytest.mark.gpu


def _prefill_gpu(case, layer=None, state=False, kv_extra=None, gemm=None):
    s = case.shape
    layer = layer or MixerLayer(s, case.params)
    if gemm is not None:
        layer.set_gemm(gemm)
    x = dev(case.x, s.dtype)
    kv = None
    keep = []
    if not s.own_kv:
        t = [dev(a, act(s.dtype)) for a in (case.k_meta, case.v_meta, case.k, case.v)]
        keep += t
        kv = make_kv(*t)
    elif kv_extra is not None:
        kv = kv_extra
    st = torch.empty((case.batch, s.d_inner, s.d_state), dtype=torch.float32, device="cuda") if state else None
    y = layer.prefill(x, kv, st)
    torch.cuda.synchronize()
    return layer, host(y), (host(st) if state else None)


def _check_prefill(case, seqs, dtype, gemm=None):
    layer, y, st = _prefill_gpu(case, state=True, gemm=gemm)
    outs = orc.prefill_batch(case, seqs)
    for b in seqs:
        check_stored(f"Y[b={b}]", y[b], outs[b].Y, dtype)
        check(f"h_T[b={b}]", st[b], outs[b].h_final, dtype)
    return layer, outs


SMALL_BF16 = LayerShape(d_model=256, n_heads=8, head_dim=64, n_kv_heads=2, d_inner=512, d_state=16,
                        n_meta=128, window=64, own_kv=True, dtype="bf16")


@pytest.mark.parametrize("shape,B,T", [
    (SMALL_BF16, 3, 200),
    (SMALL_BF16.with_(window=0), 2, 150),
    (SMALL_BF16.with_(n_meta=0), 2, 97),
    (SMALL_BF16.with_(window=1, n_meta=20), 1, 70),
    (SMALL_BF16, 2, 1),
    (SMALL_BF16.with_(n_kv_heads=8, n_meta=64), 1, 130),
    (workload(TINY_F32).shape.with_(window=5, n_meta=3), 2, 41),
    (SMALL_BF16.with_(rope_base=10000.0), 2, 150),
    (SMALL_BF16.with_(rope_base=500.0, window=0, n_meta=40), 1, 130),
    (workload(TINY_F32).shape.with_(rope_base=100.0), 1, 60),
])
def test_small_layer_prefill(shape, B, T):
    announce(f"small prefill {shape} B={B} T={T}")
    case = make_prefill_case(shape, B, T, seed=7 + T)
    _check_prefill(case, range(B), shape.dtype)


@pytest.mark.parametrize("shape,B,T", [
    (SMALL_BF16, 3, 200),
    (SMALL_BF16.with_(rope_base=10000.0, own_kv=False), 2, 150),
    (SMALL_BF16.with_(window=0, n_meta=0), 2, 333),
])
def test_small_layer_prefill_tiled_gemm(shape, B, T):
    """The prefill projections on the hand-written tiled GEMM (more than 256 rows each)."""
    announce(f"small prefill, tiled GEMM {shape} B={B} T={T}")
    case = make_prefill_case(shape, B, T, seed=17 + T)
    _check_prefill(case, range(B), shape.dtype, gemm=H.HYMBA_GEMM_TILED)


def test_meta_prefix_outputs():
    """The prepared meta prefix (K/V, SSM state, meta-row outputs) equals the oracle's meta rows."""
    for shape in (SMALL_BF16, workload(TINY_F32).shape, SMALL_BF16.with_(rope_base=1000.0)):
        announce(f"meta prefix {shape.dtype}")
        case = make_prefill_case(shape, 1, 8, seed=11)
        layer = MixerLayer(shape, case.params)
        layer.prepare()
        torch.cuda.synchronize()
        km, vm, hm, ym = layer.meta_outputs()
        ref = orc.layer_forward(case.params, case.x[0])
        M = shape.n_meta
        check_stored("K_meta", host(km), ref.K[:M], act(shape.dtype))
        check_stored("V_meta", host(vm), ref.V[:M], act(shape.dtype))
        check("h_meta", host(hm), ref.h_meta, shape.dtype)
        check_stored("Y_meta", host(ym), ref.Y_meta, shape.dtype)


def test_config0_tiny_f32_full():
    announce("tiny fp32 layer, full")
    _check_prefill(make_config_case(TINY_F32), [0], "f32")


def test_config1_full_size():
    announce("300M-ablation SWA layer, 8x2048, full size, all sequences")
    _check_prefill(make_config_case(ABLATION_300M), range(8), "bf16")


def test_config2_full_size_sampled():
    announce("1.5B SWA KV-consumer layer, 16x8192, full size, sequences 0 and 15")
    _check_prefill(make_config_case(SWA_8K), [0, 15], "bf16")


@pytest.mark.parametrize("name,seqs", [(SWA_8K, [0, 15]), (ABLATION_300M, [0, 7])])
def test_full_size_tiled_gemm(name, seqs):
    announce(f"{name}, full size, prefill projections on the tiled GEMM, sequences {seqs}")
    _check_prefill(make_config_case(name), seqs, "bf16", gemm=H.HYMBA_GEMM_TILED)


def test_config3_full_size_sampled():
    announce("1.5B global layer, 8x8192, full size, sequences 0 and 7")
    _check_prefill(make_config_case(GLOBAL_8K), [0, 7], "bf16")


def _decode_pair_gpu(case, cache_len=None):
    s, sc = case.shape, case.consumer_shape
    prod = MixerLayer(s, case.producer)
    cons = MixerLayer(sc, case.consumer)
    cons.bind(prod)
    kc, vc = dev(case.k_cache, act(s.dtype)), dev(case.v_cache, act(s.dtype))
    kv = make_kv(k_cache=kc, v_cache=vc)
    pos = torch.from_numpy(case.pos).cuda()
    stp = torch.from_numpy(case.state_p).cuda()
    stc = torch.from_numpy(case.state_c).cuda()
    prod.prepare()
    cons.prepare()
    yp = prod.decode(dev(case.x, s.dtype), pos, kv, stp)
    yc = cons.decode(dev(case.x_c, sc.dtype), pos, kv, stc)
    torch.cuda.synchronize()
    return prod, cons, host(yp), host(yc), host(stp), host(stc), host(kc), host(vc)


def _decode_pair_oracle(case, seqs):
    kmp, vmp = orc.meta_kv(case.producer)
    out = {}
    for b in seqs:
        p = int(case.pos[b])
        dp = orc.decode_step(case.producer, case.x[b], p, case.k_cache[b], case.v_cache[b], case.state_p[b],
                             kmp, vmp)
        dc = orc.decode_step(case.consumer, case.x_c[b], p, dp.k_cache, dp.v_cache, case.state_c[b], kmp, vmp)
        out[b] = (dp, dc)
    return out


def test_config4_decode_full_size():
    announce("1.5B decode pair, B=128 at 8192, full size, all sequences")
    case = make_config_case(DECODE_B128)
    _, _, yp, yc, stp, stc, kc, vc = _decode_pair_gpu(case)
    ref = _decode_pair_oracle(case, range(case.batch))
    Y_p = np.stack([ref[b][0].Y for b in ref])
    Y_c = np.stack([ref[b][1].Y for b in ref])
    check_stored("producer y", yp, Y_p, "bf16")
    check_stored("consumer y", yc, Y_c, "bf16")
    check("producer state", stp, np.stack([ref[b][0].h for b in ref]), "bf16")
    check("consumer state", stc, np.stack([ref[b][1].h for b in ref]), "bf16")
    slot = 8192 % 1024
    check_stored("written K slot", kc[:, :, slot], np.stack([ref[b][0].k_cache[:, slot] for b in ref]), "f16")
    # every other slot is untouched (the cache holds the fp16 conversion of the handed values)
    other = np.ones(1024, bool)
    other[slot] = False
    f16 = lambda a: a.astype(np.float16).astype(np.float64)
    assert np.array_equal(kc[:, :, other], f16(case.k_cache[:, :, other]))
    assert np.array_equal(vc[:, :, other], f16(case.v_cache[:, :, other]))


def test_global_decode_full_cache():
    """Global-attention decode at the 1.5B global layer's shape: 8 sequences at position 8192 over a
    full cache (every earlier real token plus the meta prefix), producer/consumer pair."""
    announce("global decode B=8, pos 8192, full cache")
    s = workload(GLOBAL_8K).shape
    case = make_decode_case(s, s.with_(own_kv=False), 8, 8192, seed=77, cache_len=8193)
    _, _, yp, yc, stp, stc, kc, _ = _decode_pair_gpu(case)
    ref = _decode_pair_oracle(case, range(case.batch))
    check_stored("producer y", yp, np.stack([ref[b][0].Y for b in ref]), "bf16")
    check_stored("consumer y", yc, np.stack([ref[b][1].Y for b in ref]), "bf16")
    check("consumer state", stc, np.stack([ref[b][1].h for b in ref]), "bf16")
    check_stored("written K slot", kc[:, :, 8192], np.stack([ref[b][0].k_cache[:, 8192] for b in ref]), "f16")


@pytest.mark.parametrize("dtype,rope", [("bf16", 0.0), ("f32", 0.0), ("bf16", 10000.0), ("f32", 300.0)])
def test_decode_small_mixed_positions(dtype, rope):
    """Positions differ per sequence: before the window fills, at the wrap, far beyond."""
    announce(f"decode small {dtype} rope {rope}")
    base = SMALL_BF16 if dtype == "bf16" else workload(TINY_F32).shape.with_(n_meta=6)
    s = base.with_(window=16, rope_base=rope)
    case = make_decode_case(s, s.with_(own_kv=False), 6, 0, seed=21, cache_len=16)
    case.pos = np.array([0, 3, 15, 16, 17, 1000], dtype=np.int64)
    _, _, yp, yc, stp, stc, _, _ = _decode_pair_gpu(case)
    ref = _decode_pair_oracle(case, range(6))
    check_stored("producer y", yp, np.stack([ref[b][0].Y for b in ref]), dtype)
    check_stored("consumer y", yc, np.stack([ref[b][1].Y for b in ref]), dtype)
    check("consumer state", stc, np.stack([ref[b][1].h for b in ref]), dtype)


@pytest.mark.parametrize("rope", [0.0, 10000.0])
def test_kv_share_bound_equals_handed(rope):
    """A consumer bound to its producer gives exactly the output of an unbound consumer handed the
    producer's K/V (spec check on the GPU path), and both match the oracle."""
    announce(f"kv share bound vs handed, rope {rope}")
    s = SMALL_BF16.with_(rope_base=rope)
    r = np.random.Generator(np.random.PCG64(31))
    from hymba_synth import make_layer_params
    prod_p = make_layer_params(r, s)
    cons_p = make_layer_params(r, s.with_(own_kv=False))
    B, T = 2, 150
    x = dev(r.standard_normal((B, T, s.d_model)).astype(np.float32), "bf16")
    xc = dev(r.standard_normal((B, T, s.d_model)).astype(np.float32), "bf16")
    prod = MixerLayer(s, prod_p)
    k = torch.empty((B, T, s.n_kv_heads, s.head_dim), dtype=torch.float16, device="cuda")
    v = torch.empty_like(k)
    prod.prefill(x, make_kv(k=k, v=v))
    kmp, vmp, _, _ = prod.meta_outputs()
    bound = MixerLayer(s.with_(own_kv=False), cons_p)
    bound.bind(prod)
    y_bound = host(bound.prefill(xc, make_kv(k=k, v=v)))
    handed = MixerLayer(s.with_(own_kv=False), cons_p)
    y_handed = host(handed.prefill(xc, make_kv(k_meta=kmp, v_meta=vmp, k=k, v=v)))
    torch.cuda.synchronize()
    assert np.array_equal(y_bound, y_handed)
    # oracle on the K/V the producer produced (rounded to bf16 by the GPU path)
    K = np.concatenate([np.broadcast_to(host(kmp), (B,) + tuple(kmp.shape)), host(k)], axis=1)
    V = np.concatenate([np.broadcast_to(host(vmp), (B,) + tuple(vmp.shape)), host(v)], axis=1)
    M = s.n_meta
    xch = host(xc)
    for b in range(B):
        ref = orc.layer_forward(cons_p, xch[b], K[b, :M], V[b, :M], K[b, M:], V[b, M:])
        check_stored(f"consumer Y[b={b}]", y_bound[b], ref.Y, "bf16")


@pytest.mark.parametrize("window,T,rope", [(16, 40, 0.0), (16, 9, 0.0), (0, 33, 0.0), (16, 40, 10000.0),
                                           (0, 33, 700.0)])
def test_prefill_then_decode_continues(window, T, rope):
    """prefill(T) leaves the cache and state that decode(T) continues from:
    its output equals row T of prefill(T+1) (GPU) and the oracle."""
    announce(f"prefill->decode window={window} T={T} rope={rope}")
    s = SMALL_BF16.with_(window=window, rope_base=rope)
    case = make_prefill_case(s, 2, T + 1, seed=41)
    layer = MixerLayer(s, case.params)
    C = window if window > 0 else T + 8
    kc = torch.zeros((2, s.n_kv_heads, C, s.head_dim), dtype=torch.float16, device="cuda")
    vc = torch.zeros_like(kc)
    st = torch.empty((2, s.d_inner, s.d_state), dtype=torch.float32, device="cuda")
    x = dev(case.x, "bf16")
    layer.prefill(x[:, :T].contiguous(), make_kv(k_cache=kc, v_cache=vc), st)
    pos = torch.full((2,), T, dtype=torch.int64, device="cuda")
    y_dec = host(layer.decode(x[:, T].contiguous(), pos, make_kv(k_cache=kc, v_cache=vc), st))
    y_full = host(layer.prefill(x))
    torch.cuda.synchronize()
    check_stored("decode vs GPU prefill(T+1)", y_dec, y_full[:, T], "bf16")
    for b in range(2):
        ref = orc.layer_forward(case.params, case.x[b])
        check_stored(f"decode vs oracle[b={b}]", y_dec[b], ref.Y[T], "bf16")
