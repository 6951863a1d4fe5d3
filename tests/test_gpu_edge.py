"""GPU parity at the numeric edges of the layer, and the device-side checks.

- Delta large (dt_bias = +30): exp(Delta A) underflows to zero for most states, so the state
  is replaced by the step's input every token.
- Delta -> 0 (dt_bias = -30): the state freezes; prefill outputs reduce to the skip term and a
  decode step leaves a handed state unchanged.
- z << 0: the gate SiLU(z) ~ 1e-12 makes the SSM branch's RMS norm epsilon-dominated.
- An input beyond fp16's range (the activation type of bf16 layers): the layer records it and
  hymba_layer_check reports HYMBA_ERR_RANGE instead of passing inf on silently.
- A negative decode position: recorded and reported the same way.
- A bf16 weight beyond fp16's range: recorded when the layer is prepared and reported by every
  check.
- The serial prefill schedule (every kernel on the call's stream) gives the bitwise result of
  the overlapped one.
"""
import numpy as np
import pytest
import torch

import hybrid_attention_ssm_swa_amd as H
from hymba_synth import LayerShape, make_decode_case, make_prefill_case
from oracle import hymba_oracle as orc

from gpu_util import MixerLayer, act, announce, check, check_stored, dev, host, make_kv

pytestmark = pytest.mark.gpu

SMALL = LayerShape(d_model=256, n_heads=8, head_dim=64, n_kv_heads=2, d_inner=512, d_state=16,
                   n_meta=64, window=48, own_kv=True, dtype="bf16")


def _prefill_with_bias(dt_bias, seed):
    case = make_prefill_case(SMALL, 2, 130, seed=seed)
    case.params.dt_bias = np.full(SMALL.d_inner, dt_bias, dtype=np.float32)
    layer = MixerLayer(SMALL, case.params)
    st = torch.empty((2, SMALL.d_inner, SMALL.d_state), dtype=torch.float32, device="cuda")
    y = host(layer.prefill(dev(case.x, "bf16"), None, st))
    torch.cuda.synchronize()
    layer.check()
    return case, y, host(st)


@pytest.mark.parametrize("dt_bias", [30.0, -30.0])
def test_prefill_extreme_delta(dt_bias):
    announce(f"prefill with dt_bias {dt_bias}")
    case, y, st = _prefill_with_bias(dt_bias, seed=91)
    for b in range(2):
        ref = orc.layer_forward(case.params, case.x[b])
        if dt_bias < 0:   # the state never leaves zero: the branch is the skip term alone
            assert np.max(np.abs(ref.h_final)) < 1e-9
        check_stored(f"Y[b={b}]", y[b], ref.Y, "bf16")
        # the final state: all but zero for tiny Delta (absolute bar); else the usual relative bar
        if dt_bias < 0:
            assert np.max(np.abs(st[b])) < 1e-6
        else:
            check(f"h_T[b={b}]", st[b], ref.h_final, "bf16")


def test_decode_tiny_delta_freezes_the_state():
    announce("decode with dt_bias -30: the handed state passes through")
    s = SMALL.with_(window=16)
    case = make_decode_case(s, s.with_(own_kv=False), 4, 40, seed=93, cache_len=16)
    for p in (case.producer, case.consumer):
        p.dt_bias = np.full(s.d_inner, -30.0, dtype=np.float32)
    prod = MixerLayer(s, case.producer)
    kc, vc = dev(case.k_cache, "f16"), dev(case.v_cache, "f16")
    st = torch.from_numpy(case.state_p).cuda()
    pos = torch.from_numpy(case.pos).cuda()
    y = host(prod.decode(dev(case.x, "bf16"), pos, make_kv(k_cache=kc, v_cache=vc), st))
    torch.cuda.synchronize()
    prod.check()
    kmp, vmp = orc.meta_kv(case.producer)
    for b in range(4):
        ref = orc.decode_step(case.producer, case.x[b], int(case.pos[b]), case.k_cache[b], case.v_cache[b],
                              case.state_p[b], kmp, vmp)
        assert np.max(np.abs(ref.h - case.state_p[b])) < 1e-9
        check_stored(f"y[b={b}]", y[b], ref.Y, "bf16")
    assert np.max(np.abs(host(st) - case.state_p)) <= 1e-6 * np.max(np.abs(case.state_p))


def test_epilogue_gate_far_negative():
    """z = -30: g = y SiLU(z) ~ 1e-12, so mean(g^2) << eps and the SSM term is ~1e-9."""
    announce("epilogue with z << 0")
    r = np.random.Generator(np.random.PCG64(95))
    rows, E = 67, 3200
    ao = r.standard_normal((rows, E)).astype(np.float16).astype(np.float32)
    y = (3 * r.standard_normal((rows, E))).astype(np.float16).astype(np.float32)
    z = np.full((rows, E), -30.0, np.float32) + r.uniform(-2, 0, (rows, E)).astype(np.float16).astype(np.float32)
    b1 = r.uniform(0.5, 1.5, E).astype(np.float32)
    b2 = r.uniform(0.5, 1.5, E).astype(np.float32)
    dao, dy, dz = dev(ao, "f16"), dev(y, "f16"), dev(z, "f16")
    f = torch.empty((rows, E), dtype=torch.bfloat16, device="cuda")
    t32 = lambda a: torch.from_numpy(a).cuda()   # noqa: E731
    db1, db2 = t32(b1), t32(b2)
    H.hymba_kernel_epilogue(H.HYMBA_F16, dao.data_ptr(), E, dy.data_ptr(), E, dz.data_ptr(), E, db1.data_ptr(),
                            db2.data_ptr(), f.data_ptr(), E, rows, E, 1e-6, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    g = y.astype(np.float64) * orc.silu(z.astype(np.float64))
    assert np.max(np.mean(g * g, axis=1)) < 1e-12          # epsilon-dominated SSM norm
    ref = orc.fuse(ao.astype(np.float64), g, b1, b2, 1e-6)
    check_stored("F", host(f), ref, "bf16")


def test_input_beyond_fp16_range_is_reported():
    announce("bf16 input beyond fp16's range: hymba_layer_check reports it")
    case = make_prefill_case(SMALL, 2, 40, seed=97)
    layer = MixerLayer(SMALL, case.params)
    x = dev(case.x, "bf16")
    layer.prefill(x)
    layer.check()                                 # an ordinary call passes the check
    x[1, 7] = 1.0e5                               # one token of sequence 1 beyond 65504
    layer.prefill(x)
    with pytest.raises(H.HymbaError) as e:
        layer.check()
    assert e.value.status == H.HYMBA_ERR_RANGE
    layer.check()                                 # the record was cleared
    x[1, 7] = 0.0
    y = host(layer.prefill(x))
    layer.check()
    assert np.all(np.isfinite(y))


def test_weight_beyond_fp16_range_is_reported():
    """A bf16 weight of W_in above 65504 is inf in the layer's fp16 copy: preparing the layer
    records it, and every check reports it (the weights do not change)."""
    announce("bf16 weight beyond fp16's range: hymba_layer_check reports it at every check")
    case = make_prefill_case(SMALL, 1, 20, seed=103)
    case.params.w_in = case.params.w_in.copy()
    case.params.w_in[5, 17] = 1.0e5
    layer = MixerLayer(SMALL, case.params)
    layer.prepare()
    for _ in range(2):
        with pytest.raises(H.HymbaError) as e:
            layer.check()
        assert e.value.status == H.HYMBA_ERR_RANGE and "weight" in str(e.value)
    layer.close()
    ok = MixerLayer(SMALL, make_prefill_case(SMALL, 1, 20, seed=103).params)
    ok.prepare()
    ok.check()
    ok.close()


def test_negative_decode_position_is_reported():
    announce("negative decode position: hymba_layer_check reports it")
    s = SMALL.with_(window=16)
    case = make_decode_case(s, s.with_(own_kv=False), 3, 20, seed=99, cache_len=16)
    prod = MixerLayer(s, case.producer)
    kc, vc = dev(case.k_cache, "f16"), dev(case.v_cache, "f16")
    st = torch.from_numpy(case.state_p).cuda()
    pos = torch.tensor([20, -1, 5], dtype=torch.int64, device="cuda")
    prod.decode(dev(case.x, "bf16"), pos, make_kv(k_cache=kc, v_cache=vc), st)
    with pytest.raises(H.HymbaError) as e:
        prod.check()
    assert e.value.status == H.HYMBA_ERR_RANGE
    pos = torch.tensor([20, 21, 5], dtype=torch.int64, device="cuda")
    prod.decode(dev(case.x, "bf16"), pos, make_kv(k_cache=kc, v_cache=vc), st)
    prod.check()


def test_serial_schedule_equals_overlapped():
    announce("prefill: serial schedule == overlapped schedule, bitwise")
    case = make_prefill_case(SMALL, 3, 200, seed=101)
    layer = MixerLayer(SMALL, case.params)
    x = dev(case.x, "bf16")
    st1 = torch.empty((3, SMALL.d_inner, SMALL.d_state), dtype=torch.float32, device="cuda")
    st2 = torch.empty_like(st1)
    y1 = host(layer.prefill(x, None, st1))
    layer.set_overlap(False)
    y2 = host(layer.prefill(x, None, st2))
    layer.set_overlap(True)
    torch.cuda.synchronize()
    assert np.array_equal(y1, y2)
    assert np.array_equal(host(st1), host(st2))
