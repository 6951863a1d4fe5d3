"""The allocation-free decode step (hymba_mixer_decode_static) against hymba_mixer_decode.

Two calls in a row through the C ABI on the 1.5B-shaped KV-sharing pair at position 8192 (ring
cache of 1024 slots, 128 meta keys): all 128 sequences, then a smaller call of 40 sequences, which
reuses the same device scratch.  Each is checked against the workspace entry point on identical
copies of the inputs (outputs, updated SSM states and the written cache slot) to the bf16 bar, and
on sampled sequences against the fp64 oracle."""
import numpy as np
import pytest
import torch

import hybrid_attention_ssm_swa_amd as H
from hymba_synth import DECODE_B128
from hymba_synth.generate import make_config_case
from oracle import hymba_oracle as orc

from gpu_util import MixerLayer, act, announce, check, check_stored, dev, host, make_kv

pytestmark = pytest.mark.gpu


def _pair(case):
    s, sc = case.shape, case.consumer_shape
    prod = MixerLayer(s, case.producer)
    cons = MixerLayer(sc, case.consumer)
    cons.bind(prod)
    prod.prepare()
    cons.prepare()
    return prod, cons


def _inputs(case, B):
    s = case.shape
    kc, vc = dev(case.k_cache[:B], act(s.dtype)), dev(case.v_cache[:B], act(s.dtype))
    return dict(x=dev(case.x[:B], s.dtype), xc=dev(case.x_c[:B], s.dtype), pos=torch.from_numpy(case.pos[:B]).cuda(),
                stp=torch.from_numpy(case.state_p[:B].copy()).cuda(), stc=torch.from_numpy(case.state_c[:B].copy()).cuda(),
                kc=kc, vc=vc, kv=make_kv(k_cache=kc, v_cache=vc))


def _static_decode(layer, x, pos, kv, state):
    y = torch.empty_like(x)
    H.hymba_mixer_decode_static(layer.handle, x.data_ptr(), pos.data_ptr(), x.shape[0], y.data_ptr(), kv,
                                state.data_ptr(), torch.cuda.current_stream().cuda_stream)
    return y


def test_static_decode_matches_the_workspace_entry():
    case = make_config_case(DECODE_B128)
    prod, cons = _pair(case)
    kmp, vmp = orc.meta_kv(case.producer)
    for B in (128, 40):
        announce(f"allocation-free decode pair, B={B}")
        ref_in, st_in = _inputs(case, B), _inputs(case, B)
        yp_ref = prod.decode(ref_in["x"], ref_in["pos"], ref_in["kv"], ref_in["stp"])
        yc_ref = cons.decode(ref_in["xc"], ref_in["pos"], ref_in["kv"], ref_in["stc"])
        yp = _static_decode(prod, st_in["x"], st_in["pos"], st_in["kv"], st_in["stp"])
        yc = _static_decode(cons, st_in["xc"], st_in["pos"], st_in["kv"], st_in["stc"])
        torch.cuda.synchronize()
        prod.check()
        cons.check()
        check_stored("producer y vs workspace entry", host(yp), host(yp_ref), "bf16")
        check_stored("consumer y vs workspace entry", host(yc), host(yc_ref), "bf16")
        check("producer state vs workspace entry", host(st_in["stp"]), host(ref_in["stp"]), "bf16")
        check("consumer state vs workspace entry", host(st_in["stc"]), host(ref_in["stc"]), "bf16")
        slot = 8192 % case.k_cache.shape[2]
        check_stored("written K slot vs workspace entry", host(st_in["kc"][:, :, slot]), host(ref_in["kc"][:, :, slot]),
                     "f16")
        for b in (0, B - 1):
            p = int(case.pos[b])
            dp = orc.decode_step(case.producer, case.x[b], p, case.k_cache[b], case.v_cache[b], case.state_p[b],
                                 kmp, vmp)
            dc = orc.decode_step(case.consumer, case.x_c[b], p, dp.k_cache, dp.v_cache, case.state_c[b], kmp, vmp)
            check_stored(f"producer y[b={b}] vs oracle", host(yp[b]), dp.Y, "bf16")
            check_stored(f"consumer y[b={b}] vs oracle", host(yc[b]), dc.Y, "bf16")


def test_static_decode_rejects_what_does_not_fit():
    case = make_config_case(DECODE_B128)
    s = case.shape
    prod = MixerLayer(s, case.producer)
    x = torch.zeros((600, s.d_model), dtype=torch.bfloat16, device="cuda")
    pos = torch.full((600,), 8192, dtype=torch.int64, device="cuda")
    kc = torch.zeros((600, s.n_kv_heads, 1024, s.head_dim), dtype=torch.float16, device="cuda")
    st = torch.zeros((600, s.d_inner, s.d_state), dtype=torch.float32, device="cuda")
    kv = make_kv(k_cache=kc, v_cache=kc)
    with pytest.raises(H.HymbaError) as e:          # not prepared yet
        _static_decode(prod, x[:4], pos[:4], kv, st[:4])
    assert e.value.status == H.HYMBA_ERR_INVALID_ARG
    prod.prepare()
    with pytest.raises(H.HymbaError) as e:          # 600 sequences need more than the 32 MiB scratch
        _static_decode(prod, x, pos, kv, st)
    assert e.value.status == H.HYMBA_ERR_WORKSPACE
