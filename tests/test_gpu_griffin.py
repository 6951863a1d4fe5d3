"""Parity of the Griffin recurrent block (griffin_block_prefill / griffin_block_decode) with the
fp64 oracle, through the C ABI.

Small blocks are checked on every sequence with the recurrence cut into several time segments
and a ragged last segment; continuation from a handed state (prefill -> prefill, prefill ->
decode) and in-place state update are checked against the oracle on the whole sequence; the
8K workload (d_model 1536, d_rnn 2048, 16 x 8192 tokens) runs in the launch configuration the
benchmark times and is checked on a sampled sequence.
"""
import numpy as np
import pytest
import torch

from hymba_synth.griffin import GRIFFIN_8K, GRIFFIN_SMALL, GriffinShape, make_griffin_case
from oracle import griffin_oracle as go

from gpu_util import announce, check, check_stored, dev, host

pytestmark = pytest.mark.gpu

MID_BF16 = GriffinShape(d_model=256, d_rnn=384, dtype="bf16")


def _block(case):
    from hybrid_attention_ssm_swa_amd.griffin import GriffinBlock
    return GriffinBlock(case.shape, case.params)


def _oracle(case, b, conv_state=None, h0=None, x=None):
    return go.griffin_block(case.params, case.x[b] if x is None else x, conv_state, h0)


@pytest.mark.parametrize("shape,B,T", [
    (GRIFFIN_SMALL, 2, 300),     # 4 segments of 75 steps (ragged step chunks)
    (GRIFFIN_SMALL, 3, 63),      # one segment
    (GRIFFIN_SMALL, 1, 1),
    (MID_BF16, 2, 1000),         # 15 segments of 67 steps
    (MID_BF16, 1, 130),
    (MID_BF16.with_(d_rnn=136), 2, 517),   # R not a multiple of 64: partial last wave
])
def test_prefill_matches_oracle(shape, B, T):
    announce(f"griffin prefill {shape} B={B} T={T}")
    case = make_griffin_case(shape, B, T, seed=100 + T)
    blk = _block(case)
    conv_out, h_out = blk.new_state(B)
    y = blk.prefill(dev(case.x, shape.dtype), conv_state_out=conv_out, h_out=h_out)
    torch.cuda.synchronize()
    y, conv_out, h_out = host(y), host(conv_out), host(h_out)
    for b in range(B):
        ref = _oracle(case, b)
        check_stored(f"y[b={b}]", y[b], ref.Y, shape.dtype)
        check(f"h_T[b={b}]", h_out[b], ref.h_T, shape.dtype)
        # the conv state is the last three branch inputs u (a GEMM output in the block's type)
        check_stored(f"conv_state[b={b}]", conv_out[b], ref.conv_state, shape.dtype)


@pytest.mark.parametrize("shape", [GRIFFIN_SMALL, MID_BF16])
def test_continuation_and_decode_match_the_whole_sequence(shape):
    """prefill(0:T1) -> prefill(T1:T2) from the handed state, in place -> decode steps."""
    B, T1, T2, n_dec = 2, 200, 333, 5
    T = T1 + T2 + n_dec
    announce(f"griffin continuation {shape}")
    case = make_griffin_case(shape, B, T, seed=7)
    blk = _block(case)
    x = dev(case.x, shape.dtype)
    conv, h = blk.new_state(B)
    conv2, _ = blk.new_state(B)
    y1 = blk.prefill(x[:, :T1].contiguous(), conv_state_out=conv, h_out=h)
    # second part: the conv state goes to a new buffer (aliasing needs seq == 1); h in place
    y2 = blk.prefill(x[:, T1:T1 + T2].contiguous(), conv_state=conv, h=h, conv_state_out=conv2, h_out=h)
    ys = [blk.decode(x[:, T1 + T2 + i].contiguous(), conv2, h) for i in range(n_dec)]
    torch.cuda.synchronize()
    y_all = np.concatenate([host(y1), host(y2), np.stack([host(t) for t in ys], axis=1)], axis=1)
    for b in range(B):
        ref = _oracle(case, b)
        check_stored(f"y[b={b}] (3 calls)", y_all[b], ref.Y, shape.dtype)
        check(f"h after decode [b={b}]", host(h)[b], ref.h_T, shape.dtype)
        check_stored(f"conv state after decode [b={b}]", host(conv2)[b], ref.conv_state, shape.dtype)


def test_state_in_place_prefill_with_segments():
    """h_out aliasing h while the recurrence runs in several segments."""
    shape, B, T = GRIFFIN_SMALL, 2, 400
    case = make_griffin_case(shape, B, T, seed=11)
    rng = np.random.default_rng(5)
    conv0 = rng.standard_normal((B, 3, shape.d_rnn)).astype(np.float32)
    h0 = rng.standard_normal((B, shape.d_rnn)).astype(np.float32)
    blk = _block(case)
    conv = torch.from_numpy(conv0).cuda()
    h = torch.from_numpy(h0).cuda()
    conv_out, _ = blk.new_state(B)
    y = blk.prefill(dev(case.x, "f32"), conv_state=conv, h=h, conv_state_out=conv_out, h_out=h)
    torch.cuda.synchronize()
    for b in range(B):
        ref = _oracle(case, b, conv0[b], h0[b])
        check(f"y[b={b}]", host(y)[b], ref.Y, "f32")
        check(f"h_T[b={b}]", host(h)[b], ref.h_T, "f32")
        check(f"conv_state[b={b}]", host(conv_out)[b], ref.conv_state, "f32")


def test_empty_calls_are_no_ops():
    case = make_griffin_case(GRIFFIN_SMALL, 1, 4, seed=1)
    blk = _block(case)
    x = torch.zeros(0, 4, GRIFFIN_SMALL.d_model, device="cuda")
    y = blk.prefill(x)
    assert y.shape == (0, 4, GRIFFIN_SMALL.d_model)


def test_griffin_8k_sampled():
    """The benchmarked workload: 16 x 8192 tokens, d_model 1536, d_rnn 2048, bf16."""
    shape, B, T = GRIFFIN_8K, 16, 8192
    announce("griffin 8k: generate")
    case = make_griffin_case(shape, B, T, seed=2024)
    blk = _block(case)
    conv_out, h_out = blk.new_state(B)
    announce("griffin 8k: run")
    y = blk.prefill(dev(case.x, shape.dtype), conv_state_out=conv_out, h_out=h_out)
    torch.cuda.synchronize()
    for b in (0, B - 1):
        announce(f"griffin 8k: oracle b={b}")
        ref = _oracle(case, b)
        check_stored(f"y[b={b}]", host(y[b]), ref.Y, shape.dtype)
        check(f"h_T[b={b}]", host(h_out[b]), ref.h_T, shape.dtype)
