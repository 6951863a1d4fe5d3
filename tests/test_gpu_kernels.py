"""Per-kernel parity of the HIP path against the fp64 oracle (through the C ABI).

Shapes span several tiles with ragged tails (T not a multiple of the 32-query
block or the 64-key tile, E not a multiple of the 64-lane wave, meta counts
not a multiple of 64), plus the degenerate cases (W = 1, no meta tokens, T = 1).
"""
import numpy as np
import pytest
import torch

import hybrid_attention_ssm_swa_amd as H
from hymba_synth import bf16_round
from oracle import hymba_oracle as orc

from gpu_util import announce, check, check_stored, dev, host

pytestmark = pytest.mark.gpu


def _round(a, dtype):
    """Values representable in the operand type (bf16-representable values are exact in fp16)."""
    return bf16_round(a) if dtype in ("bf16", "f16") else a.astype(np.float32)


CODE = {"bf16": H.HYMBA_BF16, "f16": H.HYMBA_F16, "f32": H.HYMBA_F32}

ATTN_CASES = [
    # dtype, B, T, M, H, Hkv, hd, W
    ("f16", 2, 300, 40, 10, 2, 64, 100),
    ("f16", 2, 300, 128, 10, 2, 64, 0),
    ("f16", 1, 77, 128, 16, 4, 64, 1),
    ("f16", 3, 1, 128, 25, 5, 64, 1024),
    ("f16", 1, 200, 0, 4, 4, 64, 64),
    ("f16", 2, 130, 16, 8, 1, 64, 40),
    ("f16", 1, 2100, 128, 25, 5, 64, 1024),
    ("f16", 2, 150, 200, 8, 2, 64, 50),
    ("f32", 2, 150, 16, 2, 2, 32, 32),
    ("f32", 1, 70, 5, 6, 3, 64, 0),
]


@pytest.mark.parametrize("dtype,B,T,M,Hq,Hkv,hd,W", ATTN_CASES)
def test_attention_kernel(dtype, B, T, M, Hq, Hkv, hd, W):
    _attention_case(dtype, B, T, M, Hq, Hkv, hd, W)


@pytest.mark.parametrize("dtype,qs", [("f16", 4.0), ("f16", 12.0), ("f16", 24.0), ("f16", 4000.0)])
def test_attention_kernel_peaked_scores(dtype, qs):
    """Queries scaled so scores spread over tens of units: the reference max moves by more than the
    growth threshold across tiles, and most probabilities underflow.  At x4000 raw scores pass
    fp16's range (~1e5), where the fp16 kernel must keep its reference in fp32."""
    _attention_case(dtype, 2, 700, 100, 10, 2, 64, 300, qs)


def test_attention_kernel_rejects_bf16_operands():
    """bf16 layers attend in fp16: bf16 probabilities would round the P.V operand to 8 bits."""
    q = torch.zeros((1, 4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(H.HymbaError) as e:
        H.hymba_kernel_attention(H.HYMBA_BF16, q.data_ptr(), 64, q.data_ptr(), q.data_ptr(), 64, 4 * 64, None, None, 0,
                                 q.data_ptr(), 64, 1, 4, 1, 1, 64, 4, torch.cuda.current_stream().cuda_stream)
    assert e.value.status == H.HYMBA_ERR_UNSUPPORTED


def _attention_case(dtype, B, T, M, Hq, Hkv, hd, W, qs=1.0):
    announce(f"attention {dtype} B={B} T={T} M={M} H={Hq} Hkv={Hkv} hd={hd} W={W} qscale={qs}")
    r = np.random.Generator(np.random.PCG64(100 + T + M + W))
    q = _round(qs * r.standard_normal((B, T, Hq, hd)).astype(np.float32), dtype)
    k = _round(r.standard_normal((B, T, Hkv, hd)).astype(np.float32), dtype)
    v = _round(r.standard_normal((B, T, Hkv, hd)).astype(np.float32), dtype)
    km = _round(r.standard_normal((M, Hkv, hd)).astype(np.float32), dtype)
    vm = _round(r.standard_normal((M, Hkv, hd)).astype(np.float32), dtype)
    dq, dk, dv = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    dkm = dev(km, dtype) if M else None
    dvm = dev(vm, dtype) if M else None
    o = torch.empty((B, T, Hq * hd), dtype=dq.dtype, device="cuda")
    H.hymba_kernel_attention(CODE[dtype], dq.data_ptr(), Hq * hd, dk.data_ptr(), dv.data_ptr(), Hkv * hd, T * Hkv * hd,
                             dkm.data_ptr() if M else None, dvm.data_ptr() if M else None, M, o.data_ptr(),
                             Hq * hd, B, T, Hq, Hkv, hd, W, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = host(o)
    for b in range(B):
        Q = np.concatenate([np.zeros((M, Hq, hd)), q[b]])
        K = np.concatenate([km, k[b]])
        V = np.concatenate([vm, v[b]])
        ref = orc.attention(Q, K, V, M, W)[M:]
        check(f"O[b={b}]", got[b], ref, dtype)


SCAN_CASES = [
    # dtype, B, T, E, N, with_h0
    ("f16", 2, 333, 200, 16, True),
    ("f16", 1, 64, 64, 16, False),
    ("f16", 3, 1, 72, 16, True),
    ("f16", 2, 700, 3200, 16, True),
    ("f32", 2, 257, 136, 8, True),
    ("f32", 1, 100, 64, 16, False),
]


@pytest.mark.parametrize("dtype,B,T,E,N,with_h0", SCAN_CASES)
def test_selective_scan_kernel(dtype, B, T, E, N, with_h0):
    announce(f"scan {dtype} B={B} T={T} E={E} N={N} h0={with_h0}")
    r = np.random.Generator(np.random.PCG64(200 + T + E))
    ld = 2 * E + 8                    # [u | dt | pad] in the activation type
    P = _round(r.standard_normal((B * T, ld)).astype(np.float32), dtype)
    ldbc = 2 * N + 4                  # fp32 [B | C | pad]
    BC = _round(r.standard_normal((B * T, ldbc)).astype(np.float32), dtype)
    A = (-np.exp(r.uniform(0, np.log(8), (E, N)))).astype(np.float32)
    D = r.standard_normal(E).astype(np.float32)
    bias = np.full(E, -2.0, np.float32)
    h0 = r.standard_normal((E, N)).astype(np.float32) if with_h0 else None
    dP = dev(P, dtype)
    t32 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    dBC, dA, dD, db = t32(BC), t32(A), t32(D), t32(bias)
    dh0 = t32(h0) if with_h0 else None
    y = torch.empty((B * T, E), dtype=dP.dtype, device="cuda")
    hT = torch.empty((B, E, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(E * N * 4, dtype=torch.uint8, device="cuda")
    es = dP.element_size()
    base = dP.data_ptr()
    H.hymba_kernel_selective_scan(CODE[dtype], base, base + E * es, ld, dBC.data_ptr(), ldbc, dA.data_ptr(),
                                  dD.data_ptr(), db.data_ptr(), dh0.data_ptr() if with_h0 else None, y.data_ptr(),
                                  E, hT.data_ptr(), B, T, E, N, ws.data_ptr(), ws.numel(),
                                  torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    gy, gh = host(y).reshape(B, T, E), host(hT)
    for b in range(B):
        Pb = P[b * T:(b + 1) * T].astype(np.float64)
        BCb = BC[b * T:(b + 1) * T].astype(np.float64)
        ry, rh = orc.selective_scan(Pb[:, :E], Pb[:, E:2 * E], BCb[:, :N], BCb[:, N:2 * N],
                                    A, D, bias, h0 if with_h0 else np.zeros((E, N)))
        check_stored(f"y[b={b}]", gy[b], ry, dtype)
        check(f"h_T[b={b}]", gh[b], rh, dtype)


@pytest.mark.parametrize("dtype,B,T,E,N,with_h0", [
    ("f16", 2, 1100, 520, 16, True),    # 4 segments of 288 steps, the last ragged
    ("f32", 2, 1100, 520, 8, False),
    ("f16", 1, 4000, 136, 16, True),    # 8 segments
])
def test_selective_scan_time_segments(dtype, B, T, E, N, with_h0):
    """Few long sequences: with the workspace the size query asks for, the scan splits time into
    segments (a summary launch, then every segment from its carried-in state)."""
    announce(f"segmented scan {dtype} B={B} T={T} E={E} N={N} h0={with_h0}")
    r = np.random.Generator(np.random.PCG64(400 + T + E))
    ld = 2 * E + 8
    P = _round(r.standard_normal((B * T, ld)).astype(np.float32), dtype)
    ldbc = 2 * N + 4
    BC = _round(r.standard_normal((B * T, ldbc)).astype(np.float32), dtype)
    A = (-np.exp(r.uniform(0, np.log(8), (E, N)))).astype(np.float32)
    D = r.standard_normal(E).astype(np.float32)
    bias = np.full(E, -2.0, np.float32)
    h0 = r.standard_normal((E, N)).astype(np.float32) if with_h0 else None
    dP = dev(P, dtype)
    t32 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()   # noqa: E731
    dBC, dA, dD, db = t32(BC), t32(A), t32(D), t32(bias)
    dh0 = t32(h0) if with_h0 else None
    nws = H.hymba_kernel_selective_scan_workspace(B, T, E, N)
    assert nws > E * N * 4            # the shape is one that splits
    ws = torch.full((nws,), 255, dtype=torch.uint8, device="cuda")   # NaN bytes: every summary is written
    es = dP.element_size()
    base = dP.data_ptr()
    outs = []
    for nbytes in (nws, E * N * 4):   # segmented, then one pass
        y = torch.empty((B * T, E), dtype=dP.dtype, device="cuda")
        hT = torch.empty((B, E, N), dtype=torch.float32, device="cuda")
        H.hymba_kernel_selective_scan(CODE[dtype], base, base + E * es, ld, dBC.data_ptr(), ldbc, dA.data_ptr(),
                                      dD.data_ptr(), db.data_ptr(), dh0.data_ptr() if with_h0 else None,
                                      y.data_ptr(), E, hT.data_ptr(), B, T, E, N, ws.data_ptr(), nbytes,
                                      torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        outs.append((host(y).reshape(B, T, E), host(hT)))
    for b in range(B):
        Pb = P[b * T:(b + 1) * T].astype(np.float64)
        BCb = BC[b * T:(b + 1) * T].astype(np.float64)
        ry, rh = orc.selective_scan(Pb[:, :E], Pb[:, E:2 * E], BCb[:, :N], BCb[:, N:2 * N],
                                    A, D, bias, h0 if with_h0 else np.zeros((E, N)))
        for tag, (gy, gh) in zip(("segmented", "one pass"), outs):
            check_stored(f"{tag} y[b={b}]", gy[b], ry, dtype)
            check(f"{tag} h_T[b={b}]", gh[b], rh, dtype)


@pytest.mark.parametrize("dtype,rows,E", [("f16", 37, 3200), ("f16", 5, 64), ("f16", 3, 8200), ("f16", 4, 2048),
                                          ("f16", 2, 4104), ("f32", 19, 136), ("f32", 3, 2056),
                                          # thousands of rows (workgroups over the whole grid)
                                          ("f16", 4099, 3200), ("f32", 9003, 136)])
def test_epilogue_kernel(dtype, rows, E):
    announce(f"epilogue {dtype} rows={rows} E={E}")
    r = np.random.Generator(np.random.PCG64(300 + rows + E))
    ao = _round(r.standard_normal((rows, E)).astype(np.float32) * 0.3, dtype)
    y = _round(r.standard_normal((rows, E)).astype(np.float32) * 3.0, dtype)
    zbig = _round(r.standard_normal((rows, E + 24)).astype(np.float32), dtype)
    b1 = r.uniform(0.5, 1.5, E).astype(np.float32)
    b2 = r.uniform(0.5, 1.5, E).astype(np.float32)
    dao, dy, dz = dev(ao, dtype), dev(y, dtype), dev(zbig, dtype)
    # 16-bit inputs (fp16 activations) give a bf16 F, the operand type of the bf16 output projection
    fdt = torch.bfloat16 if dtype == "f16" else torch.float32
    f = torch.empty((rows, E), dtype=fdt, device="cuda")
    t32 = lambda a: torch.from_numpy(a).cuda()
    db1, db2 = t32(b1), t32(b2)
    es = dz.element_size()
    H.hymba_kernel_epilogue(CODE[dtype], dao.data_ptr(), E, dy.data_ptr(), E, dz.data_ptr() + 8 * es, E + 24,
                            db1.data_ptr(), db2.data_ptr(), f.data_ptr(), E, rows, E, 1e-6,
                            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    z = zbig[:, 8:8 + E].astype(np.float64)
    ref = orc.fuse(ao.astype(np.float64), y.astype(np.float64) * orc.silu(z), b1, b2, 1e-6)
    check_stored("F", host(f), ref, "bf16" if dtype == "f16" else dtype)
