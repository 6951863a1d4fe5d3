"""Parity of the many-row projection kernel (hymba_kernel_gemm_tiles, the tiled matrix-core GEMM
that bf16 layers use for prefill) with an fp64 matmul of the same 16-bit operands.

Bound per element: the output type's own rounding u*|ref| plus the worst-case fp32
accumulation error K * 2^-24 * (|x| |w|^T) (products of 16-bit values are exact in fp32).
Shapes: the 8K prefill projections of the 1.5B KV-consumer layer at full size (sampled rows,
every column), the 300M layer's input projection, and ragged ones: rows and columns not
multiples of the 256 x 256 tile, K not a multiple of the 64-wide step, tile counts that are
and are not multiples of 8 (the XCD deal), padded strides, the fp32 copy of a column range,
a single row and an empty call; two calls on the same operands are bitwise equal.
"""
import numpy as np
import pytest
import torch

from hybrid_attention_ssm_swa_amd import _lib as L

from gpu_util import announce, check_bound, host

pytestmark = pytest.mark.gpu

TD = {L.HYMBA_F16: torch.float16, L.HYMBA_BF16: torch.bfloat16}
U = {L.HYMBA_F16: 2.0 ** -11, L.HYMBA_BF16: 2.0 ** -8}


def _mat(gen, rows, cols, ld, dt):
    a = torch.zeros(rows, ld, dtype=dt, device="cuda")
    a[:, :cols] = torch.randn(rows, cols, generator=gen, device="cuda", dtype=torch.float32).to(dt)
    return a


def _run(it, yt, M, N, K, pad, cols, seed, sample=None):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    ldw, ldx, ldy = K + pad, K + pad, N + (4 if pad else 0)
    w = _mat(gen, N, K, ldw, TD[it])
    x = _mat(gen, M, K, ldx, TD[it])
    y = torch.full((M, ldy), float("nan"), dtype=TD[yt], device="cuda")
    y32 = None
    c0 = c1 = 0
    if cols:
        c0, c1 = cols
        y32 = torch.full((M, c1 - c0 + 4), float("nan"), dtype=torch.float32, device="cuda")
    L.hymba_kernel_gemm_tiles(it, yt, w.data_ptr(), ldw, x.data_ptr(), ldx, y.data_ptr(), ldy,
                              None if y32 is None else y32.data_ptr(), 0 if y32 is None else y32.shape[1],
                              c0, c1, M, N, K, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    rows = np.arange(M) if sample is None else sample
    wh = host(w)[:, :K]
    xh = host(x[torch.from_numpy(rows).cuda()])[:, :K]
    ref = xh @ wh.T
    acc = K * 2.0 ** -24 * (np.abs(xh) @ np.abs(wh).T)
    got = host(y[torch.from_numpy(rows).cuda()])
    check_bound("y", got[:, :N], ref, U[yt] * np.abs(ref) + acc)
    if pad:
        assert np.all(np.isnan(got[:, N:])), "wrote past N"
    if y32 is not None:
        g32 = host(y32[torch.from_numpy(rows).cuda()])
        check_bound("y32", g32[:, :c1 - c0], ref[:, c0:c1], acc[:, c0:c1] + 1e-30)
        assert np.all(np.isnan(g32[:, c1 - c0:])), "y32 written past c1 - c0"


@pytest.mark.parametrize("it,yt,M,N,K,pad,cols", [
    (L.HYMBA_BF16, L.HYMBA_F16, 300, 520, 200, 8, (32, 96)),      # ragged M, N; K tail of 8
    (L.HYMBA_BF16, L.HYMBA_F16, 4099, 11232, 1600, 0, (11200, 11232)),   # in_proj columns, ragged rows
    (L.HYMBA_F16, L.HYMBA_F16, 1000, 3200, 1600, 0, None),        # W_O
    (L.HYMBA_BF16, L.HYMBA_BF16, 257, 1600, 3200, 0, None),       # out_proj, 2 row tiles
    (L.HYMBA_F16, L.HYMBA_BF16, 512, 1024, 64, 16, None),         # 8 tiles: the XCD deal; one K step
    (L.HYMBA_BF16, L.HYMBA_F16, 1, 4, 8, 0, (0, 4)),              # one row, one K chunk
    (L.HYMBA_BF16, L.HYMBA_F16, 16384, 7712, 1024, 0, (7680, 7712)),   # 300M in_proj (own KV)
])
def test_gemm_tiles_matches_fp64(it, yt, M, N, K, pad, cols):
    announce(f"gemm_tiles in={it} out={yt} M={M} N={N} K={K} pad={pad} cols={cols}")
    sample = None
    if M > 5000:
        sample = np.unique(np.concatenate([np.arange(0, M, M // 61), [M - 1, 255, 256]]))
    _run(it, yt, M, N, K, pad, cols, seed=M * 7 + N + K, sample=sample)


def test_gemm_tiles_8k_in_proj_full_size():
    """The 8K prefill input projection of the 1.5B KV consumer: 16 x 8192 rows, 11232 columns
    (P's row stride padded to 11264), B/C columns in fp32; sampled rows, every column."""
    M, N, K, ldy = 16 * 8192, 11232, 1600, 11264
    announce(f"gemm_tiles full-size 8K in_proj M={M} N={N} K={K}")
    gen = torch.Generator(device="cuda").manual_seed(2024)
    w = torch.randn(N, K, generator=gen, device="cuda").to(torch.bfloat16) * (1.0 / 40)
    x = torch.randn(M, K, generator=gen, device="cuda").to(torch.bfloat16)
    y = torch.empty(M, ldy, dtype=torch.float16, device="cuda")
    y32 = torch.empty(M, 32, dtype=torch.float32, device="cuda")
    L.hymba_kernel_gemm_tiles(L.HYMBA_BF16, L.HYMBA_F16, w.data_ptr(), K, x.data_ptr(), K, y.data_ptr(), ldy,
                              y32.data_ptr(), 32, 11200, 11232, M, N, K, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, M, 2039), [M - 1, M - 256, 8191, 8192]]))
    ri = torch.from_numpy(rows).cuda()
    wh, xh = host(w).astype(np.float64), host(x[ri]).astype(np.float64)
    ref = xh @ wh.T
    acc = K * 2.0 ** -24 * (np.abs(xh) @ np.abs(wh).T)
    check_bound("P", host(y[ri])[:, :N], ref, U[L.HYMBA_F16] * np.abs(ref) + acc)
    check_bound("BC", host(y32[ri]), ref[:, 11200:], acc[:, 11200:] + 1e-30)
    del x, y, y32


def test_gemm_tiles_empty_and_bad_args():
    announce("gemm_tiles: M = 0 and invalid arguments")
    w = torch.zeros(8, 16, dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(4, 8, dtype=torch.float16, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    L.hymba_kernel_gemm_tiles(L.HYMBA_BF16, L.HYMBA_F16, w.data_ptr(), 16, w.data_ptr(), 16, y.data_ptr(), 8,
                              None, 0, 0, 0, 0, 8, 16, s)
    with pytest.raises(L.HymbaError):
        L.hymba_kernel_gemm_tiles(L.HYMBA_BF16, L.HYMBA_F16, w.data_ptr(), 12, w.data_ptr(), 16, y.data_ptr(), 8,
                                  None, 0, 0, 0, 4, 8, 16, s)
    with pytest.raises(L.HymbaError):
        L.hymba_kernel_gemm_tiles(L.HYMBA_F32, L.HYMBA_F16, w.data_ptr(), 16, w.data_ptr(), 16, y.data_ptr(), 8,
                                  None, 0, 0, 0, 4, 8, 16, s)
    torch.cuda.synchronize()


def test_gemm_tiles_deterministic():
    """Two calls on the same operands give bitwise-equal results (each output's K sum is taken
    in one fixed order; no split-K, no atomics)."""
    announce("gemm_tiles: two calls, bitwise-equal outputs")
    M, N, K = 3000, 11232, 1600
    gen = torch.Generator(device="cuda").manual_seed(5)
    w = torch.randn(N, K, generator=gen, device="cuda").to(torch.bfloat16)
    x = torch.randn(M, K, generator=gen, device="cuda").to(torch.bfloat16)
    outs = []
    for _ in range(2):
        y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
        y32 = torch.full((M, 32), float("nan"), dtype=torch.float32, device="cuda")
        L.hymba_kernel_gemm_tiles(L.HYMBA_BF16, L.HYMBA_F16, w.data_ptr(), K, x.data_ptr(), K, y.data_ptr(), N,
                                  y32.data_ptr(), 32, N - 32, N, M, N, K, torch.cuda.current_stream().cuda_stream)
        outs.append((y, y32))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.isfinite(outs[0][0]).all()
