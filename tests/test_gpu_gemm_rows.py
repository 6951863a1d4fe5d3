"""Parity of the few-row projection kernel (hymba_kernel_gemm_rows, the weight-streaming GEMM
the layers use for up to 256 rows) with an fp64 matmul of the same 16-bit operands.

Bound per element: the output type's own rounding u*|ref| plus the worst-case fp32
accumulation error K * 2^-24 * (|x| |w|^T) (products of 16-bit values are exact in fp32).
Shapes: the decode projections of the 1.5B layer (128 rows), and ragged ones: rows not a
multiple of 32, features not a multiple of 32 or 64, K not a multiple of 64 or of the 512-k
phase, K walks of 1 to 10 phases (up to 8 unrolled, more in a loop), padded strides, and the
fp32 copy of a column range.
"""
import numpy as np
import pytest
import torch

from hybrid_attention_ssm_swa_amd import _lib as L

from gpu_util import announce, check_bound, host

pytestmark = pytest.mark.gpu

TD = {L.HYMBA_F16: torch.float16, L.HYMBA_BF16: torch.bfloat16}
U = {L.HYMBA_F16: 2.0 ** -11, L.HYMBA_BF16: 2.0 ** -8}


def _mat(rng, rows, cols, ld, dt):
    a = torch.zeros(rows, ld, dtype=dt)
    a[:, :cols] = torch.from_numpy(rng.standard_normal((rows, cols)).astype(np.float32)).to(dt)
    return a.cuda()


@pytest.mark.parametrize("types,M,N,K,pad,cols", [
    ((L.HYMBA_F16, L.HYMBA_BF16, L.HYMBA_F16), 128, 11232, 1600, 0, (11200, 11232)),  # 1.5B decode in_proj
    ((L.HYMBA_F16, L.HYMBA_F16, L.HYMBA_F16), 128, 3200, 1600, 0, None),             # W_O
    ((L.HYMBA_BF16, L.HYMBA_BF16, L.HYMBA_BF16), 128, 1600, 3200, 0, None),          # out_proj
    ((L.HYMBA_F16, L.HYMBA_F16, L.HYMBA_BF16), 128, 1536, 2048, 0, None),            # Griffin out_proj
    ((L.HYMBA_F16, L.HYMBA_F16, L.HYMBA_F16), 77, 196, 200, 8, (32, 96)),
    ((L.HYMBA_F16, L.HYMBA_BF16, L.HYMBA_F16), 200, 100, 72, 16, (0, 100)),
    ((L.HYMBA_BF16, L.HYMBA_BF16, L.HYMBA_BF16), 1, 4, 8, 0, None),
    ((L.HYMBA_F16, L.HYMBA_F16, L.HYMBA_BF16), 256, 260, 136, 8, None),
    ((L.HYMBA_F16, L.HYMBA_F16, L.HYMBA_F16), 40, 68, 4616, 8, None),         # K walk of 10 phases: the loop
    ((L.HYMBA_F16, L.HYMBA_BF16, L.HYMBA_F16), 33, 132, 4096, 0, (64, 132)),  # 8 phases, the longest unrolled
])
def test_gemm_rows_matches_fp64(types, M, N, K, pad, cols):
    wt, xt, yt = types
    announce(f"gemm_rows types={types} M={M} N={N} K={K} pad={pad} cols={cols}")
    rng = np.random.default_rng(M * 7 + N + K)
    ldw, ldx, ldy = K + pad, K + pad, N + (4 if pad else 0)
    w = _mat(rng, N, K, ldw, TD[wt])
    x = _mat(rng, M, K, ldx, TD[xt])
    y = torch.full((M, ldy), float("nan"), dtype=TD[yt], device="cuda")
    y32 = None
    c0 = c1 = 0
    if cols:
        c0, c1 = cols
        y32 = torch.full((M, c1 - c0 + 4), float("nan"), dtype=torch.float32, device="cuda")
    nws = L.hymba_kernel_gemm_rows_workspace(M, N, K)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda")
    L.hymba_kernel_gemm_rows(wt, xt, yt, w.data_ptr(), ldw, x.data_ptr(), ldx, y.data_ptr(), ldy,
                             None if y32 is None else y32.data_ptr(), 0 if y32 is None else y32.shape[1],
                             c0, c1, M, N, K, ws.data_ptr(), nws, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    wh, xh = host(w)[:, :K], host(x)[:, :K]
    ref = xh @ wh.T
    acc = K * 2.0 ** -24 * (np.abs(xh) @ np.abs(wh).T)
    got = host(y)
    check_bound("y", got[:, :N], ref, U[yt] * np.abs(ref) + acc)
    if pad:
        assert np.all(np.isnan(got[:, N:])), "wrote past N"
    if y32 is not None:
        g32 = host(y32)
        check_bound("y32", g32[:, :c1 - c0], ref[:, c0:c1], acc[:, c0:c1] + 1e-30)
        assert np.all(np.isnan(g32[:, c1 - c0:])), "y32 written past c1 - c0"
