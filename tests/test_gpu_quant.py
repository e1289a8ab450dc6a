"""GPU parity of the FP8 quantisers against the oracle's quantiser (needs an
MI355X).

The quantiser decides integers (codes) from floating-point values, so the
GPU and the oracle take every decision in the same precision (fp32 amax,
fp32 amax / 448, fp32 x / scale, round to nearest even) and the comparison is
bit-exact: every code byte and every scale.  Inputs are the bf16 values the
GPU reads, widened exactly to fp32 for the oracle.  The DeepGEMM page
(section 2.4) gives the scheme: one scale per (row, 128-column group) of the
activations, one per 128 x 128 block of the weights.
"""

import numpy as np
import pytest
import torch

import tiled_gemm_04_amd as tg
import workloads as wl
from oracle import gemm as og
from oracle import quant as oq

pytestmark = pytest.mark.gpu

CANARY = 0xA5


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


def _f32(x_bf16):
    return x_bf16.detach().float().cpu().numpy()


def _run(kind, x, q_view=None):
    """Quantise bf16 x on the GPU; returns (codes uint8 numpy, scales numpy)."""
    R, C = x.shape
    G = (R + 127) // 128 if kind == "blocks" else R
    H = (C + 127) // 128
    if q_view is None:
        qbuf = torch.full((R * C + 16,), CANARY, dtype=torch.uint8, device=x.device)
        q = qbuf[8:8 + R * C].view(R, C)
    else:
        qbuf, q = q_view
    s = torch.full((G, H), float("nan"), dtype=torch.float32, device=x.device)
    print(f"[gpu] quantize {kind} {R}x{C}", flush=True)
    if kind == "rows":
        tg.quantize_fp8_1x128(x, q, s)
    else:
        tg.quantize_fp8_128x128(x, q, s)
    torch.cuda.synchronize()
    return qbuf, q.cpu().numpy().copy(), s.cpu().numpy()


def _check(kind, x):
    qbuf, q, s = _run(kind, x)
    R, C = x.shape
    guard = qbuf.cpu().numpy()
    assert (guard[:8] == CANARY).all() and (guard[8 + R * C:] == CANARY).all()
    ref = oq.quantise_rows_1x128(_f32(x)) if kind == "rows" else oq.quantise_blocks_128x128(_f32(x))
    np.testing.assert_array_equal(s.view(np.uint32), ref[1].view(np.uint32))
    np.testing.assert_array_equal(q, ref[0])


ROW_SHAPES = [(1, 1), (3, 7), (5, 130), (17, 257), (64, 1000), (2, 513), (300, 4096)]
BLOCK_SHAPES = [(1, 1), (129, 131), (130, 7), (300, 257), (256, 512), (7, 1000)]


@pytest.mark.parametrize("shape", ROW_SHAPES)
def test_rows_1x128_shapes(shape):
    x = wl.bf16(shape, "normal", 1.0, 11, 0, _dev())
    _check("rows", x)


@pytest.mark.parametrize("shape", BLOCK_SHAPES)
def test_blocks_128x128_shapes(shape):
    x = wl.bf16(shape, "normal", 0.02, 12, 0, _dev())
    _check("blocks", x)


@pytest.mark.parametrize("kind", ["rows", "blocks"])
def test_special_values(kind):
    """All-zero groups (scale 1), signed zeros, the exact extremes (codes
    0x7E / 0xFE), and exact ties of the e4m3 rounding, normal and subnormal:
    a group whose amax is 448 has scale 1, so x / scale = x exactly."""
    dev = _dev()
    R, C = 130, 260
    x = torch.zeros(R, C, dtype=torch.float32)
    x[0, :128] = torch.linspace(-3, 3, 128)           # ordinary group
    x[1, 5] = -0.0                                    # all-zero group holding -0
    ties = [448.0, 1.0625, 1.1875, -1.0625, 3.25, 2.0 ** -6 * 1.0625,  # normal ties
            1.5 * 2.0 ** -9, 2.5 * 2.0 ** -9, -0.5 * 2.0 ** -9, 7.5 * 2.0 ** -9,  # subnormal ties
            -448.0, 240.0, 0.5 * 2.0 ** -9]
    x[2, :len(ties)] = torch.tensor(ties)
    x[3, 128:256] = -7.0                              # constant group: every code is -448
    x[4, 0], x[4, 1] = 448.0, 1e-30                   # far below the smallest step: code 0
    x[129, 259] = 1e-30                               # alone in its group: a tiny, normal scale
    xb = x.to(torch.bfloat16)
    assert torch.equal(xb[2].float(), x[2])           # the ties are exact in bf16
    _check(kind, xb.to(dev))


@pytest.mark.parametrize("kind", ["rows", "blocks"])
def test_strided_and_unaligned(kind):
    """X with row stride K + 3 starting one element into its buffer; Q one
    byte into its buffer (the kernels' scalar load / byte store paths)."""
    dev = _dev()
    R, C = 70, 300
    base = wl.bf16((R * (C + 3) + 1,), "normal", 1.0, 13, 0, dev)
    x = base[1:].view(R, C + 3)[:, :C]
    assert x.stride(0) == C + 3
    qbuf = torch.full((R * C + 16,), CANARY, dtype=torch.uint8, device=dev)
    q = qbuf[9:9 + R * C].view(R, C)
    _, qn, s = _run(kind, x, (qbuf, q))
    ref = (oq.quantise_rows_1x128 if kind == "rows" else oq.quantise_blocks_128x128)(_f32(x))
    np.testing.assert_array_equal(s.view(np.uint32), ref[1].view(np.uint32))
    np.testing.assert_array_equal(qn, ref[0])
    g = qbuf.cpu().numpy()
    assert (g[:9] == CANARY).all() and (g[9 + R * C:] == CANARY).all()


@pytest.mark.parametrize("kind", ["rows", "blocks"])
def test_full_size_fp8_operands(kind):
    """The FP8 workload's operands at full size: A [4096, 4096] (N(0,1) with
    outliers) by rows, B [4096, 14336] (N(0, 0.02)) by blocks."""
    a, b = wl.fp8_sources_bf16(wl.WORKLOADS["fp8"], device=_dev())
    _check(kind, a if kind == "rows" else b)


def test_quantised_operands_feed_the_gemm():
    """GPU-quantised A and B through gemm_fp8_blockscaled against the oracle
    GEMM on the dequantised codes (the producer -> consumer path)."""
    dev = _dev()
    M, N, K = 300, 264, 384
    a, b = wl.fp8_sources_bf16(wl.WORKLOADS["fp8"], device=dev, M=M, N=N, K=K)
    qa = torch.empty(M, K, dtype=torch.float8_e4m3fn, device=dev)
    sa = torch.empty(M, 3, dtype=torch.float32, device=dev)
    qb = torch.empty(K, N, dtype=torch.float8_e4m3fn, device=dev)
    sb = torch.empty(3, 3, dtype=torch.float32, device=dev)
    tg.quantize_fp8_1x128(a, qa, sa)
    tg.quantize_fp8_128x128(b, qb, sb)
    c = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    tg.gemm_fp8_blockscaled(qa, sa, qb, sb, c)
    torch.cuda.synchronize()
    y, d = og.gemm_fp8_blockscaled_bits(wl.bits_u8(qa), sa.cpu().numpy(), wl.bits_u8(qb),
                                        sb.cpu().numpy())
    r = og.compare(c.float().cpu().double().numpy(), y, d, 1.5e-2)
    assert r["ok"], r
