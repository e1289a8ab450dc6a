"""GPU parity of the strided-batched bf16 GEMM (gemm_bf16_strided_batched)
(needs an MI355X).

Every problem of a batch runs the same kernel code as a single gemm_bf16 /
gemm_bf16_nt call on its own operands, so each must equal that call bit for
bit; a few problems are also checked against the fp64 oracle (bf16 output
8e-3, fp32 output 1e-5).
"""

import numpy as np
import pytest
import torch

import tiled_gemm_04_amd as tg
import workloads as wl
from oracle import gemm as og

pytestmark = pytest.mark.gpu

TOL_F32, TOL_BF16 = 1e-5, 8e-3


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


def _single(a, b, bias, c, layout, epi):
    if layout == tg.B_KN:
        tg.gemm_bf16(a, b, bias, c, epilogue=epi)
    else:
        tg.gemm_bf16_nt(a, b, bias, c, epilogue=epi)


def _run(batch, M, N, K, layout, seed, out=torch.bfloat16, epi=tg.EPI_NONE, share_b=False):
    dev = _dev()
    a = wl.bf16((batch, M, K), "normal", 1.0, seed, 1, dev)
    bshape = (K, N) if layout == tg.B_KN else (N, K)
    if share_b:
        b = wl.bf16(bshape, "normal", 1.0, seed, 2, dev).unsqueeze(0).expand(batch, *bshape)
    else:
        b = wl.bf16((batch,) + bshape, "normal", 1.0, seed, 2, dev)
    bias = wl.bf16((N,), "normal", 1.0, seed, 3, dev) if epi != tg.EPI_NONE else None
    c = torch.full((batch, M, N), float("nan"), dtype=out, device=dev)
    print(f"[gpu] batched batch={batch} M={M} N={N} K={K} layout={layout} share_b={share_b} out={out}",
          flush=True)
    tg.gemm_bf16_strided_batched(a, b, bias, c, b_layout=layout, epilogue=epi)
    ref = torch.empty(M, N, dtype=out, device=dev)
    for z in range(batch):
        _single(a[z], b[z].contiguous() if share_b else b[z], bias, ref, layout, epi)
        torch.cuda.synchronize()
        assert torch.equal(c[z].view(torch.uint8), ref.view(torch.uint8)), f"problem {z}"
    for z in (0, batch - 1):
        bz = b[z].contiguous()
        bits = wl.bits_u16(bz)
        if layout == tg.B_NK:
            y, d = og.gemm_bf16_nt_bits(wl.bits_u16(a[z]), bits, None if bias is None else wl.bits_u16(bias), epi)
        else:
            y, d = og.gemm_bf16_bits(wl.bits_u16(a[z]), bits, None if bias is None else wl.bits_u16(bias), epi)
        r = og.compare(c[z].float().cpu().double().numpy(), y, d, TOL_F32 if out == torch.float32 else TOL_BF16)
        assert r["ok"], f"problem {z}: {r}"


@pytest.mark.parametrize("shape", [(5, 1, 512, 256), (3, 17, 1000, 136), (4, 64, 768, 384),
                                   (3, 300, 520, 200), (2, 600, 1024, 512)])
@pytest.mark.parametrize("layout", [0, 1])
def test_batched_equals_single_calls(shape, layout):
    batch, M, N, K = shape
    _run(batch, M, N, K, layout, 101 + M)


@pytest.mark.parametrize("layout", [0, 1])
def test_batched_shared_weight_stride_zero(layout):
    _run(6, 40, 640, 256, layout, 102, share_b=True)


def test_batched_bias_gelu_fp32_output():
    _run(3, 130, 264, 128, tg.B_KN, 103, out=torch.float32, epi=tg.EPI_BIAS_GELU_TANH)


def test_batched_unaligned_strides_use_general_kernels():
    """Batch strides that are not multiples of 8 elements: problem bases lose
    16-byte alignment, so the register-staged kernels run; still equal to the
    single calls on copies and to the oracle."""
    dev = _dev()
    batch, M, N, K = 3, 70, 200, 96
    abuf = wl.bf16((batch * (M * K + 3),), "normal", 1.0, 104, 1, dev)
    a = torch.as_strided(abuf, (batch, M, K), (M * K + 3, K, 1))
    b = wl.bf16((batch, K, N), "normal", 1.0, 104, 2, dev)
    c = torch.empty(batch, M, N, dtype=torch.bfloat16, device=dev)
    tg.gemm_bf16_strided_batched(a, b, None, c)
    torch.cuda.synchronize()
    for z in range(batch):
        y, d = og.gemm_bf16_bits(wl.bits_u16(a[z].contiguous()), wl.bits_u16(b[z]))
        r = og.compare(c[z].float().cpu().double().numpy(), y, d, TOL_BF16)
        assert r["ok"], f"problem {z}: {r}"


def test_batched_rejects_overlapping_outputs():
    dev = _dev()
    a = wl.bf16((2, 8, 64), "normal", 1.0, 105, 1, dev)
    b = wl.bf16((2, 64, 64), "normal", 1.0, 105, 2, dev)
    c = torch.empty(8, 64, dtype=torch.bfloat16, device=dev).unsqueeze(0).expand(2, 8, 64)
    with pytest.raises(tg.TgemmError):
        tg.gemm_bf16_strided_batched(a, b, None, c)
