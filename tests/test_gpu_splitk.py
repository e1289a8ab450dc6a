"""GPU parity of the split-K path of the small-M kernel (needs an MI355X).

With few 512-column stripes (N below 65536) and M <= 64, gemm_bf16 splits K
into chunks whose fp32 partial sums a second kernel adds in a fixed order
before the bias, the epilogue and the single rounding; the shapes below all
take that path (N = 1000 .. 4104: 2 .. 9 stripes).  Checked against the
fp64 oracle at the bf16 path's tolerances, and bit for bit run to run.
"""

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


def _check(M, N, K, seed, epi=tg.EPI_NONE, out=torch.bfloat16):
    dev = _dev()
    a = wl.bf16((M, K), "normal", 1.0, seed, 1, dev)
    b = wl.bf16((K, N), "normal", 0.05, seed, 2, dev)
    bias = wl.bf16((N,), "normal", 0.5, seed, 3, dev) if epi != tg.EPI_NONE else None
    c = torch.full((M, N), float("nan"), dtype=out, device=dev)
    print(f"[gpu] splitk M={M} N={N} K={K} epi={epi} out={out}", flush=True)
    tg.gemm_bf16(a, b, bias, c, epilogue=epi)
    torch.cuda.synchronize()
    y, d = og.gemm_bf16_bits(wl.bits_u16(a), wl.bits_u16(b), None if bias is None else wl.bits_u16(bias), epi)
    r = og.compare(c.float().cpu().double().numpy(), y, d, TOL_F32 if out == torch.float32 else TOL_BF16)
    assert r["ok"], r
    return a, b, bias, c


@pytest.mark.parametrize("shape", [(1, 4096, 4096), (8, 4096, 14336), (16, 2048, 1000), (33, 4096, 4096),
                                   (64, 4104, 4096), (1, 1000, 8192), (5, 3000, 2056)])
def test_splitk_shapes(shape):
    M, N, K = shape
    _check(M, N, K, 111 + M)


@pytest.mark.parametrize("epi", [tg.EPI_BIAS, tg.EPI_BIAS_GELU_TANH])
@pytest.mark.parametrize("out", [torch.bfloat16, torch.float32])
def test_splitk_epilogues(epi, out):
    _check(12, 4096, 4096, 112, epi, out)


def test_splitk_deterministic():
    a, b, bias, c1 = _check(4, 4096, 4096, 113, tg.EPI_BIAS, torch.float32)
    c2 = torch.empty_like(c1)
    tg.gemm_bf16(a, b, bias, c2, epilogue=tg.EPI_BIAS)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int32), c2.view(torch.int32))


def test_splitk_on_two_streams():
    """Concurrent calls on two streams keep separate partial buffers."""
    dev = _dev()
    M, N, K = 8, 4096, 4096
    a1, a2 = wl.bf16((M, K), "normal", 1.0, 114, 1, dev), wl.bf16((M, K), "normal", 1.0, 115, 1, dev)
    b = wl.bf16((K, N), "normal", 0.05, 114, 2, dev)
    c1, c2 = torch.empty(M, N, dtype=torch.float32, device=dev), torch.empty(M, N, dtype=torch.float32, device=dev)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(5):
        tg.gemm_bf16(a1, b, None, c1, stream=s1)
        tg.gemm_bf16(a2, b, None, c2, stream=s2)
    torch.cuda.synchronize()
    for a, c in ((a1, c1), (a2, c2)):
        y, d = og.gemm_bf16_bits(wl.bits_u16(a), wl.bits_u16(b))
        r = og.compare(c.cpu().double().numpy(), y, d, TOL_F32)
        assert r["ok"], r
