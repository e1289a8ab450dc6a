"""The bf16 GEMMs on special inputs (needs an MI355X).

The GEMM compute-cost page takes bf16 as the operand format and fp32 as the
accumulator (section 4.2); nothing in the pages allows flushing or dropping
values, so the fp64 oracle uses every bf16 value as it is.  Pinned here:

* subnormal operands (exponent field 0) are used exactly: a subnormal A
  times normal B values around 2^12 gives normal fp32 products, and the
  result must match the oracle at the fp32 tolerance (a flush to zero would
  give zeros);
* a NaN in A[i, k] makes row i of C NaN, a NaN in B[k, j] column j, a NaN
  bias entry its column (through the bias + tanh-GeLU epilogue); everything
  else stays finite and matches the oracle.

Each on the tiled kernel, the small-M kernel and the [N, K] weight.
"""

import numpy as np
import pytest
import torch

import tiled_gemm_04_amd as tg
import workloads as wl
from oracle import gemm as og

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


def _subnormals(shape, seed, dev):
    g = torch.Generator().manual_seed(seed)
    mant = torch.randint(1, 128, shape, generator=g, dtype=torch.int32)
    sign = torch.randint(0, 2, shape, generator=g, dtype=torch.int32) << 15
    return (mant | sign).to(torch.int16).view(torch.bfloat16).to(dev)


def _gemm(a, b, bias, epi, layout, algo=tg.ALGO_AUTO):
    M, N = a.shape[0], b.shape[1]
    c = torch.empty(M, N, dtype=torch.float32, device=a.device)
    if layout == "nt":
        tg.gemm_bf16_nt(a, b.t().contiguous(), bias, c, epilogue=epi)
    else:
        tg.gemm_bf16_ex(a, b, bias, c, epilogue=epi, algo=algo)
    torch.cuda.synchronize()
    return c.cpu().double().numpy()


CASES = [(300, 520, 256, "kn", tg.ALGO_AUTO), (300, 520, 256, "kn", tg.ALGO_TILED_128x128),
         (8, 520, 256, "kn", tg.ALGO_AUTO), (300, 520, 256, "nt", None), (8, 520, 256, "nt", None)]


@pytest.mark.parametrize("M,N,K,layout,algo", CASES)
@pytest.mark.parametrize("which", ["a", "b"])
def test_subnormal_operands_are_exact(M, N, K, layout, algo, which):
    dev = _dev()
    g = torch.Generator().manual_seed(7)
    if which == "a":
        a = _subnormals((M, K), 11, dev)
        b = (torch.randn(K, N, generator=g) * 4096.0).to(torch.bfloat16).to(dev)
    else:
        a = (torch.randn(M, K, generator=g) * 4096.0).to(torch.bfloat16).to(dev)
        b = _subnormals((K, N), 12, dev)
    print(f"[gpu] bf16 subnormal {which} {layout} M={M} N={N} K={K}", flush=True)
    got = _gemm(a, b, None, tg.EPI_NONE, layout, algo)
    y, d = og.gemm_bf16_bits(wl.bits_u16(a), wl.bits_u16(b))
    assert np.count_nonzero(got) == np.count_nonzero(y)
    r = og.compare(got, y, d, TOL_F32)
    assert r["ok"], r


@pytest.mark.parametrize("M,N,K,layout,algo", CASES)
def test_nan_reaches_its_row_and_column(M, N, K, layout, algo):
    dev = _dev()
    a = wl.bf16((M, K), "normal", 1.0, 13, 1, dev)
    b = wl.bf16((K, N), "normal", 0.05, 13, 2, dev)
    bias = wl.bf16((N,), "normal", 0.5, 13, 3, dev)
    i_nan, j_nan, j_bias = M // 2, 100, N - 3
    a[i_nan, 7] = float("nan")
    b[9, j_nan] = float("nan")
    bias[j_bias] = float("nan")
    print(f"[gpu] bf16 NaN {layout} M={M} N={N} K={K}", flush=True)
    got = _gemm(a, b, bias, tg.EPI_BIAS_GELU_TANH, layout, algo)
    mask = np.zeros((M, N), dtype=bool)
    mask[i_nan, :] = True
    mask[:, j_nan] = True
    mask[:, j_bias] = True
    assert np.isnan(got[mask]).all()
    assert np.isfinite(got[~mask]).all()
    y, d = og.gemm_bf16_bits(wl.bits_u16(a), wl.bits_u16(b), wl.bits_u16(bias), tg.EPI_BIAS_GELU_TANH)
    r = og.compare(got[~mask], y[~mask], d[~mask], TOL_F32)
    assert r["ok"], r
