"""The weight-only integer heads on special inputs (needs an MI355X).

The activations stay bf16 (GEMM compute-cost page, section 7.2, plan A) and
every code becomes a bf16 exactly, so the MFMA sees the same values as the
fp64 oracle.  Pinned here for int8 and int4 codes, at 8 rows (registers)
and 64 rows (straight into LDS, int8 with the zero start of each group):

* subnormal activations (exponent field 0) are used exactly: scaled by the
  weights they give normal fp32 outputs, equal to the oracle's at the fp32
  tolerance (a flush to zero would give zeros);
* a NaN in X[i, k] makes row i of C NaN, a NaN scale S[g, j] or bias
  entry its column (through the bias + tanh-GeLU epilogue); everything
  else stays finite and matches the oracle.
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


def _weights(bits, K, N, seed, dev):
    return wl.w8_weights(K, N, seed, dev) if bits == 8 else wl.w4_weights(K, N, seed, dev)


def _run(bits, x, q, s, bias=None, epi=tg.EPI_NONE):
    c = torch.empty(x.shape[0], s.shape[1], dtype=torch.float32, device=x.device)
    (tg.gemm_bf16_w8 if bits == 8 else tg.gemm_bf16_w4)(x, q, s, bias, c, epilogue=epi)
    torch.cuda.synchronize()
    return c.cpu().double().numpy()


def _oracle(bits, x, q, s, bias=None, epi=tg.EPI_NONE):
    f = og.gemm_bf16_w8_bits if bits == 8 else og.gemm_bf16_w4_bits
    bb = None if bias is None else wl.bits_u16(bias)
    return f(wl.bits_u16(x), q.cpu().numpy(), s.cpu().numpy(), bb, epi)


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("M", [8, 64])
def test_subnormal_activations_are_exact(bits, M):
    dev = _dev()
    N, K = 1040, 512
    g = torch.Generator().manual_seed(21)
    mant = torch.randint(1, 128, (M, K), generator=g, dtype=torch.int32)
    sign = torch.randint(0, 2, (M, K), generator=g, dtype=torch.int32) << 15
    x = (mant | sign).to(torch.int16).view(torch.bfloat16).to(dev)
    q, s = _weights(bits, K, N, 22, dev)
    s = s * 1e6  # outputs well inside fp32's normal range
    print(f"[gpu] w{bits} subnormal X M={M} N={N} K={K}", flush=True)
    got = _run(bits, x, q, s)
    y, d = _oracle(bits, x, q, s)
    assert np.count_nonzero(got) == np.count_nonzero(y)
    r = og.compare(got, y, d, TOL_F32)
    assert r["ok"], r


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("M", [8, 64])
def test_nan_reaches_its_row_and_column(bits, M):
    dev = _dev()
    N, K = 1040, 512
    x = wl.bf16((M, K), "normal", 1.0, 23, 1, dev)
    q, s = _weights(bits, K, N, 24, dev)
    bias = wl.bf16((N,), "normal", 0.5, 23, 2, dev)
    i_nan, j_nan, j_bias = M // 2, 517, N - 3
    x[i_nan, 300] = float("nan")
    s[2, j_nan] = float("nan")
    bias[j_bias] = float("nan")
    epi = tg.EPI_BIAS_GELU_TANH
    print(f"[gpu] w{bits} NaN M={M} N={N} K={K}", flush=True)
    got = _run(bits, x, q, s, bias, epi)
    mask = np.zeros((M, N), dtype=bool)
    mask[i_nan, :] = True
    mask[:, j_nan] = True
    mask[:, j_bias] = True
    assert np.isnan(got[mask]).all()
    assert np.isfinite(got[~mask]).all()
    y, d = _oracle(bits, x, q, s, bias, epi)
    r = og.compare(got[~mask], y[~mask], d[~mask], TOL_F32)
    assert r["ok"], r
