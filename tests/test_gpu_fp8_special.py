"""The FP8 block-scaled GEMM on special inputs (needs an MI355X).

* NaN codes.  OCP e4m3fn, the FP8 storage format of the DeepGEMM page's
  low-precision path (section 2.4), has no infinities; S.1111.111 (0x7F,
  0xFF) is NaN, and the C ABI promises that a NaN code reaches every output
  it touches: a NaN in A[i, k] makes row i of C NaN, a NaN in B[k, j]
  column j.  Checked on the automatic path (half tiles), on whole tiles, on
  the [N, K] weight, and on the last row of B when N % 4 != 0, whose final
  bytes the kernel adds after the MFMAs.  Everything else must match the
  fp64 oracle.
* Scales over many orders of magnitude.  Per-group fp32 scales from 2^-40 to
  2^40 (and some zero) leave every product finite in fp32; the result must
  match the oracle within the FP8 tolerance, which is relative to the sum
  of |scaled products|.
* Every code.  Each of the 254 finite e4m3 values appears in every row of A
  and every column of B, so the MFMA's decoding of normals, subnormals and
  both zeros is checked against the oracle's decoding of the OCP format.
"""

import numpy as np
import pytest
import torch

import tiled_gemm_04_amd as tg
import workloads as wl
from oracle import gemm as og

pytestmark = pytest.mark.gpu

TOL_FP8 = 1.5e-2


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


def _run(qa, sa, qb, sb, path):
    M, N = qa.shape[0], qb.shape[1]
    c = torch.empty(M, N, dtype=torch.bfloat16, device=qa.device)
    if path == "auto":
        tg.gemm_fp8_blockscaled(qa, sa, qb, sb, c)
    elif path == "whole":
        tg.gemm_fp8_blockscaled_ex(qa, sa, qb, sb, c, split_parts=1)
    else:  # the weight as [N, K]
        bt = qb.view(torch.uint8).t().contiguous().view(torch.float8_e4m3fn)
        tg.gemm_fp8_blockscaled_nt(qa, sa, bt, sb, c)
    torch.cuda.synchronize()
    return c.float().cpu().double().numpy()


@pytest.mark.parametrize("path", ["auto", "whole", "nt"])
@pytest.mark.parametrize("shape", [(300, 700, 384), (260, 703, 384)])
def test_nan_codes_reach_their_row_and_column(shape, path):
    dev = _dev()
    M, N, K = shape
    if path == "nt" and K % 16:
        pytest.skip("the [N, K] kernel needs K % 16 == 0")
    qa, sa, qb, sb = wl.fp8_inputs(wl.WORKLOADS["fp8"], device=dev, M=M, N=N, K=K)
    ra, rb = qa.view(torch.uint8), qb.view(torch.uint8)
    i_nan, k_a = 5, 17
    k_b, j_nan = (200, 123) if N % 4 == 0 else (K - 1, N - 1)  # N % 4 != 0: B's last row, last column
    ra[i_nan, k_a] = 0x7F
    rb[k_b, j_nan] = 0xFF
    print(f"[gpu] fp8 NaN codes {path} M={M} N={N} K={K}", flush=True)
    got = _run(qa, sa, qb, sb, path)
    mask = np.zeros((M, N), dtype=bool)
    mask[i_nan, :] = True
    mask[:, j_nan] = True
    assert np.isnan(got[mask]).all()
    assert np.isfinite(got[~mask]).all()
    y, d = og.gemm_fp8_blockscaled_bits(wl.bits_u8(qa), sa.cpu().numpy(), wl.bits_u8(qb), sb.cpu().numpy())
    assert np.isnan(y[mask]).all() and np.isfinite(y[~mask]).all()
    r = og.compare(got[~mask], y[~mask], d[~mask], TOL_FP8)
    assert r["ok"], r


@pytest.mark.parametrize("path", ["auto", "whole"])
def test_scales_over_many_orders_of_magnitude(path):
    dev = _dev()
    M, N, K = 257, 300, 1024
    qa, _, qb, _ = wl.fp8_inputs(wl.WORKLOADS["fp8"], device=dev, M=M, N=N, K=K)
    G, H = (K + 127) // 128, (N + 127) // 128
    g = torch.Generator().manual_seed(97)
    sa = (torch.rand(M, G, generator=g) + 1.0) * torch.pow(2.0, torch.randint(-40, 41, (M, G), generator=g).float())
    sb = (torch.rand(G, H, generator=g) + 1.0) * torch.pow(2.0, torch.randint(-40, 41, (G, H), generator=g).float())
    sa[3, 2] = 0.0
    sb[1, 0] = 0.0
    sa, sb = sa.to(dev), sb.to(dev)
    print(f"[gpu] fp8 extreme scales {path} M={M} N={N} K={K}", flush=True)
    got = _run(qa, sa, qb, sb, path)
    assert np.isfinite(got).all()
    y, d = og.gemm_fp8_blockscaled_bits(wl.bits_u8(qa), sa.cpu().numpy(), wl.bits_u8(qb), sb.cpu().numpy())
    r = og.compare(got, y, d, TOL_FP8)
    assert r["ok"], r


def test_every_finite_code():
    dev = _dev()
    M, N, K = 256, 256, 256
    r = np.arange(M)[:, None]
    k = np.arange(K)[None, :]
    a_codes = ((r + k) % 256).astype(np.uint8)
    kk = np.arange(K)[:, None]
    n = np.arange(N)[None, :]
    b_codes = ((3 * kk + 7 * n) % 256).astype(np.uint8)
    for codes in (a_codes, b_codes):
        codes[(codes & 0x7F) == 0x7F] = 0x00  # the two NaN codes become +0
    qa = torch.from_numpy(a_codes).to(dev).view(torch.float8_e4m3fn)
    qb = torch.from_numpy(b_codes).to(dev).view(torch.float8_e4m3fn)
    sa = torch.ones(M, K // 128, device=dev)
    sb = torch.ones(K // 128, (N + 127) // 128, device=dev)
    print(f"[gpu] fp8 every code M={M} N={N} K={K}", flush=True)
    got_auto = _run(qa, sa, qb, sb, "auto")
    got_whole = _run(qa, sa, qb, sb, "whole")
    assert np.array_equal(got_auto, got_whole)
    y, d = og.gemm_fp8_blockscaled_bits(a_codes, sa.cpu().numpy(), b_codes, sb.cpu().numpy())
    res = og.compare(got_auto, y, d, TOL_FP8)
    assert res["ok"], res
