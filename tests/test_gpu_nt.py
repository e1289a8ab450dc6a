"""GPU parity of the bf16 GEMM with K-contiguous weights (gemm_bf16_nt,
Bt [N, K] as nn.Linear stores it) against the fp64 oracle, and against the
[K, N] path on the transposed weight (needs an MI355X).

Both layouts feed the same MFMA sequence with the same operand values, so
the two paths agree bit for bit; against the oracle the bf16 path's
tolerances hold: 1e-5 for fp32 output, 8e-3 for bf16 output.
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


def _inputs(M, N, K, seed, dev, bias=False):
    a = wl.bf16((M, K), "normal", 1.0, seed, 1, dev)
    bt = wl.bf16((N, K), "normal", 1.0, seed, 2, dev)
    b = wl.bf16((N,), "normal", 1.0, seed, 3, dev) if bias else None
    return a, bt, b


def _check(a, bt, b, epi, out_dtype, label, rows=None):
    M, N = a.shape[0], bt.shape[0]
    c = torch.full((M, N), float("nan"), dtype=out_dtype, device=a.device)
    print(f"[gpu] nt {label} M={M} N={N} K={a.shape[1]} epi={epi} out={out_dtype} "
          f"kernel={tg.gemm_bf16_nt_kernel_name(M, N, a.shape[1])}", flush=True)
    tg.gemm_bf16_nt(a, bt, b, c, epilogue=epi)
    torch.cuda.synchronize()
    ar = a if rows is None else a[rows]
    y, d = og.gemm_bf16_nt_bits(wl.bits_u16(ar), wl.bits_u16(bt), None if b is None else wl.bits_u16(b), epi)
    got = c if rows is None else c[rows]
    tol = TOL_F32 if out_dtype == torch.float32 else TOL_BF16
    r = og.compare(got.float().cpu().double().numpy(), y, d, tol)
    assert r["ok"], f"{label}: {r}"
    return c


@pytest.mark.parametrize("shape", [(1, 1, 8), (64, 64, 64), (100, 130, 72), (257, 255, 136),
                                   (300, 517, 200), (513, 1000, 64), (1024, 2048, 512),
                                   (2048, 1536, 256), (96, 16390, 128)])
def test_nt_shapes_every_tile_shape(shape):
    M, N, K = shape
    a, bt, _ = _inputs(M, N, K, 81, _dev())
    _check(a, bt, None, tg.EPI_NONE, torch.bfloat16, "shape")


@pytest.mark.parametrize("epi", [tg.EPI_NONE, tg.EPI_BIAS, tg.EPI_BIAS_GELU_TANH])
@pytest.mark.parametrize("out", [torch.bfloat16, torch.float32])
def test_nt_epilogues_and_outputs(epi, out):
    a, bt, b = _inputs(200, 300, 96, 82, _dev(), bias=True)
    _check(a, bt, b, epi, out, "epilogue")


@pytest.mark.parametrize("shape", [(4096, 4096, 512), (2048, 16384, 256), (2048, 4096, 2048),
                                   (600, 1000, 264)])
def test_nt_equals_kn_path_bit_for_bit(shape):
    M, N, K = shape
    dev = _dev()
    a, bt, b = _inputs(M, N, K, 83, dev, bias=True)
    b_kn = bt.t().contiguous()
    c1 = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    c2 = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    print(f"[gpu] nt vs kn M={M} N={N} K={K}", flush=True)
    tg.gemm_bf16_nt(a, bt, b, c1, epilogue=tg.EPI_BIAS_GELU_TANH)
    tg.gemm_bf16(a, b_kn, b, c2, epilogue=tg.EPI_BIAS_GELU_TANH)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))


def test_nt_strided_weight_rows():
    """Bt rows padded (ldb = K + 24) and A rows padded (lda = K + 8)."""
    dev = _dev()
    M, N, K = 130, 260, 200
    abuf = wl.bf16((M, K + 8), "normal", 1.0, 84, 1, dev)
    btbuf = wl.bf16((N, K + 24), "normal", 1.0, 84, 2, dev)
    _check(abuf[:, :K], btbuf[:, :K], None, tg.EPI_NONE, torch.float32, "strided")


def test_nt_full_size_square_and_ffn():
    """4096^3 and the FFN up-projection with the weight K-contiguous, on
    three sampled rows per 256-row tile."""
    dev = _dev()
    for name in ("square", "ffn_up"):
        w = wl.WORKLOADS[name]
        a, b, bias = wl.bf16_inputs(w, device=dev)
        bt = b.t().contiguous()
        del b
        g = torch.Generator().manual_seed(94)
        rows = torch.cat([torch.tensor([0, w.M - 1]),
                          torch.randint(0, w.M, (3 * (w.M // 256),), generator=g)]).to(dev)
        out = torch.float32 if w.out_f32 else torch.bfloat16
        _check(a, bt, bias, w.epilogue, out, name, rows=rows)


def test_nt_unsupported_and_invalid():
    dev = _dev()
    a, bt, _ = _inputs(64, 64, 60, 85, dev)
    c = torch.empty(64, 64, dtype=torch.bfloat16, device=dev)
    with pytest.raises(tg.TgemmError):
        tg.gemm_bf16_nt(a, bt, None, c)      # K % 8 != 0
    assert tg.gemm_bf16_nt_kernel_name(64, 64, 60) is None
    a, bt, _ = _inputs(4, 8, 16, 85, dev)
    c = torch.empty(4, 8, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        tg.gemm_bf16_nt(a, bt[:, :8], None, c)   # K mismatch


@pytest.mark.parametrize("shape", [(1, 512, 4096), (5, 1000, 200), (16, 130, 64), (17, 2056, 136),
                                   (33, 4096, 1000), (48, 300, 8), (64, 768, 384), (64, 4, 64)])
def test_nt_thin_m_shapes(shape):
    """M <= 64 runs the thin kernel for K-contiguous weights."""
    M, N, K = shape
    assert tg.gemm_bf16_nt_kernel_name(M, N, K).startswith("tgemm_bf16_thin_nt")
    a, bt, _ = _inputs(M, N, K, 86, _dev())
    _check(a, bt, None, tg.EPI_NONE, torch.bfloat16, "thin")


@pytest.mark.parametrize("epi", [tg.EPI_BIAS, tg.EPI_BIAS_GELU_TANH])
@pytest.mark.parametrize("out", [torch.bfloat16, torch.float32])
def test_nt_thin_epilogues(epi, out):
    a, bt, b = _inputs(9, 700, 264, 87, _dev(), bias=True)
    _check(a, bt, b, epi, out, "thin epilogue")


def test_nt_thin_full_lm_head():
    """The LM head 4096 x 128256 with the weight stored [vocab, d_model],
    against the oracle on 2,048 sampled columns and within the same bound of
    the [K, N] thin kernel on the transposed weight (the K-contiguous kernel
    sums the slices in a rotated order, so the bits may differ), for M = 1,
    8, 32, 64."""
    dev = _dev()
    w = wl.WORKLOADS["thin_m64"]
    x, b_kn, _ = wl.bf16_inputs(w, device=dev)
    bt = b_kn.t().contiguous()
    g = torch.Generator().manual_seed(95)
    cols = torch.cat([torch.arange(0, 256), torch.randint(256, w.N - 256, (1536,), generator=g),
                      torch.arange(w.N - 256, w.N)]).to(dev)
    for M in (1, 8, 32, 64):
        xm = x[:M].contiguous()
        c_nt = torch.empty(M, w.N, dtype=torch.float32, device=dev)
        c_kn = torch.empty(M, w.N, dtype=torch.float32, device=dev)
        print(f"[gpu] nt lm_head M={M}", flush=True)
        tg.gemm_bf16_nt(xm, bt, None, c_nt)
        tg.gemm_bf16(xm, b_kn, None, c_kn)
        torch.cuda.synchronize()
        y, d = og.gemm_bf16_nt_bits(wl.bits_u16(xm), wl.bits_u16(bt[cols]))
        r = og.compare(c_nt[:, cols].cpu().double().numpy(), y, d, TOL_F32)
        assert r["ok"], f"M={M}: {r}"
        dfull = (xm.float().abs() @ b_kn.float().abs())
        assert float(((c_nt - c_kn).abs() / dfull.clamp_min(1e-30)).max()) <= 2 * TOL_F32, f"M={M}"
