"""GPU parity of the weight-only int8 GEMM (gemm_bf16_w8) against the fp64
oracle on the dequantised weights (needs an MI355X).

The kernel forms exact products x * q (a code is exact in bf16), sums them
in fp32 per 128-row group and scales each group's sum by its fp32 scale, so
its error is that of an fp32-accumulated GEMM: the same tolerances as the
bf16 path, max |c - y| / (sum_k |x||q s| + |bias|) <= 1e-5 for fp32 output
and 8e-3 for bf16 output.  Shapes follow the LM head of the GEMM
compute-cost page (section 7.2): few rows, very many columns.
"""

import numpy as np
import pytest
import torch

import tiled_gemm_04_amd as tg
import workloads as wl
from oracle import gemm as og

pytestmark = pytest.mark.gpu

TOL_F32, TOL_BF16 = 1e-5, 8e-3
CANARY_BF16 = 0x7FC1
CANARY_F32 = 0x7FC00001


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


def _guarded_out(M, N, dtype, dev, pad_cols=6):
    ldc = N + pad_cols
    if dtype == torch.bfloat16:
        big = torch.full((M + 2, ldc), CANARY_BF16, dtype=torch.int16, device=dev).view(torch.bfloat16)
    else:
        big = torch.full((M + 2, ldc), CANARY_F32, dtype=torch.int32, device=dev).view(torch.float32)
    return big, big[1:M + 1, :N]


def _guards_intact(big, M, N):
    raw = big.view(torch.int16 if big.dtype == torch.bfloat16 else torch.int32)
    canary = CANARY_BF16 if big.dtype == torch.bfloat16 else CANARY_F32
    return bool((raw[0] == canary).all()) and bool((raw[M + 1] == canary).all()) and \
        bool((raw[1:M + 1, N:] == canary).all())


def _inputs(M, N, K, seed, dev, bias=False):
    x = wl.bf16((M, K), "normal", 1.0, seed, 1, dev)
    q, s = wl.w8_weights(K, N, seed, dev)
    b = wl.bf16((N,), "normal", 0.02, seed, 3, dev) if bias else None
    return x, q, s, b


def _check(x, q, s, b, epi, out_dtype, label, cols=None, workspace=None):
    dev = x.device
    M, N = x.shape[0], q.shape[1]
    big, c = _guarded_out(M, N, out_dtype, dev)
    print(f"[gpu] w8 {label} M={M} N={N} K={x.shape[1]} epi={epi} out={out_dtype}", flush=True)
    tg.gemm_bf16_w8(x, q, s, b, c, epilogue=epi, workspace=workspace)
    torch.cuda.synchronize()
    assert _guards_intact(big, M, N)
    qc, sc = (q, s) if cols is None else (q[:, cols], s[:, cols])
    y, d = og.gemm_bf16_w8_bits(wl.bits_u16(x), qc.cpu().numpy(), sc.cpu().numpy(),
                                None if b is None else wl.bits_u16(b if cols is None else b[cols]), epi)
    got = c if cols is None else c[:, cols]
    tol = TOL_F32 if out_dtype == torch.float32 else TOL_BF16
    r = og.compare(got.float().cpu().double().numpy(), y, d, tol)
    assert r["ok"], f"{label}: {r}"


@pytest.mark.parametrize("shape", [(1, 512, 4096), (5, 100, 200), (16, 1000, 256), (17, 1028, 136),
                                   (33, 2048, 1000), (64, 516, 384), (64, 4, 8), (48, 1536, 128)])
def test_w8_shapes(shape):
    M, N, K = shape
    x, q, s, _ = _inputs(M, N, K, 31, _dev())
    _check(x, q, s, None, tg.EPI_NONE, torch.bfloat16, "shape")


@pytest.mark.parametrize("shape", [(1, 4096, 4096), (8, 14336, 4096), (33, 2048, 4096), (64, 4096, 4096),
                                   (5, 1000, 1992), (16, 516, 2056)])
@pytest.mark.parametrize("out", [torch.bfloat16, torch.float32])
def test_w8_split_k(shape, out):
    """Narrow weights (at most 128 stripes of 512 columns) are cut along K
    into chunks of whole 128-row scale groups when a workspace is given; the
    fp32 partials are summed in chunk order with the bias and tanh-GeLU.
    Checked against the oracle with and without the workspace (unsplit)."""
    M, N, K = shape
    dev = _dev()
    x, q, s, b = _inputs(M, N, K, 4700 + M + K, dev, bias=True)
    need = tg.gemm_wq_workspace_size(M, N, K)
    assert need > 0 and need % 256 == 0
    assert "splitk" in tg.gemm_w8_kernel_name(M, N, K, with_workspace=True)
    assert "splitk" not in tg.gemm_w8_kernel_name(M, N, K)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=dev)
    _check(x, q, s, b, tg.EPI_BIAS_GELU_TANH, out, "split-k", workspace=ws)
    _check(x, q, s, b, tg.EPI_BIAS_GELU_TANH, out, "unsplit")


@pytest.mark.parametrize("epi", [tg.EPI_NONE, tg.EPI_BIAS, tg.EPI_BIAS_GELU_TANH])
@pytest.mark.parametrize("out", [torch.bfloat16, torch.float32])
def test_w8_epilogues_and_outputs(epi, out):
    x, q, s, b = _inputs(8, 700, 512, 32, _dev(), bias=True)
    _check(x, q, s, b, epi, out, "epilogue")


def test_w8_strided_and_unaligned():
    """X with row stride K + 3 starting one element into its buffer, Q with
    row stride N + 4 bytes starting 4 bytes in, C at an odd element offset."""
    dev = _dev()
    M, N, K = 9, 600, 264
    xb = wl.bf16((M * (K + 3) + 1,), "normal", 1.0, 33, 1, dev)
    x = xb[1:].view(M, K + 3)[:, :K]
    q0, s = wl.w8_weights(K, N, 33, dev)
    qbuf = torch.zeros(K * (N + 4) + 4, dtype=torch.int8, device=dev)
    q = qbuf[4:].view(K, N + 4)[:, :N]
    q.copy_(q0)
    cbuf = torch.full((M * N + 2,), CANARY_BF16, dtype=torch.int16, device=dev)
    c = cbuf[1:M * N + 1].view(torch.bfloat16).view(M, N)
    print(f"[gpu] w8 strided M={M} N={N} K={K}", flush=True)
    tg.gemm_bf16_w8(x, q, s, None, c)
    torch.cuda.synchronize()
    assert int(cbuf[0]) == CANARY_BF16 and int(cbuf[M * N + 1]) == CANARY_BF16
    y, d = og.gemm_bf16_w8_bits(wl.bits_u16(x.contiguous()), q.cpu().numpy(), s.cpu().numpy())
    r = og.compare(c.float().cpu().double().numpy(), y, d, TOL_BF16)
    assert r["ok"], r


def test_w8_stripe_beyond_2gib_rebuilds_windows_per_slice():
    """A weight whose rows are 16 MiB apart: a stripe of 256 rows spans
    4.3 GB, past what one buffer window can address, so the kernel builds a
    window per slice instead of one for the whole stripe."""
    dev = _dev()
    M, N, K, ldq = 5, 600, 256, 1 << 24
    assert (K - 1) * ldq >= 1 << 31
    x, q0, s, b = _inputs(M, N, K, 34, dev, bias=True)
    qbuf = torch.empty(K * ldq, dtype=torch.int8, device=dev)
    q = qbuf.view(K, ldq)[:, :N]
    q.copy_(q0)
    _check(x, q, s, b, tg.EPI_BIAS, torch.float32, "rows 16 MiB apart")
    del qbuf, q
    torch.cuda.empty_cache()


def test_w8_k_zero_is_epilogue_of_bias():
    dev = _dev()
    M, N = 3, 64
    x = torch.empty(M, 0, dtype=torch.bfloat16, device=dev)
    q = torch.empty(0, N, dtype=torch.int8, device=dev)
    s = torch.empty(0, N, dtype=torch.float32, device=dev)
    b = wl.bf16((N,), "normal", 1.0, 34, 3, dev)
    c = torch.empty(M, N, dtype=torch.float32, device=dev)
    tg.gemm_bf16_w8(x, q, s, b, c, epilogue=tg.EPI_BIAS)
    torch.cuda.synchronize()
    assert torch.equal(c.cpu(), b.float().cpu().expand(M, N))


def test_w8_unsupported_shapes_raise():
    dev = _dev()
    x, q, s, _ = _inputs(65, 64, 64, 35, dev)
    c = torch.empty(65, 64, dtype=torch.bfloat16, device=dev)
    with pytest.raises(tg.TgemmError):
        tg.gemm_bf16_w8(x, q, s, None, c)           # M > 64
    x, q, s, _ = _inputs(4, 66, 64, 35, dev)
    c = torch.empty(4, 66, dtype=torch.bfloat16, device=dev)
    with pytest.raises(tg.TgemmError):
        tg.gemm_bf16_w8(x, q, s, None, c)           # N % 4 != 0


def test_full_size_lm_head_w8():
    """The LM head [M, 4096] x [4096, 128256] with int8 weights at M = 1, 8,
    32, 64 (the thin-M workloads' X), checked on 2,048 sampled columns
    including both edges."""
    dev = _dev()
    w = wl.WORKLOADS["thin_m64"]
    x, _, _ = wl.bf16_inputs(w, device=dev)
    q, s = wl.w8_weights(w.K, w.N, w.seed, dev)
    g = torch.Generator().manual_seed(92)
    cols = torch.cat([torch.arange(0, 256), torch.randint(256, w.N - 256, (1536,), generator=g),
                      torch.arange(w.N - 256, w.N)]).to(dev)
    for M in (1, 8, 32, 64):
        _check(x[:M].contiguous(), q, s, None, tg.EPI_NONE, torch.bfloat16, f"lm_head M={M}", cols=cols)
