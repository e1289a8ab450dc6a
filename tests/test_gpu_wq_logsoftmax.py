"""GPU parity of the int8 / int4 weight-only LM head with bias and
log-softmax (gemm_bf16_w8_logsoftmax, gemm_bf16_w4_logsoftmax; needs an
MI355X).

The GEMM compute-cost page (section 7.2) names two remedies for the LM
head's cost: an integer weight (plan A) and fusing the output projection,
bias and LogSoftmax (plan B); these calls do both.  Each case is checked
against the fp64 oracle (dequantised weight, bias, row-wise log-softmax)
with the oracle's log-softmax error bound (oracle.gemm.logsoftmax_bound):
|c - out| <= 2 tau max_n D[i, n] + tau |lse_i| + r |out|, tau = 1e-5 (the
fp32 GEMM tolerance), r = 2^-8 for bf16 output and 2^-23 for fp32.  The
logits must also match the plain integer head's (gemm_bf16_w8 with fp32
output) followed by torch's log_softmax.
"""

import numpy as np
import pytest
import torch

import tiled_gemm_04_amd as tg
import workloads as wl
from oracle import gemm as og

pytestmark = pytest.mark.gpu

CANARY_BF16 = 0x7FC1
CANARY_F32 = 0x7FC00001


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


def _guarded_out(M, N, dtype, dev, pad_cols=8):
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


def _inputs(bits, M, N, K, seed, dev, bias=True):
    x = wl.bf16((M, K), "normal", 1.0, seed, 1, dev)
    q, s = (wl.w8_weights if bits == 8 else wl.w4_weights)(K, N, seed, dev)
    b = wl.bf16((N,), "normal", 0.02, seed, 3, dev) if bias else None
    return x, q, s, b


def _run(bits, x, q, s, b, out_dtype):
    M, N = x.shape[0], q.shape[1]
    big, c = _guarded_out(M, N, out_dtype, x.device)
    out = tg.OUT_BF16 if out_dtype == torch.bfloat16 else tg.OUT_F32
    ws = torch.full((tg.gemm_logsoftmax_workspace_size(M, N, out),), 0xFF, dtype=torch.uint8, device=x.device)
    print(f"[gpu] w{bits} logsoftmax M={M} N={N} K={x.shape[1]} bias={b is not None} out={out_dtype}",
          flush=True)
    fn = tg.gemm_bf16_w8_logsoftmax if bits == 8 else tg.gemm_bf16_w4_logsoftmax
    fn(x, q, s, b, c, workspace=ws)
    torch.cuda.synchronize()
    assert _guards_intact(big, M, N)
    return c


def _oracle(bits, x, q, s, b):
    bb = None if b is None else wl.bits_u16(b)
    fn = og.gemm_bf16_w8_logsoftmax_bits if bits == 8 else og.gemm_bf16_w4_logsoftmax_bits
    return fn(wl.bits_u16(x), q.cpu().numpy(), s.cpu().numpy(), bb)


def _fmt(out_dtype):
    return "f32" if out_dtype == torch.float32 else "bf16"


def _compare(c, ref, out_dtype, rows=None):
    out, dmax, lse = ref
    if rows is not None:
        out, dmax, lse = out[:rows], dmax[:rows], lse[:rows]
    bound = og.logsoftmax_bound(out, dmax, lse, _fmt(out_dtype))
    return og.compare(c.float().cpu().double().numpy(), out, bound, 1.0)


def _check(bits, x, q, s, b, out_dtype):
    c = _run(bits, x, q, s, b, out_dtype)
    r = _compare(c, _oracle(bits, x, q, s, b), out_dtype)
    assert r["ok"], r
    return c


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("shape", [(1, 512, 4096), (5, 1000, 256), (17, 2048, 136), (33, 8192, 1000),
                                   (64, 520, 384), (2, 131072, 32), (3, 200008, 64)])
def test_wq_logsoftmax_shapes(bits, shape):
    dev = _dev()
    M, N, K = shape
    x, q, s, b = _inputs(bits, M, N, K, 9100 + M + K, dev)
    _check(bits, x, q, s, b, torch.bfloat16)


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("bias", [False, True])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_wq_logsoftmax_bias_and_outputs(bits, bias, out):
    dev = _dev()
    x, q, s, b = _inputs(bits, 24, 3000, 520, 9200 + bits, dev, bias=bias)
    _check(bits, x, q, s, b, out)


@pytest.mark.parametrize("bits", [8, 4])
def test_wq_logsoftmax_matches_unfused_path(bits):
    """Rows normalise to 1, and the result equals the plain integer head
    (fp32 output, bias epilogue) followed by torch's log_softmax within the
    fp32 tolerance."""
    dev = _dev()
    M, N, K = 9, 5000, 768
    x, q, s, b = _inputs(bits, M, N, K, 9300 + bits, dev)
    c = _check(bits, x, q, s, b, torch.float32)
    assert torch.allclose(c.double().exp().sum(dim=1), torch.ones(M, dtype=torch.float64, device=dev),
                          rtol=1e-5)
    logits = torch.empty(M, N, dtype=torch.float32, device=dev)
    (tg.gemm_bf16_w8 if bits == 8 else tg.gemm_bf16_w4)(x, q, s, b, logits, epilogue=tg.EPI_BIAS)
    ref = torch.log_softmax(logits.double(), dim=1)
    out, dmax, lse = _oracle(bits, x, q, s, b)
    bound = og.logsoftmax_bound(out, dmax, lse, "f32")
    err = ((c.double() - ref).abs().cpu().numpy() / bound).max()
    assert err <= 2.0, err


def test_wq_logsoftmax_k_zero_and_rejects():
    dev = _dev()
    M, N = 3, 1000
    x = torch.empty(M, 0, dtype=torch.bfloat16, device=dev)
    q = torch.empty(0, N, dtype=torch.int8, device=dev)
    s = torch.empty(0, N, dtype=torch.float32, device=dev)
    b = wl.bf16((N,), "normal", 0.5, 9400, 3, dev)
    c = _run(8, x, q, s, b, torch.float32)
    ref = torch.log_softmax(b.double(), dim=0).expand(M, N)
    assert torch.allclose(c.double(), ref, atol=1e-5)
    # M > 64 and N % 4 != 0 are unsupported
    x2, q2, s2, _ = _inputs(8, 65, 512, 128, 9401, dev)
    with pytest.raises(tg.TgemmError):
        tg.gemm_bf16_w8_logsoftmax(x2, q2, s2, None, torch.empty(65, 512, dtype=torch.bfloat16, device=dev))
    x3, q3, s3, _ = _inputs(8, 4, 510, 128, 9402, dev)
    with pytest.raises(tg.TgemmError):
        tg.gemm_bf16_w8_logsoftmax(x3, q3, s3, None, torch.empty(4, 510, dtype=torch.bfloat16, device=dev))


@pytest.mark.parametrize("bits", [8, 4])
def test_wq_logsoftmax_full_lm_head(bits):
    """The 4096 x 128256 LM head with bias at M = 1 and 64, bf16 and fp32
    output, every output checked against the oracle; with fp32 output each
    row's probabilities also sum to 1."""
    dev = _dev()
    w = wl.WORKLOADS["thin_m64"]
    N, K = w.N, w.K
    q, s = (wl.w8_weights if bits == 8 else wl.w4_weights)(K, N, w.seed, dev)
    b = wl.bf16((N,), "normal", 0.02, w.seed, 3, dev)
    x64 = wl.thin_x(w, 64, dev)
    ref = _oracle(bits, x64, q, s, b)  # rows are independent: M = 1 is row 0
    for M in (1, 64):
        x = wl.thin_x(w, M, dev)
        assert torch.equal(x, x64[:M])
        for out_dtype in (torch.bfloat16, torch.float32):
            c = _run(bits, x, q, s, b, out_dtype)
            r = _compare(c, ref, out_dtype, rows=M)
            assert r["ok"], (M, out_dtype, r)
            if out_dtype == torch.float32:
                total = c.double().exp().sum(dim=1).cpu()
                assert torch.allclose(total, torch.ones(M, dtype=torch.float64), rtol=0, atol=2e-4), total
