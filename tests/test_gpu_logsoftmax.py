"""GPU parity of the fused LM head, GEMM + bias + row log-softmax
(gemm_bf16_logsoftmax), against the fp64 oracle (needs an MI355X).

The error of an output is at most twice the largest logit error of its
row (the log-sum-exp moves by at most the largest logit error), plus the
fp32 evaluation of the normaliser and the output's own rounding: the check
is |c - ref| <= 2 tau max_n D[i, n] + tau |lse_i| + r |ref| with
D = sum_k |x||w| + |bias|, tau = 1e-5 (the fp32 GEMM tolerance) and
r = 2^-8 for bf16 output, 2^-23 for fp32 (oracle.gemm.logsoftmax_bound).
Shapes follow the LM head of the GEMM compute-cost page (section 7.2).
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


def _inputs(M, N, K, seed, dev, bias=True, w_sigma=0.02):
    x = wl.bf16((M, K), "normal", 1.0, seed, 1, dev)
    w = wl.bf16((K, N), "normal", w_sigma, seed, 2, dev)
    b = wl.bf16((N,), "normal", 0.02, seed, 3, dev) if bias else None
    return x, w, b


def _run(x, w, b, out_dtype, label):
    M, N = x.shape[0], w.shape[1]
    big, c = _guarded_out(M, N, out_dtype, x.device)
    out = tg.OUT_BF16 if out_dtype == torch.bfloat16 else tg.OUT_F32
    ws = torch.full((tg.gemm_logsoftmax_workspace_size(M, N, out),), 0xFF, dtype=torch.uint8, device=x.device)
    print(f"[gpu] logsoftmax {label} M={M} N={N} K={x.shape[1]} bias={b is not None} out={out_dtype}",
          flush=True)
    tg.gemm_bf16_logsoftmax(x, w, b, c, workspace=ws)
    torch.cuda.synchronize()
    assert _guards_intact(big, M, N)
    return c


def _check(x, w, b, out_dtype, label, ref=None):
    c = _run(x, w, b, out_dtype, label)
    if ref is None:
        ref = og.gemm_bf16_logsoftmax_bits(wl.bits_u16(x), wl.bits_u16(w),
                                           None if b is None else wl.bits_u16(b))
    M = x.shape[0]
    out, dmax, lse = ref[0][:M], ref[1][:M], ref[2][:M]
    bound = og.logsoftmax_bound(out, dmax, lse, "f32" if out_dtype == torch.float32 else "bf16")
    r = og.compare(c.float().cpu().double().numpy(), out, bound, 1.0)
    assert r["ok"], f"{label}: {r}"
    return c


@pytest.mark.parametrize("shape", [(1, 512, 4096), (5, 1000, 256), (16, 4104, 64), (17, 2048, 136),
                                   (33, 8192, 1000), (64, 520, 384), (64, 8, 8), (48, 65536, 64),
                                   (2, 131072, 32), (3, 200008, 64)])
def test_logsoftmax_shapes(shape):
    M, N, K = shape
    x, w, b = _inputs(M, N, K, 61, _dev())
    _check(x, w, b, torch.bfloat16, "shape")


@pytest.mark.parametrize("bias", [False, True])
@pytest.mark.parametrize("out", [torch.bfloat16, torch.float32])
def test_logsoftmax_bias_and_outputs(bias, out):
    x, w, b = _inputs(9, 3000, 512, 62, _dev(), bias=bias, w_sigma=0.1)
    _check(x, w, b, out, "bias/out")


def test_logsoftmax_k_zero_is_log_softmax_of_bias():
    dev = _dev()
    M, N = 3, 1024
    x = torch.empty(M, 0, dtype=torch.bfloat16, device=dev)
    w = torch.empty(0, N, dtype=torch.bfloat16, device=dev)
    b = wl.bf16((N,), "normal", 2.0, 63, 3, dev)
    c = _run(x, w, b, torch.float32, "K=0")
    ref = og.log_softmax_rows(np.tile(b.float().cpu().double().numpy(), (M, 1)))
    assert np.allclose(c.cpu().double().numpy(), ref, rtol=0, atol=2e-6)


def test_logsoftmax_rows_normalised_and_matches_unfused_path():
    """exp(out) sums to 1 per row, and out equals log_softmax of the plain
    GEMM's fp32 logits (gemm_bf16 with the bias epilogue) up to fp32 rounding."""
    dev = _dev()
    M, N, K = 24, 50000 - 50000 % 8, 1024
    x, w, b = _inputs(M, N, K, 64, dev, w_sigma=0.05)
    c = _run(x, w, b, torch.float32, "vs unfused")
    logits = torch.empty(M, N, dtype=torch.float32, device=dev)
    tg.gemm_bf16(x, w, b, logits, epilogue=tg.EPI_BIAS)
    ref = torch.log_softmax(logits, dim=1)
    torch.cuda.synchronize()
    assert torch.allclose(torch.exp(c.double()).sum(dim=1), torch.ones(M, dtype=torch.float64, device=dev),
                          rtol=0, atol=1e-4)
    assert (c - ref).abs().max().item() < 1e-4


def test_logsoftmax_fp32_output_with_padded_rows():
    """fp32 output in a wider buffer (ldc = N + 8): the logits pass through C
    itself; the guard columns stay intact."""
    x, w, b = _inputs(6, 2056, 256, 67, _dev())
    _check(x, w, b, torch.float32, "fp32 padded")


def test_logsoftmax_deterministic_and_workspace_contents_irrelevant():
    dev = _dev()
    x, w, b = _inputs(8, 20000, 512, 65, dev)
    c1 = _run(x, w, b, torch.bfloat16, "run 1").clone()
    c2 = _run(x, w, b, torch.bfloat16, "run 2")
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))


def test_logsoftmax_rejects_bad_arguments():
    dev = _dev()
    x, w, b = _inputs(4, 1024, 64, 66, dev)
    c = torch.empty(4, 1024, dtype=torch.bfloat16, device=dev)
    small = torch.empty(tg.gemm_logsoftmax_workspace_size(4, 1024) - 1, dtype=torch.uint8, device=dev)
    with pytest.raises(tg.TgemmError):
        tg.gemm_bf16_logsoftmax(x, w, b, c, workspace=small)     # workspace too small
    x65, w65, _ = _inputs(65, 1024, 64, 66, dev)
    c65 = torch.empty(65, 1024, dtype=torch.bfloat16, device=dev)
    with pytest.raises(tg.TgemmError):
        tg.gemm_bf16_logsoftmax(x65, w65, None, c65)             # M > 64
    w12 = torch.zeros(64, 1028, dtype=torch.bfloat16, device=dev)
    c12 = torch.empty(4, 1028, dtype=torch.bfloat16, device=dev)
    with pytest.raises(tg.TgemmError):
        tg.gemm_bf16_logsoftmax(x, w12, None, c12)               # N % 8 != 0


def test_full_size_lm_head_logsoftmax():
    """The LM head [M, 4096] x [4096, 128256] + bias with log-softmax, M = 1,
    8, 32, 64 (nested rows of one X), bf16 and fp32 output, every output
    checked; with fp32 output each row's probabilities also sum to 1."""
    dev = _dev()
    w = wl.WORKLOADS["thin_m64"]
    x, wt, _ = wl.bf16_inputs(w, device=dev)
    b = wl.bf16((w.N,), "normal", 0.02, w.seed, 3, dev)
    ref = og.gemm_bf16_logsoftmax_bits(wl.bits_u16(x), wl.bits_u16(wt), wl.bits_u16(b))
    for M in (1, 8, 32, 64):
        for out_dtype in (torch.bfloat16, torch.float32):
            c = _check(x[:M].contiguous(), wt, b, out_dtype, f"lm_head M={M}", ref=ref)
            if out_dtype == torch.float32:
                total = c.double().exp().sum(dim=1).cpu()
                assert torch.allclose(total, torch.ones(M, dtype=torch.float64), rtol=0, atol=2e-4), total
