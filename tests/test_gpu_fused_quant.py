"""GPU parity of the bf16 GEMM with the FP8 1 x 128 quantiser in its epilogue
(gemm_bf16_quant_fp8; needs an MI355X).

The DeepGEMM page (section 1.2) welds activation, quantisation and scaling
into the producing kernel; section 2.4 fixes the per-group scaling.  Three
kinds of check:

* oracle, exact: integer-valued operands whose products and sums are exact in
  fp32 and bf16, so the GEMM output is known exactly; the codes and scales
  must equal the fp64 oracle's quantiser on the oracle's result bit for bit;
* oracle, bound: for random operands, every dequantised output decode(q) * s
  lies within the GEMM tolerance plus half an e4m3 step of the oracle's
  fp64 result, and every scale within the same bound of max |y| / 448 over
  its group;
* the library against itself: codes and scales equal, bit for bit, the
  two-call path (gemm_bf16_ex with bf16 output on the same tile shape, then
  quantize_fp8_1x128 on that output), which is what the header promises.
"""

import numpy as np
import pytest
import torch

import tiled_gemm_04_amd as tg
import workloads as wl
from oracle import formats as of
from oracle import gemm as og
from oracle import quant as oq

pytestmark = pytest.mark.gpu

TOL_BF16 = 8e-3
ALGOS = [tg.ALGO_TILED_256x256, tg.ALGO_TILED_256x128, tg.ALGO_TILED_128x128]
EPIS = [tg.EPI_NONE, tg.EPI_BIAS, tg.EPI_BIAS_GELU_TANH]


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


def _fused(a, b, bias, epi, algo):
    M, N = a.shape[0], b.shape[1]
    G = (N + 127) // 128
    q = torch.full((M, N), 0x7F, dtype=torch.uint8, device=a.device)  # NaN code canary
    s = torch.full((M, G), float("nan"), dtype=torch.float32, device=a.device)
    tg.gemm_bf16_quant_fp8(a, b, bias if epi else None, q, s, epilogue=epi, algo=algo)
    torch.cuda.synchronize()
    return q, s


def _two_calls(a, b, bias, epi, algo):
    M, N = a.shape[0], b.shape[1]
    h = torch.empty(M, N, dtype=torch.bfloat16, device=a.device)
    tg.gemm_bf16_ex(a, b, bias if epi else None, h, epilogue=epi, algo=algo)
    q = torch.empty(M, N, dtype=torch.uint8, device=a.device)
    s = torch.empty(M, (N + 127) // 128, dtype=torch.float32, device=a.device)
    tg.quantize_fp8_1x128(h, q, s)
    torch.cuda.synchronize()
    return q, s


def _bound_check(q, s, y, d):
    """|decode(q) s - y| <= tol D + 2^-4 (|y| + tol D) + 2^-10 s, and the scale
    within the same distance of max|y| / 448 over its group."""
    M, N = y.shape
    qn, sn = q.cpu().numpy(), s.cpu().numpy().astype(np.float64)
    col_scale = np.repeat(sn, 128, axis=1)[:, :N]
    dq = of.e4m3_decode(qn) * col_scale
    gemm_err = TOL_BF16 * d
    bound = gemm_err + 2.0 ** -4 * (np.abs(y) + gemm_err) + 2.0 ** -10 * col_scale
    err = np.abs(dq - y)
    assert np.isfinite(dq).all()
    assert bool((err <= bound).all()), float((err / np.maximum(bound, 1e-300)).max())
    G = sn.shape[1]
    for g in range(G):
        sl = slice(128 * g, min(N, 128 * g + 128))
        amax = np.abs(y[:, sl]).max(axis=1)
        dmax = d[:, sl].max(axis=1)
        want = np.where(amax == 0, 1.0, amax / 448.0)
        ok = np.abs(sn[:, g] - want) <= (TOL_BF16 * dmax * 1.01 + 2.0 ** -8 * amax) / 448.0 + 1e-30
        ok |= (amax == 0) & (sn[:, g] == 1.0)
        assert bool(ok.all()), g


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("epi", [tg.EPI_NONE, tg.EPI_BIAS])
def test_exact_integer_operands_match_oracle_quantiser(algo, epi):
    """Operands in {-1, 0, 1}, integer bias: the GEMM output is exact, so the
    codes and scales are the oracle quantiser's on the oracle's result."""
    dev = _dev()
    M, N, K = 300, 392, 96
    print(f"[gpu] fused q8 exact M={M} N={N} K={K} epi={epi} algo={algo}", flush=True)
    g = torch.Generator().manual_seed(7100 + 10 * algo + epi)
    a = torch.randint(-1, 2, (M, K), generator=g).to(torch.bfloat16).to(dev)
    b = torch.randint(-1, 2, (K, N), generator=g).to(torch.bfloat16).to(dev)
    bias = torch.randint(-3, 4, (N,), generator=g).to(torch.bfloat16).to(dev)
    q, s = _fused(a, b, bias, epi, algo)
    y, _ = og.gemm_bf16_bits(wl.bits_u16(a), wl.bits_u16(b), wl.bits_u16(bias) if epi else None, epi)
    qo, so = oq.quantise_rows_1x128(y.astype(np.float32))
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(s.cpu().numpy(), so)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("epi", EPIS)
@pytest.mark.parametrize("shape", [(300, 264, 200), (257, 1024, 64), (64, 136, 1032), (513, 384, 8)])
def test_random_operands_within_bound_and_equal_two_calls(shape, epi, algo):
    dev = _dev()
    M, N, K = shape
    print(f"[gpu] fused q8 M={M} N={N} K={K} epi={epi} algo={algo}", flush=True)
    seed = 7200 + M + N + K
    a = wl.bf16((M, K), "normal", 1.0, seed, 1, dev)
    b = wl.bf16((K, N), "normal", 0.05, seed, 2, dev)
    bias = wl.bf16((N,), "normal", 0.5, seed, 3, dev)
    q, s = _fused(a, b, bias, epi, algo)
    q2, s2 = _two_calls(a, b, bias, epi, algo)
    assert torch.equal(q, q2)
    assert torch.equal(s, s2)
    y, d = og.gemm_bf16_bits(wl.bits_u16(a), wl.bits_u16(b), wl.bits_u16(bias) if epi else None, epi)
    _bound_check(q, s, y, d)


def test_all_zero_groups_get_unit_scale():
    """A zero row of A gives zero outputs: codes 0 and scale 1 per group
    (without bias); with a bias those rows quantise the bias alone."""
    dev = _dev()
    M, N, K = 256, 256, 64
    print(f"[gpu] fused q8 zero rows M={M} N={N} K={K}", flush=True)
    a = wl.bf16((M, K), "normal", 1.0, 7300, 1, dev)
    a[5] = 0
    a[200] = 0
    b = wl.bf16((K, N), "normal", 0.05, 7300, 2, dev)
    q, s = _fused(a, b, None, tg.EPI_NONE, tg.ALGO_AUTO)
    for r in (5, 200):
        assert bool((q[r] == 0).all()) and bool((s[r] == 1.0).all())
    bias = wl.bf16((N,), "normal", 0.5, 7300, 3, dev)
    qb, sb = _fused(a, b, bias, tg.EPI_BIAS, tg.ALGO_AUTO)
    qo, so = oq.quantise_rows_1x128(bias.float().cpu().numpy()[None, :])
    assert np.array_equal(qb[5].cpu().numpy(), qo[0]) and np.array_equal(sb[5].cpu().numpy(), so[0])


def test_k_zero_quantises_the_bias():
    dev = _dev()
    M, N = 40, 264
    print(f"[gpu] fused q8 K=0 M={M} N={N}", flush=True)
    a = torch.empty(M, 0, dtype=torch.bfloat16, device=dev)
    b = torch.empty(0, N, dtype=torch.bfloat16, device=dev)
    bias = wl.bf16((N,), "normal", 0.5, 7400, 3, dev)
    q, s = _fused(a, b, bias, tg.EPI_BIAS, tg.ALGO_AUTO)
    qo, so = oq.quantise_rows_1x128(np.repeat(bias.float().cpu().numpy()[None, :], M, axis=0))
    assert np.array_equal(q.cpu().numpy(), qo) and np.array_equal(s.cpu().numpy(), so)


def test_unsupported_operands_raise():
    dev = _dev()
    a = wl.bf16((64, 64), "normal", 1.0, 7500, 1, dev)
    b = wl.bf16((64, 100), "normal", 1.0, 7500, 2, dev)  # N % 8 != 0
    q = torch.empty(64, 100, dtype=torch.uint8, device=dev)
    s = torch.empty(64, 1, dtype=torch.float32, device=dev)
    with pytest.raises(tg.TgemmError):
        tg.gemm_bf16_quant_fp8(a, b, None, q, s)
    b2 = wl.bf16((64, 128), "normal", 1.0, 7500, 2, dev)
    q2 = torch.empty(64, 128, dtype=torch.uint8, device=dev)
    with pytest.raises(tg.TgemmError):
        tg.gemm_bf16_quant_fp8(a, b2, None, q2, s, algo=tg.ALGO_THIN)


def test_full_ffn_up_workload():
    """The FFN up-projection (bias + tanh-GeLU) quantised for an FP8
    down-projection: the whole output equals the two-call path bit for bit,
    sampled rows of every tile row are within the bound of the oracle, and
    the codes feed gemm_fp8_blockscaled."""
    dev = _dev()
    w = wl.WORKLOADS["ffn_up"]
    print(f"[gpu] fused q8 ffn_up M={w.M} N={w.N} K={w.K}", flush=True)
    a, b, bias = wl.bf16_inputs(w, device=dev)
    q, s = _fused(a, b, bias, w.epilogue, tg.ALGO_AUTO)
    shape_algo = {"tgemm_bf16_tiled_256x256x32": tg.ALGO_TILED_256x256,
                  "tgemm_bf16_tiled_256x128x64": tg.ALGO_TILED_256x128,
                  "tgemm_bf16_tiled_128x128x64": tg.ALGO_TILED_128x128}[
        tg.gemm_bf16_kernel_name(w.M, w.N, w.K, w.epilogue, tg.OUT_BF16)]
    q2, s2 = _two_calls(a, b, bias, w.epilogue, shape_algo)
    assert torch.equal(q, q2) and torch.equal(s, s2)
    rows = sorted({min(w.M - 1, r) for t in range(0, w.M, 256) for r in (t, t + 255, t + 77)})
    sel = torch.as_tensor(rows, device=dev)
    y, d = og.gemm_bf16_bits(wl.bits_u16(a[sel]), wl.bits_u16(b), wl.bits_u16(bias), w.epilogue)
    _bound_check(q[sel], s[sel], y, d)
