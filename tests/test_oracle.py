"""Pins of the CPU oracle against things other than itself (no GPU needed).

Each test fixes one part of the oracle to a library routine run exhaustively,
exact rational arithmetic, a closed form, an invariant, or a figure the pages
print (tests/golden/page_figures.json), chosen so that a dropped term, a
wrong sign or index, or a transposed operand in the oracle fails one of them.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads as wl
from oracle import formats, gemm, native, quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


# ---------------------------------------------------------------- formats ---

def test_bf16_decode_all_codes_match_torch():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = formats.bf16_decode(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_bf16_encode_rne_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
        (rng.standard_normal(20000) * 1e-30).astype(np.float32),
        # exact ties: low half == 0x8000 with even and odd upper halves
        (np.arange(0x3F800000, 0x3F800000 + 64 * 0x10000, 0x10000, dtype=np.uint32)
         | np.uint32(0x8000)).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38], dtype=np.float32),
    ])
    ours = formats.bf16_encode_rne(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # 1 + 2**-8 is exactly half way between 1 and 1 + 2**-7: ties to even -> 1.0
    assert formats.bf16_encode_rne(np.float32(1 + 2.0 ** -8)) == 0x3F80
    assert formats.bf16_encode_rne(np.float32(1 + 3 * 2.0 ** -8)) == 0x3F82


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = formats.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_e4m3_encode_round_trips_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = formats.e4m3_decode(codes)
    assert np.array_equal(formats.e4m3_encode_rne(vals), codes)


def test_e4m3_encode_ties_and_clamped_cast_match_torch():
    assert formats.e4m3_encode_rne(np.array([1.0625]))[0] == formats.e4m3_encode_rne(np.array([1.0]))[0]
    assert formats.e4m3_decode(formats.e4m3_encode_rne(np.array([1.1875])))[0] == 1.25
    assert formats.e4m3_decode(formats.e4m3_encode_rne(np.array([2.0 ** -10])))[0] == 0.0
    assert formats.e4m3_decode(formats.e4m3_encode_rne(np.array([3 * 2.0 ** -10])))[0] == 2 * 2.0 ** -9
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.uniform(-448, 448, 100000), rng.standard_normal(100000) * 0.01,
        rng.standard_normal(100000) * 30, np.array([448.0, -448.0, 0.0, -0.0, 2.0 ** -6]),
    ]).astype(np.float32)
    x = np.clip(x, -448, 448)
    ours = formats.e4m3_encode_rne(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    with pytest.raises(ValueError):
        formats.e4m3_encode_rne(np.array([449.0]))


# --------------------------------------------------------------- quantiser ---

def _ulp_e4m3(v):
    """Spacing of e4m3 codes at magnitude v (subnormal spacing below 2**-6)."""
    v = np.abs(v)
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -6)))
    return np.ldexp(1.0, (e - 3).astype(int))


def test_quantiser_invariants():
    rng = np.random.default_rng(2)
    a = rng.standard_normal((5, 300)).astype(np.float32)
    a[1, 128:256] = 0.0                      # an all-zero group
    a[2, 7] = 40.0                           # an outlier
    q, s = quant.quantise_rows_1x128(a)
    assert s.shape == (5, 3)
    assert s[1, 1] == 1.0 and np.all(q[1, 128:256] == 0)
    dec = formats.e4m3_decode(q)
    for i in range(5):
        for g in range(3):
            sl = slice(128 * g, min(300, 128 * (g + 1)))
            x = a[i, sl].astype(np.float64)
            if np.all(x == 0):
                continue
            assert np.max(np.abs(dec[i, sl])) == 448.0
            assert s[i, g] == np.float32(np.float32(np.max(np.abs(a[i, sl]))) / np.float32(448))
            scaled = x / float(s[i, g])
            err = np.abs(scaled - dec[i, sl])
            assert np.all(err <= 0.5 * _ulp_e4m3(scaled) * (1 + 1e-6) + 1e-12)
            nz = dec[i, sl] != 0
            assert np.all(np.sign(dec[i, sl][nz]) == np.sign(x[nz]))


def test_quantiser_matches_generator_bits():
    rng = np.random.default_rng(3)
    a = (rng.standard_normal((33, 300)) * np.where(rng.random((33, 300)) < 0.01, 20, 1)).astype(np.float32)
    b = (rng.standard_normal((260, 390)) * 0.02).astype(np.float32)
    qa, sa = quant.quantise_rows_1x128(a)
    qb, sb = quant.quantise_blocks_128x128(b)
    tqa, tsa = wl.quantise_a_1x128(torch.from_numpy(a))
    tqb, tsb = wl.quantise_b_128x128(torch.from_numpy(b))
    assert np.array_equal(qa, wl.bits_u8(tqa)) and np.array_equal(sa, tsa.numpy())
    assert np.array_equal(qb, wl.bits_u8(tqb)) and np.array_equal(sb, tsb.numpy())
    assert sb.shape == (3, 4)


# ----------------------------------------------------------- contraction ---

def _exact_gemm(a, b, bias=None):
    M, K = a.shape
    N = b.shape[1]
    fa = [[Fraction(float(a[i, k])) for k in range(K)] for i in range(M)]
    fb = [[Fraction(float(b[k, j])) for j in range(N)] for k in range(K)]
    y = np.zeros((M, N), dtype=object)
    d = np.zeros((M, N), dtype=object)
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            t = Fraction(0)
            for k in range(K):
                p = fa[i][k] * fb[k][j]
                s += p
                t += abs(p)
            if bias is not None:
                s += Fraction(float(bias[j]))
                t += abs(Fraction(float(bias[j])))
            y[i, j] = s
            d[i, j] = t
    return y, d


@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 7), (8, 8, 8), (6, 4, 9), (67, 50, 9)])
def test_contraction_matches_exact_rationals(shape):
    M, N, K = shape
    g = torch.Generator().manual_seed(M * 1000 + N * 10 + K)
    a = torch.randn(M, K, generator=g).to(torch.bfloat16)
    b = torch.randn(K, N, generator=g).to(torch.bfloat16)
    bias = torch.randn(N, generator=g).to(torch.bfloat16)
    ab, bb, biasb = wl.bits_u16(a), wl.bits_u16(b), wl.bits_u16(bias)
    for epi in (gemm.EPI_NONE, gemm.EPI_BIAS):
        y, d = gemm.gemm_bf16_bits(ab, bb, biasb if epi else None, epi)
        ey, ed = _exact_gemm(formats.bf16_decode(ab), formats.bf16_decode(bb),
                             formats.bf16_decode(biasb) if epi else None)
        bound = (K + 1) * 2.0 ** -52
        for i in range(M):
            for j in range(N):
                assert abs(Fraction(float(y[i, j])) - ey[i, j]) <= Fraction(bound) * ed[i, j]
                assert abs(Fraction(float(d[i, j])) - ed[i, j]) <= Fraction(bound) * ed[i, j]


def test_identity_gives_b_exactly():
    K, N = 37, 23
    eye = torch.eye(K).to(torch.bfloat16)
    b = torch.randn(K, N, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    y, _ = gemm.gemm_bf16_bits(wl.bits_u16(eye), wl.bits_u16(b))
    assert np.array_equal(y, formats.bf16_decode(wl.bits_u16(b)))
    # right identity on a non-square A: A @ I == A (catches a transposed operand)
    a = torch.randn(11, K, generator=torch.Generator().manual_seed(6)).to(torch.bfloat16)
    y2, _ = gemm.gemm_bf16_bits(wl.bits_u16(a), wl.bits_u16(eye))
    assert np.array_equal(y2, formats.bf16_decode(wl.bits_u16(a)))


def test_rank_one_and_all_ones_closed_forms():
    M, N, K = 9, 13, 300
    rng = np.random.default_rng(7)
    u = rng.integers(-8, 9, M).astype(np.float32)
    v = rng.integers(-8, 9, N).astype(np.float32)
    a = np.repeat(u[:, None], K, axis=1)
    b = np.repeat(v[None, :], K, axis=0)
    y, d = gemm.gemm_bf16_bits(formats.bf16_encode_rne(a), formats.bf16_encode_rne(b))
    assert np.array_equal(y, K * np.outer(u, v).astype(np.float64))
    assert np.array_equal(d, K * np.abs(np.outer(u, v)).astype(np.float64))
    ones_a = formats.bf16_encode_rne(np.ones((M, K), np.float32))
    ones_b = formats.bf16_encode_rne(np.ones((K, N), np.float32))
    y1, _ = gemm.gemm_bf16_bits(ones_a, ones_b)
    assert np.all(y1 == K)


@pytest.mark.parametrize("K", [4096, 16384])
def test_rank_one_and_all_ones_at_production_k(K):
    """The FFN and LM-head depths (K = 4096, 16384): integer rank-1 operands
    give C = K * u_i * v_j exactly and all-ones operands give C = K (every
    partial sum is an integer below 2**53, so the plain loop is exact)."""
    M, N = 3, 40
    rng = np.random.default_rng(K)
    u = rng.integers(-8, 9, M).astype(np.float32)
    v = rng.integers(-8, 9, N).astype(np.float32)
    a = formats.bf16_encode_rne(np.repeat(u[:, None], K, axis=1))
    b = formats.bf16_encode_rne(np.repeat(v[None, :], K, axis=0))
    y, d = gemm.gemm_bf16_bits(a, b)
    assert np.array_equal(y, K * np.outer(u, v).astype(np.float64))
    assert np.array_equal(d, K * np.abs(np.outer(u, v)).astype(np.float64))
    ones_a = formats.bf16_encode_rne(np.ones((M, K), np.float32))
    ones_b = formats.bf16_encode_rne(np.ones((K, N), np.float32))
    y1, d1 = gemm.gemm_bf16_bits(ones_a, ones_b)
    assert np.all(y1 == K) and np.all(d1 == K)


def test_contraction_is_the_plain_loop_k_ascending_without_fma():
    """The golden reference is the naive loop (DeepGEMM page, section 3.2):
    each product rounded once, then added to the running sum, k ascending.
    Two hand-worked cases separate it from other orders and from a fused
    multiply-add:
      * a = [1, 1, 1], b = [2**53, 1, -2**53]: k ascending gives
        (2**53 + 1 -> 2**53, ties to even) - 2**53 = 0, while k descending
        or an exact sum gives 1;
      * a = [1, 1 + 2**-30], b = [-1, 1 + 2**-30]: the product
        1 + 2**-29 + 2**-60 rounds to 1 + 2**-29 before the add, giving
        2**-29; a fused multiply-add would keep the 2**-60."""
    a = np.array([[1.0, 1.0, 1.0]])
    b = np.array([[2.0 ** 53], [1.0], [-(2.0 ** 53)]])
    y, d = gemm.gemm_f64(a, b)
    assert y[0, 0] == 0.0 and d[0, 0] == 2.0 ** 54
    y_rev, _ = gemm.gemm_f64(a[:, ::-1], b[::-1])
    assert y_rev[0, 0] == 1.0
    e = 1.0 + 2.0 ** -30
    y2, _ = gemm.gemm_f64(np.array([[1.0, e]]), np.array([[-1.0], [e]]))
    assert y2[0, 0] == 2.0 ** -29
    assert float(Fraction(-1) + Fraction(e) * Fraction(e)) != 2.0 ** -29  # exact value differs


def test_contraction_does_not_depend_on_the_thread_count():
    rng = np.random.default_rng(8)
    a = rng.standard_normal((37, 300))
    b = rng.standard_normal((300, 51))
    y1, d1 = native.contract(a, b, threads=1)
    y7, d7 = native.contract(a, b, threads=7)
    assert np.array_equal(y1, y7) and np.array_equal(d1, d7)
    # strided views (every other row and column of a larger matrix)
    big = rng.standard_normal((80, 700))
    ys, ds = native.contract(big[::2, :300], b, threads=3)
    yc, dc = native.contract(np.ascontiguousarray(big[::2, :300]), b, threads=3)
    assert np.array_equal(ys, yc) and np.array_equal(ds, dc)


def test_empty_k_gives_bias_only():
    a = np.zeros((3, 0), np.uint16)
    b = np.zeros((0, 4), np.uint16)
    bias = formats.bf16_encode_rne(np.array([1.0, -2.0, 0.5, 3.0], np.float32))
    y, d = gemm.gemm_bf16_bits(a, b, bias, gemm.EPI_BIAS)
    assert np.array_equal(y, np.tile([1.0, -2.0, 0.5, 3.0], (3, 1)))
    assert np.array_equal(d, np.abs(y))


# --------------------------------------------------------------- epilogue ---

def test_gelu_tanh_pins():
    assert gemm.gelu_tanh(0.0) == 0.0
    y = np.linspace(-9, 9, 2001)
    # tanh is odd, so gelu(y) - gelu(-y) == y
    assert np.allclose(gemm.gelu_tanh(y) - gemm.gelu_tanh(-y), y, rtol=1e-15, atol=1e-15)
    ref = F.gelu(torch.from_numpy(y), approximate="tanh").numpy()
    assert np.allclose(gemm.gelu_tanh(y), ref, rtol=1e-14, atol=1e-15)
    assert abs(float(gemm.gelu_tanh(1.0)) - 0.8411919906082768) < 1e-15
    # and it differs from the erf form (catches a wrong activation)
    assert abs(float(gemm.gelu_tanh(1.0)) - 0.5 * (1 + math.erf(1 / math.sqrt(2)))) > 1e-5


def test_bias_gelu_order_is_bias_then_activation():
    a = formats.bf16_encode_rne(np.array([[1.0, 2.0]], np.float32))
    b = formats.bf16_encode_rne(np.array([[0.5, -1.0], [0.25, 1.0]], np.float32))
    bias = formats.bf16_encode_rne(np.array([-1.0, 0.5], np.float32))
    y, d = gemm.gemm_bf16_bits(a, b, bias, gemm.EPI_BIAS_GELU_TANH)
    pre = np.array([1 * 0.5 + 2 * 0.25 - 1.0, -1.0 + 2.0 + 0.5])
    assert np.allclose(y[0], F.gelu(torch.from_numpy(pre), approximate="tanh").numpy(), rtol=0, atol=1e-15)
    assert np.array_equal(d[0], np.array([0.5 + 0.5 + 1.0, 1.0 + 2.0 + 0.5]))


# ------------------------------------------------------------------ FP8 -----

def _fp8_small(M, N, K, seed):
    g = torch.Generator().manual_seed(seed)
    a = torch.randn(M, K, generator=g)
    b = torch.randn(K, N, generator=g) * 0.02
    qa, sa = quant.quantise_rows_1x128(a.numpy())
    qb, sb = quant.quantise_blocks_128x128(b.numpy())
    return qa, sa, qb, sb


def test_fp8_dequantisation_indexing_brute_force():
    M, N, K = 5, 300, 260
    qa, sa, qb, sb = _fp8_small(M, N, K, 8)
    ah = gemm.dequant_fp8_a(qa, sa)
    bh = gemm.dequant_fp8_b(qb, sb)
    for i in range(M):
        for k in range(0, K, 7):
            assert ah[i, k] == formats.e4m3_decode(qa[i, k]) * float(sa[i, k // 128])
    for k in range(0, K, 13):
        for j in range(0, N, 11):
            assert bh[k, j] == formats.e4m3_decode(qb[k, j]) * float(sb[k // 128, j // 128])


def test_fp8_integer_codes_unit_scales_exact():
    M, N, K = 4, 6, 256
    rng = np.random.default_rng(9)
    ia = rng.integers(-4, 5, (M, K)).astype(np.float64)
    ib = rng.integers(-4, 5, (K, N)).astype(np.float64)
    qa, qb = formats.e4m3_encode_rne(ia), formats.e4m3_encode_rne(ib)
    y, _ = gemm.gemm_fp8_blockscaled_bits(qa, np.ones((M, 2), np.float32), qb, np.ones((2, 1), np.float32))
    assert np.array_equal(y, ia @ ib)  # small integers: float64 matmul is exact


def test_fp8_scale_power_of_two_scales_row_and_block():
    M, N, K = 6, 260, 384
    qa, sa, qb, sb = _fp8_small(M, N, K, 10)
    y, _ = gemm.gemm_fp8_blockscaled_bits(qa, sa, qb, sb)
    sa2 = sa.copy()
    sa2[3, :] *= 8.0
    y2, _ = gemm.gemm_fp8_blockscaled_bits(qa, sa2, qb, sb)
    assert np.array_equal(y2[3], 8.0 * y[3])
    assert np.array_equal(np.delete(y2, 3, 0), np.delete(y, 3, 0))
    # one 128x128 block of B scaled by 2**-3: only columns of that block change,
    # and only by the contribution of that K group
    sb2 = sb.copy()
    sb2[1, 2] *= 0.125
    y3, _ = gemm.gemm_fp8_blockscaled_bits(qa, sa, qb, sb2)
    assert np.array_equal(y3[:, :256], y[:, :256])
    ah = gemm.dequant_fp8_a(qa, sa)
    bh = gemm.dequant_fp8_b(qb, sb)
    part = ah[:, 128:256] @ bh[128:256, 256:]
    assert np.allclose(y3[:, 256:], y[:, 256:] - part + 0.125 * part, rtol=0, atol=1e-12)


def test_fp8_equals_bf16_path_on_dequantised_inputs():
    qa, sa, qb, sb = _fp8_small(7, 130, 200, 11)
    y, d = gemm.gemm_fp8_blockscaled_bits(qa, sa, qb, sb)
    y2, d2 = gemm.gemm_f64(gemm.dequant_fp8_a(qa, sa), gemm.dequant_fp8_b(qb, sb))
    assert np.array_equal(y, y2) and np.array_equal(d, d2)


# --------------------------------------------------- metric and FLOP count ---

def test_error_metric_reports_injected_delta():
    rng = np.random.default_rng(12)
    y = rng.standard_normal((5, 7))
    d = np.abs(y) + 1.0
    c = y.copy()
    c[2, 3] += 0.25
    r = gemm.compare(c, y, d, tol=1e-3)
    assert r["argmax"] == (2, 3) and not r["ok"]
    assert abs(r["max_err"] - 0.25 / d[2, 3]) < 1e-15
    z = gemm.error_ratio(np.array([0.0, 1.0, np.nan]), np.zeros(3), np.zeros(3))
    assert z[0] == 0 and np.isinf(z[1]) and np.isinf(z[2])


def test_flop_count_against_page_figures():
    fig = json.load(open(GOLDEN))
    sq = fig["square_4096_flops"]
    flops = gemm.flop_count(sq["M"], sq["N"], sq["K"])
    assert flops == 137_438_953_472
    assert abs(flops - sq["page_value"]) <= sq["rounding"]
    rate = fig["square_4096_rate_at_half_ms"]
    tflops = flops / rate["seconds"] / 1e12
    assert abs(tflops - rate["page_value_tflops"]) <= rate["rounding"]
    util = fig["square_4096_utilisation_vs_500"]
    assert abs(tflops / util["peak_tflops"] - util["page_value_fraction"]) <= util["rounding"]
    assert gemm.flop_count(1, 1, 1) == 2 and gemm.flop_count(3, 5, 0) == 0


# ----------------------------------------------------------------- inputs ---

def test_generator_is_deterministic_and_shaped():
    w = wl.WORKLOADS["tiny"]
    a1, b1, _ = wl.bf16_inputs(w)
    a2, b2, _ = wl.bf16_inputs(w)
    assert torch.equal(a1, a2) and torch.equal(b1, b2)
    assert a1.dtype == torch.bfloat16 and a1.shape == (64, 64)
    assert float(a1.abs().max()) <= 1.0


def test_fp8_generator_outlier_rate_and_scale_shapes():
    w = wl.WORKLOADS["fp8"]
    qa, sa, qb, sb = wl.fp8_inputs(w, M=256, N=384, K=512)
    assert qa.shape == (256, 512) and sa.shape == (256, 4)
    assert qb.shape == (512, 384) and sb.shape == (4, 3)
    dec = formats.e4m3_decode(wl.bits_u8(qa))
    assert np.all(np.max(np.abs(dec.reshape(256, 4, 128)), axis=2) == 448.0)


# ---------------------------------------------------------- weight-only int8 ----

def _w8_small(K, N, seed):
    rng = np.random.default_rng(seed)
    q = rng.integers(-127, 128, (K, N)).astype(np.int8)
    s = (rng.uniform(0.5, 2.0, ((K + 127) // 128, N)) * 1e-3).astype(np.float32)
    return q, s


def test_w8_dequantisation_indexing_brute_force():
    q, s = _w8_small(300, 37, 21)
    w = gemm.dequant_w8(q, s)
    for k in range(0, 300, 7):
        for n in range(37):
            assert w[k, n] == float(q[k, n]) * float(s[k // 128, n])


def test_w8_integer_codes_unit_scales_exact():
    rng = np.random.default_rng(22)
    M, K, N = 3, 260, 9
    x = rng.integers(-3, 4, (M, K)).astype(np.float32)
    q = rng.integers(-127, 128, (K, N)).astype(np.int8)
    xb = formats.bf16_encode_rne(x)
    y, d = gemm.gemm_bf16_w8_bits(xb, q, np.ones((3, N), np.float32))
    assert np.array_equal(y, x.astype(np.float64) @ q.astype(np.float64))
    assert np.array_equal(d, np.abs(x.astype(np.float64)) @ np.abs(q.astype(np.float64)))


def test_w8_power_of_two_scale_changes_one_group():
    rng = np.random.default_rng(23)
    M, K, N = 4, 384, 12
    xb = formats.bf16_encode_rne(rng.standard_normal((M, K)).astype(np.float32))
    q, s = _w8_small(K, N, 24)
    y, _ = gemm.gemm_bf16_w8_bits(xb, q, s)
    s2 = s.copy()
    s2[1, 5] *= 0.25
    y2, _ = gemm.gemm_bf16_w8_bits(xb, q, s2)
    x = formats.bf16_decode(xb)
    part = x[:, 128:256] @ (q[128:256, 5].astype(np.float64) * float(s[1, 5]))
    assert np.array_equal(np.delete(y2, 5, 1), np.delete(y, 5, 1))
    assert np.allclose(y2[:, 5], y[:, 5] - 0.75 * part, rtol=0, atol=1e-12)


def test_w8_equals_bf16_path_when_weights_are_bf16_exact():
    """With power-of-two scales every q * s (|q| <= 127) is exact in bf16, so
    the int8 oracle must equal the bf16 oracle on those weights."""
    rng = np.random.default_rng(25)
    M, K, N = 5, 200, 33
    xb = formats.bf16_encode_rne(rng.standard_normal((M, K)).astype(np.float32))
    q = rng.integers(-127, 128, (K, N)).astype(np.int8)
    s = np.ldexp(1.0, rng.integers(-12, -4, (2, N))).astype(np.float32)
    w = gemm.dequant_w8(q, s)
    wb = formats.bf16_encode_rne(w.astype(np.float32))
    assert np.array_equal(formats.bf16_decode(wb), w)
    y8, d8 = gemm.gemm_bf16_w8_bits(xb, q, s)
    yb, db = gemm.gemm_bf16_bits(xb, wb)
    assert np.array_equal(y8, yb) and np.array_equal(d8, db)


def test_int8_quantiser_invariants_and_ties():
    rng = np.random.default_rng(26)
    w = rng.standard_normal((300, 6)).astype(np.float32)
    w[128:256, 2] = 0.0                      # an all-zero group
    w[0, 4] = 127.0                          # group (0, 4): scale exactly 1 ...
    w[1, 4], w[2, 4], w[3, 4] = 2.5, 3.5, -0.5   # ... so these are exact ties
    q, s = quant.quantise_int8_k128(w)
    assert q.dtype == np.int8 and s.shape == (3, 6)
    assert s[1, 2] == 1.0 and np.all(q[128:256, 2] == 0)
    assert s[0, 4] == 1.0 and (q[1, 4], q[2, 4], q[3, 4]) == (2, 4, 0)
    for g in range(3):
        rs = slice(128 * g, min(300, 128 * (g + 1)))
        for n in range(6):
            col = w[rs, n].astype(np.float64)
            if np.all(col == 0):
                continue
            amax = np.float32(np.max(np.abs(w[rs, n])))
            assert s[g, n] == np.float32(amax / np.float32(127.0))
            assert np.max(np.abs(q[rs, n].astype(np.int64))) == 127
            assert np.all(np.abs(col - q[rs, n] * float(s[g, n])) <= 0.5 * float(s[g, n]) * (1 + 1e-6))


def test_w8_generator_shapes_and_ranges():
    q, s = wl.w8_weights(300, 40, 4)
    assert q.dtype == torch.int8 and tuple(q.shape) == (300, 40)
    assert s.dtype == torch.float32 and tuple(s.shape) == (3, 40)
    assert int(q.min()) >= -127 and int(q.max()) <= 127
    assert float(s.min()) > 0
    q2, s2 = wl.w8_weights(300, 40, 4)
    assert torch.equal(q, q2) and torch.equal(s, s2)


# ---------------------------------------------------------- weight-only int4 ----

def test_int4_unpack_hand_decoded_bytes():
    """Bytes decoded by hand from the storage rule (low nibble = even K row,
    high nibble = odd K row, 4-bit two's complement)."""
    packed = np.array([[0x9F, 0x70], [0x08, 0x80], [0x00, 0xFF]], dtype=np.uint8)
    q = gemm.unpack_int4(packed)
    expect = np.array([[-1, 0], [-7, 7], [-8, 0], [0, -8], [0, -1], [0, -1]], dtype=np.int8)
    assert np.array_equal(q, expect)


def test_int4_unpack_every_byte_closed_form_and_pack_round_trip():
    b = np.arange(256, dtype=np.uint8).reshape(1, 256)
    q = gemm.unpack_int4(b).astype(np.int64)
    lo, hi = q[0], q[1]
    assert lo.min() == -8 and lo.max() == 7 and hi.min() == -8 and hi.max() == 7
    assert np.array_equal(np.mod(lo, 16) + 16 * np.mod(hi, 16), np.arange(256))
    assert np.array_equal(quant.pack_int4(q.astype(np.int8)), b)


def _w4_small(K, N, seed):
    rng = np.random.default_rng(seed)
    packed = rng.integers(0, 256, (K // 2, N)).astype(np.uint8)
    s = (rng.uniform(0.5, 2.0, ((K + 127) // 128, N)) * 1e-2).astype(np.float32)
    return packed, s


def test_w4_dequantisation_indexing_brute_force():
    packed, s = _w4_small(300, 37, 31)
    w = gemm.dequant_w4(packed, s)
    for k in range(0, 300, 5):
        for n in range(37):
            byte = int(packed[k // 2, n])
            nib = (byte >> 4) if k % 2 else (byte & 15)
            code = nib - 16 if nib >= 8 else nib
            assert w[k, n] == code * float(s[k // 128, n])


def test_w4_integer_codes_unit_scales_exact():
    rng = np.random.default_rng(32)
    M, K, N = 3, 260, 9
    x = rng.integers(-3, 4, (M, K)).astype(np.float32)
    q = rng.integers(-8, 8, (K, N)).astype(np.int8)
    xb = formats.bf16_encode_rne(x)
    y, d = gemm.gemm_bf16_w4_bits(xb, quant.pack_int4(q), np.ones((3, N), np.float32))
    assert np.array_equal(y, x.astype(np.float64) @ q.astype(np.float64))
    assert np.array_equal(d, np.abs(x.astype(np.float64)) @ np.abs(q.astype(np.float64)))


def test_w4_equals_w8_oracle_on_the_same_codes():
    """int4 codes are valid int8 codes: both oracles must agree bit for bit,
    bias and epilogue included."""
    rng = np.random.default_rng(33)
    M, K, N = 4, 392, 21
    xb = formats.bf16_encode_rne(rng.standard_normal((M, K)).astype(np.float32))
    bb = formats.bf16_encode_rne(rng.standard_normal(N).astype(np.float32))
    packed, s = _w4_small(K, N, 34)
    for epi in (gemm.EPI_NONE, gemm.EPI_BIAS, gemm.EPI_BIAS_GELU_TANH):
        y4, d4 = gemm.gemm_bf16_w4_bits(xb, packed, s, None if epi == gemm.EPI_NONE else bb, epi)
        y8, d8 = gemm.gemm_bf16_w8_bits(xb, gemm.unpack_int4(packed), s,
                                        None if epi == gemm.EPI_NONE else bb, epi)
        assert np.array_equal(y4, y8) and np.array_equal(d4, d8)


def test_int4_quantiser_invariants_and_ties():
    rng = np.random.default_rng(35)
    w = rng.standard_normal((300, 6)).astype(np.float32)
    w[128:256, 2] = 0.0                          # an all-zero group
    w[0, 4] = 7.0                                # group (0, 4): scale exactly 1 ...
    w[1, 4], w[2, 4], w[3, 4] = 2.5, 3.5, -0.5   # ... so these are exact ties
    q, s = quant.quantise_int4_k128(w)
    assert q.dtype == np.int8 and s.shape == (3, 6)
    assert s[1, 2] == 1.0 and np.all(q[128:256, 2] == 0)
    assert s[0, 4] == 1.0 and (q[1, 4], q[2, 4], q[3, 4]) == (2, 4, 0)
    assert q.min() >= -7 and q.max() <= 7
    for g in range(3):
        rs = slice(128 * g, min(300, 128 * (g + 1)))
        for n in range(6):
            col = w[rs, n].astype(np.float64)
            if np.all(col == 0):
                continue
            amax = np.float32(np.max(np.abs(w[rs, n])))
            assert s[g, n] == np.float32(amax / np.float32(7.0))
            assert np.max(np.abs(q[rs, n].astype(np.int64))) == 7
            assert np.all(np.abs(col - q[rs, n] * float(s[g, n])) <= 0.5 * float(s[g, n]) * (1 + 1e-6))
    assert np.array_equal(gemm.unpack_int4(quant.pack_int4(q)), q)
    with pytest.raises(ValueError):
        quant.quantise_int4_k128(w[:299])


def test_w4_generator_shapes_and_ranges():
    p, s = wl.w4_weights(300, 40, 4)
    assert p.dtype == torch.uint8 and tuple(p.shape) == (150, 40)
    assert s.dtype == torch.float32 and tuple(s.shape) == (3, 40)
    q = gemm.unpack_int4(p.numpy())
    assert q.min() >= -7 and q.max() <= 7 and 1.5 < q.std() < 3.0
    assert float(s.min()) > 0
    p2, s2 = wl.w4_weights(300, 40, 4)
    assert torch.equal(p, p2) and torch.equal(s, s2)


# ---------------------------------------------------------- log-softmax head ----

def test_log_softmax_uniform_logits_is_minus_log_n():
    """W = 0, no bias: every logit is 0, so every output is -log N."""
    rng = np.random.default_rng(51)
    x = formats.bf16_encode_rne(rng.standard_normal((3, 40)).astype(np.float32))
    w = formats.bf16_encode_rne(np.zeros((40, 1000), np.float32))
    out, _, lse = gemm.gemm_bf16_logsoftmax_bits(x, w)
    assert np.allclose(out, -math.log(1000.0), rtol=0, atol=1e-15)
    assert np.allclose(lse, math.log(1000.0), rtol=0, atol=1e-15)


def test_log_softmax_two_columns_closed_form():
    """Two logits a, b: out = (-softplus(b - a), -softplus(a - b)), with
    softplus(t) = max(t, 0) + log1p(exp(-|t|))."""
    def softplus(t):
        return max(t, 0.0) + math.log1p(math.exp(-abs(t)))

    y = np.array([[0.0, 0.0], [1.0, 3.0], [-2.0, 5.0], [1000.0, 0.0]])
    out = gemm.log_softmax_rows(y)
    for (a, b), (oa, ob) in zip(y, out):
        assert abs(oa + softplus(b - a)) < 1e-12
        assert abs(ob + softplus(a - b)) < 1e-12
    assert out[0, 0] == -math.log(2.0)


def test_log_softmax_rows_normalised_shift_invariant_and_library():
    rng = np.random.default_rng(52)
    y = rng.standard_normal((5, 777)) * 7.0
    out = gemm.log_softmax_rows(y)
    assert np.allclose(np.sum(np.exp(out), axis=1), 1.0, rtol=0, atol=1e-13)
    assert np.allclose(gemm.log_softmax_rows(y + 123.25), out, rtol=0, atol=1e-12)
    ref = torch.log_softmax(torch.from_numpy(y), dim=1).numpy()
    assert np.allclose(out, ref, rtol=0, atol=1e-13)
    big = gemm.log_softmax_rows(np.array([[1e4, 0.0, -1e4]]))
    assert np.all(np.isfinite(big)) and big[0, 0] == 0.0


def test_logsoftmax_oracle_applies_bias_before_normalising():
    """Bias enters the logits: a bias that is constant over columns changes
    nothing; a bias on one column moves the distribution by its closed form."""
    rng = np.random.default_rng(53)
    M, K, N = 4, 64, 96
    xb = formats.bf16_encode_rne(rng.standard_normal((M, K)).astype(np.float32))
    wb = formats.bf16_encode_rne((rng.standard_normal((K, N)) * 0.05).astype(np.float32))
    out0, dmax0, lse0 = gemm.gemm_bf16_logsoftmax_bits(xb, wb)
    const = formats.bf16_encode_rne(np.full(N, 2.5, np.float32))
    out1, _, lse1 = gemm.gemm_bf16_logsoftmax_bits(xb, wb, const)
    assert np.allclose(out1, out0, rtol=0, atol=1e-12)
    one = np.zeros(N, np.float32)
    one[7] = 1.0
    out2, _, _ = gemm.gemm_bf16_logsoftmax_bits(xb, wb, formats.bf16_encode_rne(one))
    y = formats.bf16_decode(xb) @ formats.bf16_decode(wb)
    y[:, 7] += 1.0
    ref = y - np.log(np.sum(np.exp(y), axis=1, keepdims=True))
    assert np.allclose(out2, ref, rtol=0, atol=1e-12)
    # A constant bias of 2.5 moves every logit, so the normaliser, by 2.5.
    assert np.allclose(lse1, lse0 + 2.5, rtol=0, atol=1e-12)
    # The row maxima of the logit denominators sum_k |x||w|, by explicit loops.
    xd, wd = formats.bf16_decode(xb), formats.bf16_decode(wb)
    for i in range(M):
        dk = [math.fsum(abs(float(xd[i, k]) * float(wd[k, n])) for k in range(K)) for n in range(N)]
        assert abs(dmax0[i, 0] - max(dk)) <= 1e-13 * max(dk)


# ------------------------------------------------------- K-contiguous weights ----

def test_nt_oracle_brute_force_and_transpose_relation():
    """y[i, n] = sum_k a[i, k] * bt[n, k] by explicit loops on a tiny case,
    and equality with the [K, N] oracle on the transposed weight."""
    rng = np.random.default_rng(71)
    M, N, K = 3, 5, 7
    ab = formats.bf16_encode_rne(rng.standard_normal((M, K)).astype(np.float32))
    btb = formats.bf16_encode_rne(rng.standard_normal((N, K)).astype(np.float32))
    y, d = gemm.gemm_bf16_nt_bits(ab, btb)
    a, bt = formats.bf16_decode(ab), formats.bf16_decode(btb)
    for i in range(M):
        for n in range(N):
            ref = math.fsum(float(a[i, k]) * float(bt[n, k]) for k in range(K))
            assert abs(y[i, n] - ref) <= 1e-15 * max(1.0, abs(ref))
            assert abs(d[i, n] - math.fsum(abs(float(a[i, k]) * float(bt[n, k])) for k in range(K))) < 1e-14
    bias = formats.bf16_encode_rne(rng.standard_normal(N).astype(np.float32))
    y1, d1 = gemm.gemm_bf16_nt_bits(ab, btb, bias, gemm.EPI_BIAS_GELU_TANH)
    y2, d2 = gemm.gemm_bf16_bits(ab, np.ascontiguousarray(btb.T), bias, gemm.EPI_BIAS_GELU_TANH)
    assert np.array_equal(y1, y2) and np.array_equal(d1, d2)


def test_w8_logsoftmax_equals_bf16_head_on_bf16_exact_weights():
    """With power-of-two scales the int8 weights are exact in bf16: the int8
    log-softmax oracle must equal the bf16 one (values and denominators), with
    and without bias; the int4 oracle on the same codes packed must equal the
    int8 one; every row sums to 1 in probability."""
    rng = np.random.default_rng(61)
    M, K, N = 4, 256, 300
    xb = formats.bf16_encode_rne(rng.standard_normal((M, K)).astype(np.float32))
    q = rng.integers(-7, 8, (K, N)).astype(np.int8)
    s = np.ldexp(1.0, rng.integers(-8, -3, (2, N))).astype(np.float32)
    wb = formats.bf16_encode_rne(gemm.dequant_w8(q, s).astype(np.float32))
    bb = formats.bf16_encode_rne((0.3 * rng.standard_normal(N)).astype(np.float32))
    for bias in (None, bb):
        o8, d8, l8 = gemm.gemm_bf16_w8_logsoftmax_bits(xb, q, s, bias)
        ob, db, lb = gemm.gemm_bf16_logsoftmax_bits(xb, wb, bias)
        assert np.array_equal(o8, ob) and np.array_equal(d8, db) and np.array_equal(l8, lb)
        o4, d4, l4 = gemm.gemm_bf16_w4_logsoftmax_bits(xb, quant.pack_int4(q), s, bias)
        assert np.array_equal(o4, o8) and np.array_equal(d4, d8) and np.array_equal(l4, l8)
        assert np.allclose(np.exp(o8).sum(axis=1), 1.0, rtol=1e-12)


def test_w8_logsoftmax_brute_force_small():
    """A 2 x 3 case by hand: logits from explicit loops over the dequantised
    weights, then log-softmax by its definition."""
    xb = formats.bf16_encode_rne(np.array([[1.0, -2.0], [0.5, 0.25]], dtype=np.float32))
    q = np.array([[3, -1, 0], [2, 5, -7]], dtype=np.int8)
    s = np.array([[0.5, 0.25, 2.0]], dtype=np.float32)
    bias = formats.bf16_encode_rne(np.array([0.125, -1.0, 0.0], dtype=np.float32))
    x = formats.bf16_decode(xb)
    b = formats.bf16_decode(bias)
    out, _, _ = gemm.gemm_bf16_w8_logsoftmax_bits(xb, q, s, bias)
    for i in range(2):
        y = [sum(x[i, k] * q[k, n] * float(s[0, n]) for k in range(2)) + b[n] for n in range(3)]
        lse = math.log(sum(math.exp(v) for v in y))
        for n in range(3):
            assert abs(out[i, n] - (y[n] - lse)) <= 1e-14 * max(1.0, abs(y[n] - lse))


# ------------------------------------------- log-softmax error bound ----

def test_logsoftmax_logit_term_bounded_by_twice_the_largest_logit_error_and_tight():
    """Perturbing every logit of a row by at most delta moves each output by
    at most 2 * delta, and the factor 2 is reached: with one dominant logit
    raised by delta (the normaliser follows it almost fully) and another
    lowered by delta, that other output moves by 2 * delta (1 - p) with p the
    dominant probability, here 1 - 1e-13."""
    rng = np.random.default_rng(81)
    delta = 1e-3
    for _ in range(20):
        y = rng.standard_normal((3, 500)) * 4.0
        e = rng.uniform(-delta, delta, y.shape)
        moved = np.abs(gemm.log_softmax_rows(y + e) - gemm.log_softmax_rows(y))
        assert moved.max() <= 2 * delta * (1 + 1e-9)
    y = np.zeros((1, 50))
    y[0, 0] = 35.0  # p0 = 1 / (1 + 49 e^-35) ~ 1 - 3e-14
    e = np.zeros_like(y)
    e[0, 0], e[0, 1] = delta, -delta
    moved = np.abs(gemm.log_softmax_rows(y + e) - gemm.log_softmax_rows(y))
    assert abs(moved[0, 1] - 2 * delta) <= 1e-12
    # One logit alone moved by delta moves the outputs by at most delta.
    e1 = np.zeros_like(y)
    e1[0, 7] = delta
    assert np.abs(gemm.log_softmax_rows(y + e1) - gemm.log_softmax_rows(y)).max() <= delta * (1 + 1e-12)


def test_logsoftmax_rounding_term_is_half_an_ulp_and_tight():
    """Rounding to nearest moves a value by at most half an ulp: 2**-8 of
    its magnitude for bfloat16 (8 significant bits), 2**-24 for float32 (the
    bound uses 2**-23, one ulp); the bfloat16 ratio comes within 1 % of
    2**-8 just below a power of two's first tie."""
    rng = np.random.default_rng(82)
    x = np.concatenate([rng.standard_normal(200000) * 10.0,
                        1.0 + 2.0 ** -8 - rng.uniform(0, 2.0 ** -16, 1000)])
    xb = formats.bf16_decode(formats.bf16_encode_rne(x.astype(np.float32)))
    x32 = x.astype(np.float32).astype(np.float64)
    rb = np.abs(xb - x32) / np.abs(x32)
    assert rb.max() <= gemm.LSM_OUT_ROUNDING["bf16"] and rb.max() > 0.99 * 2.0 ** -8
    r32 = np.abs(x32 - x) / np.abs(x)
    assert r32.max() <= 2.0 ** -24 < gemm.LSM_OUT_ROUNDING["f32"]


def _lm_head_case(M=4, K=4096, N=2048, seed=83):
    """LM-head-like operands: x N(0,1), w N(0,0.02), bias N(0,0.02), bf16."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16)
    w = (torch.randn(K, N, generator=g) * 0.02).to(torch.bfloat16)
    b = (torch.randn(N, generator=g) * 0.02).to(torch.bfloat16)
    return x, w, b


def test_logsoftmax_bound_admits_fp32_arithmetic_and_rejects_planted_mistakes():
    """At the LM head's depth (K = 4096, max D ~ 50) the bound is about
    1.2e-3 nat for fp32 output and 2**-8 |out| more for bf16.  A plain fp32
    implementation (fp32 GEMM, fp32 log-softmax) and its bf16 rounding pass;
    a normaliser off by 0.01 nat (fp32) or 0.1 nat (bf16), a dropped bias, or
    a normaliser that misses half of the exp-sum (ln 2) fail."""
    x, w, b = _lm_head_case()
    out, dmax, lse = gemm.gemm_bf16_logsoftmax_bits(wl.bits_u16(x), wl.bits_u16(w), wl.bits_u16(b))
    assert 30.0 < float(dmax.min()) and float(dmax.max()) < 80.0
    bf32 = gemm.logsoftmax_bound(out, dmax, lse, "f32")
    bb16 = gemm.logsoftmax_bound(out, dmax, lse, "bf16")
    assert float(bf32.max()) < 2e-3

    def ok(c, bound):
        return gemm.compare(c, out, bound, 1.0)["ok"]

    logits32 = x.float() @ w.float() + b.float()
    c32 = torch.log_softmax(logits32, dim=1).double().numpy()
    assert ok(c32, bf32)
    c16 = torch.log_softmax(logits32, dim=1).to(torch.bfloat16).double().numpy()
    assert ok(c16, bb16)
    assert not ok(out - 0.01, bf32)
    assert not ok(out - 0.1, bb16)
    no_bias = torch.log_softmax(x.double() @ w.double(), dim=1).numpy()
    assert not ok(no_bias, bf32)
    assert not ok(out + math.log(2.0), bf32) and not ok(out + math.log(2.0), bb16)
