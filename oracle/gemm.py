"""The plain GEMM the hot path must reproduce, in float64 -- test infrastructure.

What is computed (all in float64 on exactly decoded inputs):

* Contraction.  ``y[i, j] = sum_k a[i, k] * b[k, j]`` for row-major
  ``a[M, K]`` and ``b[K, N]``: the naive triple loop that the DeepGEMM page
  (section 3.2, 朴素版的性能基线) keeps as the golden reference, with the
  element ``A[m*K + k] * B[k*N + n]`` indexing of that section.  The loop is
  plain C in float64 (``contract.c``, called through ``native.py``): every
  output element adds its K products one at a time, k ascending, each
  product and each addition rounded once.  Its rounding error (at most about
  ``K * 2**-53`` relative to ``sum_k |a||b|``) is eight orders of magnitude
  below the tolerances it is used against.
* Bias.  A linear layer is a GEMM followed by a bias add (GEMM compute-cost
  page, section 2.1, the note on nn.Linear; the formula ``Y = X W + b`` of its
  section 3.1): ``y[i, j] += bias[j]``, broadcast over rows.
* Activation.  Fused epilogue order is "add bias, apply activation, write
  back" (GEMM compute-cost page, section 5.1).  The activation is the tanh
  form of GeLU: ``0.5 * y * (1 + tanh(sqrt(2/pi) * (y + 0.044715 * y**3)))``.
* FP8 block scales.  FP8 inputs carry one fp32 scale per group (DeepGEMM page,
  section 2.4): one per (row, 128-wide K group) of A and one per 128 x 128
  block of B.  Each element is dequantised as ``decode(q) * scale`` before the
  same contraction; both factors are exact in float64, so the dequantised
  operands are exact.
* Weight-only int8.  The LM head's first remedy on the GEMM compute-cost page
  (section 7.2) keeps the weight in a low-precision integer format; with the
  per-group scales of the DeepGEMM page (section 2.4) each weight is
  ``q[k, n] * s[k // 128, n]`` (int8 code times the fp32 scale of its
  128-row group and column), exact in float64, before the same contraction
  with the bf16 activations.
* Weight-only int4.  The same with 4-bit codes (the GEMM compute-cost page,
  section 4.3, names int4 beside int8).  Storage: byte ``(r, n)`` of the
  packed matrix holds the codes of K rows ``2r`` (bits 0-3) and ``2r + 1``
  (bits 4-7) of column ``n``, each a 4-bit two's-complement number, so a
  nibble ``v`` is the code ``v - 16`` when ``v >= 8`` and ``v`` otherwise.
* Log-softmax head.  The LM head's second remedy on the GEMM compute-cost
  page (section 7.2) fuses the output GEMM, the bias add and the LogSoftmax
  that follows it.  Per row: ``out[i, n] = y[i, n] - lse_i`` with
  ``y = x w + b`` and ``lse_i = m_i + log(sum_n exp(y[i, n] - m_i))``,
  ``m_i = max_n y[i, n]`` (the textbook log-sum-exp, shifted by the maximum
  so no exponential overflows).  Error bound (the page gives none; this is
  derived from the arithmetic): logits computed with fp32 accumulation
  carry errors ``|e_n| <= tau * D[i, n]`` (``tau`` the fp32 GEMM tolerance,
  ``D`` as below).  Since ``lse`` is a softmax-weighted mean of its
  arguments to first order, it moves by at most ``max_n |e_n|``, so each
  output moves by at most ``2 * tau * max_n D[i, n]`` (reached when the
  dominant logit errs one way and another logit the other way).  The
  normaliser itself is evaluated in fp32 (exponentials, their sum, the
  logarithm), which adds ``tau * |lse_i|``.  Rounding the output to its
  format adds half an ulp: at most ``2**-8 * |out|`` for bfloat16 (8
  significant bits) and ``2**-23 * |out|`` for float32 (one ulp, covering
  the final subtraction as well).  The bound is the sum of the three.
* FLOP count.  A multiply-add counts as two operations, so an ``[M,K]x[K,N]``
  product costs ``2*M*N*K`` (GEMM compute-cost page, section 3.1); the bias is
  not counted.
* Error metric.  ``err[i, j] = |c - y| / D[i, j]`` with
  ``D = sum_k |a[i,k]| |b[k,j]| + |bias[j]|``; the check passes when
  ``max err <= tol``.  ``D == 0`` gives 0 when ``c == y`` and infinity
  otherwise; a NaN in ``c`` gives infinity.
"""

import math

import numpy as np

from . import native
from .formats import bf16_decode, e4m3_decode

EPI_NONE = 0
EPI_BIAS = 1
EPI_BIAS_GELU_TANH = 2

FP8_GROUP = 128  # K-group width of the A scales; B scales cover 128 x 128 blocks
W8_GROUP = 128   # rows of Q sharing one scale per column (weight-only int8)

GELU_C = math.sqrt(2.0 / math.pi)
GELU_A = 0.044715


def gelu_tanh(y):
    """tanh-approximation GeLU in float64."""
    y = np.asarray(y, dtype=np.float64)
    return 0.5 * y * (1.0 + np.tanh(GELU_C * (y + GELU_A * y * y * y)))


def gemm_f64(a, b, bias=None, epilogue=EPI_NONE, threads=None):
    """Reference result and tolerance denominators for ``epi(a @ b + bias)``.

    a: float64 [M, K]; b: float64 [K, N]; bias: float64 [N] or None;
    threads: worker threads of the loop (None: native.default_threads()).
    Returns (y, D): y float64 [M, N] is the exact-input result (no output
    rounding); D float64 [M, N] is ``sum_k |a||b| (+ |bias|)``.
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[0]:
        raise ValueError(f"shape mismatch: a{a.shape} b{b.shape}")
    M, N = a.shape[0], b.shape[1]
    y, d = native.contract(a, b, threads)
    if epilogue in (EPI_BIAS, EPI_BIAS_GELU_TANH):
        if bias is None:
            raise ValueError("bias epilogue without bias")
        bias = np.asarray(bias, dtype=np.float64).reshape(1, N)
        y = y + bias
        d = d + np.abs(bias)
    elif epilogue != EPI_NONE:
        raise ValueError(f"unknown epilogue {epilogue}")
    if epilogue == EPI_BIAS_GELU_TANH:
        y = gelu_tanh(y)
    return y, d


def gemm_bf16_bits(a_bits, b_bits, bias_bits=None, epilogue=EPI_NONE, threads=None):
    """Oracle for the bf16 path on raw uint16 codes (row-major, any 2-D view)."""
    a = bf16_decode(a_bits)
    b = bf16_decode(b_bits)
    bias = None if bias_bits is None else bf16_decode(bias_bits)
    return gemm_f64(a, b, bias, epilogue, threads)


def dequant_fp8_a(qa_bits, sa):
    """A[i, k] = decode(qa[i, k]) * sA[i, k // 128]  (exact in float64)."""
    qa = e4m3_decode(qa_bits)
    sa = np.asarray(sa, dtype=np.float32).astype(np.float64)
    M, K = qa.shape
    g = np.arange(K) // FP8_GROUP
    if sa.shape != (M, (K + FP8_GROUP - 1) // FP8_GROUP):
        raise ValueError(f"sA shape {sa.shape} for A {qa.shape}")
    return qa * sa[:, g]


def dequant_fp8_b(qb_bits, sb):
    """B[k, j] = decode(qb[k, j]) * sB[k // 128, j // 128]  (exact in float64)."""
    qb = e4m3_decode(qb_bits)
    sb = np.asarray(sb, dtype=np.float32).astype(np.float64)
    K, N = qb.shape
    gk = np.arange(K) // FP8_GROUP
    gn = np.arange(N) // FP8_GROUP
    if sb.shape != ((K + FP8_GROUP - 1) // FP8_GROUP, (N + FP8_GROUP - 1) // FP8_GROUP):
        raise ValueError(f"sB shape {sb.shape} for B {qb.shape}")
    return qb * sb[gk][:, gn]


def gemm_bf16_nt_bits(a_bits, bt_bits, bias_bits=None, epilogue=EPI_NONE):
    """The same product with the weight given K-contiguous, bt [N, K]:
    ``y[i, n] = sum_k a[i, k] * bt[n, k]``, i.e. the contraction with
    ``b = bt`` transposed (decoding is elementwise, so it commutes with the
    transpose)."""
    bias = None if bias_bits is None else bf16_decode(bias_bits)
    return gemm_f64(bf16_decode(a_bits), bf16_decode(bt_bits).T, bias, epilogue)


def dequant_w8(q, s):
    """W[k, n] = q[k, n] * s[k // 128, n] for int8 codes q [K, N] and fp32
    scales s [ceil(K/128), N] (exact in float64)."""
    q = np.asarray(q, dtype=np.int8).astype(np.float64)
    s = np.asarray(s, dtype=np.float32).astype(np.float64)
    K, N = q.shape
    if s.shape != ((K + W8_GROUP - 1) // W8_GROUP, N):
        raise ValueError(f"scale shape {s.shape} for codes {q.shape}")
    return q * s[np.arange(K) // W8_GROUP, :]


def gemm_bf16_w8_bits(x_bits, q, s, bias_bits=None, epilogue=EPI_NONE):
    """Oracle for the weight-only int8 path: bf16 activations times the
    dequantised weights, then bias and epilogue."""
    bias = None if bias_bits is None else bf16_decode(bias_bits)
    return gemm_f64(bf16_decode(x_bits), dequant_w8(q, s), bias, epilogue)


def unpack_int4(packed):
    """Packed bytes [K/2, N] -> int4 codes as int8 [K, N] (values -8 .. 7):
    row 2r from the low nibble of byte row r, row 2r + 1 from the high one."""
    p = np.asarray(packed, dtype=np.uint8).astype(np.int16)
    half, N = p.shape
    q = np.zeros((2 * half, N), dtype=np.int8)
    for h, nib in ((0, p & 0x0F), (1, p >> 4)):
        q[h::2] = np.where(nib >= 8, nib - 16, nib).astype(np.int8)
    return q


def dequant_w4(packed, s):
    """W[k, n] = q[k, n] * s[k // 128, n] for packed int4 codes (exact)."""
    return dequant_w8(unpack_int4(packed), s)


def gemm_bf16_w4_bits(x_bits, packed, s, bias_bits=None, epilogue=EPI_NONE):
    """Oracle for the weight-only int4 path (as gemm_bf16_w8_bits)."""
    bias = None if bias_bits is None else bf16_decode(bias_bits)
    return gemm_f64(bf16_decode(x_bits), dequant_w4(packed, s), bias, epilogue)


def log_softmax_rows(y):
    """Row-wise log-softmax of float64 logits: y - (m + log sum exp(y - m))."""
    out, _ = log_softmax_with_lse(y)
    return out


def log_softmax_with_lse(y):
    """(y - lse, lse) per row, lse = m + log sum_n exp(y[:, n] - m), m = row max."""
    y = np.asarray(y, dtype=np.float64)
    m = np.max(y, axis=1, keepdims=True)
    lse = m + np.log(np.sum(np.exp(y - m), axis=1, keepdims=True))
    return y - lse, lse


# Error bound of the log-softmax heads (module docstring): logit term
# 2 * tau * max_n D, normaliser term tau * |lse|, output rounding r * |out|.
LSM_TAU = 1e-5
LSM_OUT_ROUNDING = {"bf16": 2.0 ** -8, "f32": 2.0 ** -23}


def logsoftmax_bound(out, dmax, lse, out_format):
    """Absolute error allowed on each log-softmax output.

    out: float64 [M, N] reference outputs; dmax: [M, 1] the row maxima of
    the logit denominators D; lse: [M, 1] the row normalisers; out_format
    "bf16" or "f32".  Compare with ``compare(c, out, bound, 1.0)``.
    """
    r = LSM_OUT_ROUNDING[out_format]
    return 2.0 * LSM_TAU * np.asarray(dmax) + LSM_TAU * np.abs(np.asarray(lse)) + r * np.abs(out)


def _logsoftmax_reference(y, d):
    out, lse = log_softmax_with_lse(y)
    return out, np.max(d, axis=1, keepdims=True), lse


def gemm_bf16_logsoftmax_bits(x_bits, w_bits, bias_bits=None):
    """Oracle for the fused LM head: (out, dmax, lse) with out the row-wise
    log-softmax of ``x w + b`` in float64, dmax the row maxima of the logit
    denominators ``D = sum_k |x||w| + |b|`` and lse the row normalisers
    (inputs of logsoftmax_bound)."""
    bias = None if bias_bits is None else bf16_decode(bias_bits)
    y, d = gemm_f64(bf16_decode(x_bits), bf16_decode(w_bits), bias, EPI_BIAS if bias is not None
                    else EPI_NONE)
    return _logsoftmax_reference(y, d)


def gemm_bf16_w8_logsoftmax_bits(x_bits, q, s, bias_bits=None):
    """Oracle for the int8-weight LM head with bias and log-softmax (the GEMM
    compute-cost page, section 7.2, plans A and B together): the row-wise
    log-softmax of ``x (q s) + b``, with dmax and lse as
    gemm_bf16_logsoftmax_bits."""
    y, d = gemm_bf16_w8_bits(x_bits, q, s, bias_bits, EPI_BIAS if bias_bits is not None else EPI_NONE)
    return _logsoftmax_reference(y, d)


def gemm_bf16_w4_logsoftmax_bits(x_bits, packed, s, bias_bits=None):
    """As gemm_bf16_w8_logsoftmax_bits for packed int4 codes."""
    y, d = gemm_bf16_w4_bits(x_bits, packed, s, bias_bits, EPI_BIAS if bias_bits is not None else EPI_NONE)
    return _logsoftmax_reference(y, d)


def gemm_fp8_blockscaled_bits(qa_bits, sa, qb_bits, sb):
    """Oracle for the FP8 block-scaled path: dequantise, then contract."""
    return gemm_f64(dequant_fp8_a(qa_bits, sa), dequant_fp8_b(qb_bits, sb))


def flop_count(M, N, K):
    """2*M*N*K: one multiply-add is two floating-point operations."""
    return 2 * int(M) * int(N) * int(K)


def error_ratio(c, y, d):
    """Elementwise ``|c - y| / D`` with the zero-denominator and NaN rules."""
    c = np.asarray(c, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    d = np.asarray(d, dtype=np.float64)
    diff = np.abs(c - y)
    with np.errstate(divide="ignore", invalid="ignore"):
        err = np.where(d > 0, diff / np.where(d > 0, d, 1.0), np.where(diff == 0, 0.0, np.inf))
    err = np.where(np.isnan(c) | np.isnan(diff), np.inf, err)
    return err


def compare(c, y, d, tol):
    """Summary of the check: max / mean error ratio, its position, pass flag."""
    err = error_ratio(c, y, d)
    if err.size == 0:
        return {"max_err": 0.0, "mean_err": 0.0, "argmax": None, "ok": True, "tol": tol}
    idx = int(np.argmax(err))
    mx = float(err.flat[idx])
    return {
        "max_err": mx,
        "mean_err": float(np.mean(np.where(np.isfinite(err), err, 0.0))),
        "argmax": tuple(int(v) for v in np.unravel_index(idx, err.shape)),
        "ok": bool(mx <= tol),
        "tol": tol,
    }
