"""Number formats of the GEMM inputs and outputs, written from their definitions.

bfloat16: the top 16 bits of an IEEE-754 binary32 (1 sign, 8 exponent, 7
fraction bits).  Decoding appends 16 zero bits; encoding rounds a binary32 to
the nearest bfloat16, ties to even.

e4m3fn (OCP 8-bit floating point, "E4M3"): byte ``s eeee mmm`` with exponent
bias 7, no infinities, NaN only for ``e == 15 and m == 7``; subnormals for
``e == 0`` are ``m * 2**-9``; the largest finite value is 448.  The DeepGEMM
page (section 2.4, low-precision numerics) calls for FP8 inputs with group
scale factors; the scale ``amax / 448`` fixes this flavour (448 is the e4m3fn
maximum).

Every function works on numpy arrays and returns float64 (decode) or raw bits
(encode).  Test infrastructure only.
"""

import numpy as np

E4M3_MAX = 448.0
E4M3_MIN_NORMAL_EXP = -6  # 2**-6 is the smallest normal magnitude
E4M3_SUBNORMAL_STEP = 2.0 ** -9


def bf16_decode(bits):
    """uint16 bfloat16 codes -> float64 values (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    as32 = bits.astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # NaN payloads widen quietly
        return as32.view(np.float32).astype(np.float64)


def bf16_encode_rne(x):
    """binary32 values -> uint16 bfloat16 codes, round to nearest, ties to even.

    NaN inputs give a quiet NaN code with the input's sign.  Infinities and
    values that round beyond the largest finite bfloat16 become infinity, as
    IEEE round-to-nearest prescribes.
    """
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lower = u & np.uint64(0xFFFF)
    upper = u >> np.uint64(16)
    half = np.uint64(0x8000)
    round_up = (lower > half) | ((lower == half) & ((upper & np.uint64(1)) == np.uint64(1)))
    out = (upper + round_up.astype(np.uint64)).astype(np.uint16)
    nan = np.isnan(f)
    if np.any(nan):
        sign = (u[nan] >> np.uint64(31)).astype(np.uint16)
        out[nan] = (sign << np.uint16(15)) | np.uint16(0x7FC0)
    return out


def e4m3_decode(codes):
    """uint8 e4m3fn codes -> float64 values (exact; NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.ldexp(1.0, e - 7)
    subnormal = m * E4M3_SUBNORMAL_STEP
    mag = np.where(e == 0, subnormal, normal)
    out = sign * mag
    out = np.where((e == 15) & (c & 0x7 == 7), np.nan, out)
    return out


def e4m3_encode_rne(x):
    """Finite values with |x| <= 448 -> uint8 e4m3fn codes, nearest, ties to even.

    The caller clamps to [-448, 448] first (the quantiser saturates before it
    casts).  Values that are not finite or lie outside that range raise.
    Zero keeps its sign (0x00 or 0x80).
    """
    v = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(v)) or np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("e4m3_encode_rne expects finite values in [-448, 448]")
    sign = np.signbit(v).astype(np.int64)
    a = np.abs(v)
    # Subnormal range: a < 2**-6, value = m * 2**-9 with m in 0..7; m = 8
    # rounds up into the smallest normal, whose code is exactly 8 (e=1, m=0).
    sub_m = np.rint(a / E4M3_SUBNORMAL_STEP).astype(np.int64)
    # Normal range: a = (1 + f) * 2**E with E >= -6.
    mant, exp2 = np.frexp(a)  # a = mant * 2**exp2, mant in [0.5, 1)
    E = exp2.astype(np.int64) - 1
    frac = np.where(a > 0, a / np.ldexp(1.0, E) - 1.0, 0.0)  # exact
    m = np.rint(frac * 8.0).astype(np.int64)  # np.rint: ties to even
    carry = m == 8
    m = np.where(carry, 0, m)
    E = np.where(carry, E + 1, E)
    normal_code = ((E + 7) << 3) | m
    is_sub = a < 2.0 ** E4M3_MIN_NORMAL_EXP
    mag_code = np.where(is_sub, sub_m, normal_code)
    return ((sign << 7) | mag_code).astype(np.uint8)
