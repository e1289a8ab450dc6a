"""Per-group FP8 quantiser -- test infrastructure.

The DeepGEMM page (section 2.4, low-precision numerics) describes scaling a
row or a small block of data by one factor so that it fits the narrow FP8
range, with groups of about 128 elements or a small matrix block.  The
groups here are the ones the GEMM consumes: one scale per (row, 128-wide K
group) of the activation matrix A and one per 128 x 128 block of the weight
matrix B.  The readings used for the points the page leaves open:

* scale ``s = amax / 448`` in fp32 (round to nearest), where ``amax`` is the
  largest magnitude over the in-range elements of the group; a group that is
  all zero gets ``s = 1``;
* code ``q = e4m3(clamp(x / s, -448, 448))`` with ``x / s`` in fp32 and the
  cast rounding to nearest, ties to even (saturating before the cast);
* dequantised value ``decode(q) * s``;
* groups at ragged edges cover only the elements inside the matrix.

Weight-only int8 (the GEMM compute-cost page, section 7.2: store the LM-head
weight in a low-precision integer format), round to nearest per group: one
scale per (128 consecutive rows, column) of W [K, N]:

* ``s = amax / 127`` in fp32 (round to nearest), 1 for an all-zero group;
* ``q = rint(clamp(w / s, -127, 127))`` with ``w / s`` in fp32 and ties to
  even, stored as int8 (the code -128 is never produced).

Weight-only int4 (section 4.3 of the same page lists int4 beside int8), the
same scheme with 4-bit codes: ``s = amax / 7``, ``q = rint(clamp(w / s, -7,
7))`` (the code -8 is never produced), packed two per byte along K: byte
``(r, n)`` holds ``q[2r, n]`` in bits 0-3 and ``q[2r + 1, n]`` in bits 4-7,
two's complement.
"""

import numpy as np

from .formats import E4M3_MAX, e4m3_encode_rne

GROUP = 128


def _quantise_group(x):
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    s = np.float32(1.0) if amax == 0 else np.float32(amax / np.float32(E4M3_MAX))
    scaled = (x / s).astype(np.float32)
    scaled = np.clip(scaled, -E4M3_MAX, E4M3_MAX)
    return e4m3_encode_rne(scaled), s


def quantise_rows_1x128(x):
    """A [M, K] fp32 -> (codes uint8 [M, K], scales fp32 [M, ceil(K/128)])."""
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    G = (K + GROUP - 1) // GROUP
    q = np.zeros((M, K), dtype=np.uint8)
    s = np.zeros((M, G), dtype=np.float32)
    for i in range(M):
        for g in range(G):
            sl = slice(g * GROUP, min(K, (g + 1) * GROUP))
            q[i, sl], s[i, g] = _quantise_group(x[i, sl])
    return q, s


def quantise_blocks_128x128(x):
    """B [K, N] fp32 -> (codes uint8 [K, N], scales fp32 [ceil(K/128), ceil(N/128)])."""
    x = np.asarray(x, dtype=np.float32)
    K, N = x.shape
    G, H = (K + GROUP - 1) // GROUP, (N + GROUP - 1) // GROUP
    q = np.zeros((K, N), dtype=np.uint8)
    s = np.zeros((G, H), dtype=np.float32)
    for g in range(G):
        for h in range(H):
            rs = slice(g * GROUP, min(K, (g + 1) * GROUP))
            cs = slice(h * GROUP, min(N, (h + 1) * GROUP))
            q[rs, cs], s[g, h] = _quantise_group(x[rs, cs])
    return q, s


INT8_MAX = 127.0


INT4_MAX = 7.0


def _quantise_int_k128(w, qmax):
    w = np.asarray(w, dtype=np.float32)
    K, N = w.shape
    G = (K + GROUP - 1) // GROUP
    q = np.zeros((K, N), dtype=np.int8)
    s = np.zeros((G, N), dtype=np.float32)
    for g in range(G):
        rs = slice(g * GROUP, min(K, (g + 1) * GROUP))
        amax = np.max(np.abs(w[rs]), axis=0).astype(np.float32)
        sg = np.where(amax == 0, np.float32(1.0), (amax / np.float32(qmax)).astype(np.float32))
        sg = sg.astype(np.float32)
        scaled = (w[rs] / sg[None, :]).astype(np.float32)
        q[rs] = np.rint(np.clip(scaled, -qmax, qmax)).astype(np.int8)
        s[g] = sg
    return q, s


def quantise_int8_k128(w):
    """W [K, N] fp32 -> (int8 codes [K, N], fp32 scales [ceil(K/128), N])."""
    return _quantise_int_k128(w, INT8_MAX)


def quantise_int4_k128(w):
    """W [K, N] fp32 (K even) -> (int4 codes as int8 [K, N], fp32 scales
    [ceil(K/128), N]); pack_int4 gives the stored bytes."""
    if np.asarray(w).shape[0] % 2:
        raise ValueError("int4 codes pair up along K: K must be even")
    return _quantise_int_k128(w, INT4_MAX)


def pack_int4(q):
    """int4 codes [K, N] (K even, values -8 .. 7) -> bytes [K/2, N]: the
    two's-complement nibble of row 2r in bits 0-3, of row 2r + 1 in 4-7."""
    q = np.asarray(q, dtype=np.int16)
    if q.shape[0] % 2 or q.min(initial=0) < -8 or q.max(initial=0) > 7:
        raise ValueError("int4 codes must be in [-8, 7] with an even row count")
    nib = (q & 0x0F).astype(np.uint8)
    return (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)
