"""GPU parity of the FP8 kernel's half tiles (needs an MI355X).

When the last round of 256 x 256 output tiles would occupy at most half of
the compute units, gemm_fp8_blockscaled runs each of those tiles as two
128-row halves over all of K (DeepGEMM page, section 2.1: a grid too small
for the machine leaves compute units idle).  Every output element then sees
the same MFMAs and the same per-group folds in the same order, so the
result must equal the whole-tile one (gemm_fp8_blockscaled_ex with
split_parts = 1) bit for bit, and both must match the fp64 oracle at the
FP8 tolerance.  The shapes cover a grid made only of halves, a tile row
with at most 128 rows (its second half is empty), K not a multiple of 128,
N % 4 != 0 (the last-row patch inside a half) and a 16 x 56 grid whose
last round of 128 tiles is halved; the weight stored [N, K] takes the same
halves (bit-equal to the [K, N] whole-tile call where N % 4 == 0).
"""

import numpy as np
import pytest
import torch

import tiled_gemm_04_amd as tg
import workloads as wl
from oracle import gemm as og

pytestmark = pytest.mark.gpu

TOL_FP8 = 1.5e-2
CANARY = 0x7FC1


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


def _out(M, N, dev):
    buf = torch.full((M * N + 2,), CANARY, dtype=torch.int16, device=dev)
    return buf, buf[1:M * N + 1].view(torch.bfloat16).view(M, N)


def _rows(M, seed):
    """Both edge rows of every 128-row half tile plus one seeded row per 16."""
    rng = np.random.default_rng(seed)
    rows = set()
    for t0 in range(0, M, 128):
        rows.update({t0, min(M - 1, t0 + 127)})
    for b0 in range(0, M, 16):
        rows.add(int(rng.integers(b0, min(M, b0 + 16))))
    return sorted(rows)


@pytest.mark.parametrize("shape", [
    (600, 700, 384),      # 9 tiles, all halved; the third tile row holds 88 rows
    (100, 300, 256),      # one tile row of 100 rows: every second half is empty
    (129, 520, 272),      # K % 128 != 0; a half of one row
    (300, 1027, 256),     # N % 4 == 3: the last-row patch inside a half
    (4000, 14330, 512),   # 896 tiles: the last round's 128 tiles halved, ragged N
])
def test_halves_match_whole_tiles_and_oracle(shape):
    dev = _dev()
    M, N, K = shape
    qa, sa, qb, sb = wl.fp8_inputs(wl.WORKLOADS["fp8"], device=dev, M=M, N=N, K=K)
    print(f"[gpu] fp8 halves M={M} N={N} K={K}", flush=True)
    buf_h, c_h = _out(M, N, dev)
    tg.gemm_fp8_blockscaled(qa, sa, qb, sb, c_h)  # automatic: halves
    buf_w, c_w = _out(M, N, dev)
    tg.gemm_fp8_blockscaled_ex(qa, sa, qb, sb, c_w, split_parts=1)  # whole tiles only
    torch.cuda.synchronize()
    for buf in (buf_h, buf_w):
        assert int(buf[0]) == CANARY and int(buf[M * N + 1]) == CANARY
    assert torch.equal(c_h.view(torch.int16), c_w.view(torch.int16))
    sel = _rows(M, seed=M + N)
    idx = torch.as_tensor(sel, device=dev)
    y, d = og.gemm_fp8_blockscaled_bits(wl.bits_u8(qa[idx]), sa[idx].cpu().numpy(), wl.bits_u8(qb),
                                        sb.cpu().numpy())
    r = og.compare(c_h[idx].float().cpu().double().numpy(), y, d, TOL_FP8)
    assert r["ok"], r


@pytest.mark.parametrize("shape", [(600, 700, 384), (4000, 14336, 512), (4000, 14330, 512)])
def test_halves_weight_nk(shape):
    """[N, K] weight: halves against the oracle; with N % 4 == 0 also bit-equal
    to the whole-tile [K, N] call (for N % 4 != 0 the [K, N] kernel adds the
    last B row's final bytes after the folds, so only the tolerance holds)."""
    dev = _dev()
    M, N, K = shape
    qa, sa, qb, sb = wl.fp8_inputs(wl.WORKLOADS["fp8"], device=dev, M=M, N=N, K=K)
    bt = qb.view(torch.uint8).t().contiguous().view(torch.float8_e4m3fn)
    print(f"[gpu] fp8 halves [N,K] M={M} N={N} K={K}", flush=True)
    buf_h, c_h = _out(M, N, dev)
    tg.gemm_fp8_blockscaled_nt(qa, sa, bt, sb, c_h)
    buf_w, c_w = _out(M, N, dev)
    tg.gemm_fp8_blockscaled_ex(qa, sa, qb, sb, c_w, split_parts=1)
    torch.cuda.synchronize()
    for buf in (buf_h, buf_w):
        assert int(buf[0]) == CANARY and int(buf[M * N + 1]) == CANARY
    if N % 4 == 0:
        assert torch.equal(c_h.view(torch.int16), c_w.view(torch.int16))
    sel = _rows(M, seed=M + N + 1)
    idx = torch.as_tensor(sel, device=dev)
    y, d = og.gemm_fp8_blockscaled_bits(wl.bits_u8(qa[idx]), sa[idx].cpu().numpy(), wl.bits_u8(qb),
                                        sb.cpu().numpy())
    r = og.compare(c_h[idx].float().cpu().double().numpy(), y, d, TOL_FP8)
    assert r["ok"], r
