"""GPU parity of the FP8 tile scheduler's K split (needs an MI355X).

When the last round of 256 x 256 tiles leaves compute units idle, each of its
tiles runs as P workgroups over disjoint ranges of whole 128-wide scale
groups; their fp32 partial tiles are added by the workgroup that finishes
last (DeepGEMM page, section 2.1: small grids leave compute units idle).
Every case is checked against the fp64 oracle at the FP8 tolerance; the
split must not depend on arrival order (bit-identical repeats) and must
leave its counters (the head of the caller's workspace) at zero for the next
call.
"""

import pytest
import torch

import tiled_gemm_04_amd as tg
import workloads as wl
from oracle import gemm as og

pytestmark = pytest.mark.gpu

TOL_FP8 = 1.5e-2
CANARY_BF16 = 0x7FC1


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


def _workspace(M, N, K, parts, dev):
    """A zero-filled workspace for the split (None when the plan does not split)."""
    need = tg.gemm_fp8_workspace_size(M, N, K, parts)
    assert need >= 0 and need % 256 == 0
    return torch.zeros(need, dtype=torch.uint8, device=dev) if need else None


def _run(qa, sa, qb, sb, parts, ws="new"):
    M, K = qa.shape
    N = qb.shape[1]
    if isinstance(ws, str):
        ws = _workspace(M, N, K, parts, qa.device)
    buf = torch.full((M * N + 2,), CANARY_BF16, dtype=torch.int16, device=qa.device)
    c = buf[1:M * N + 1].view(torch.bfloat16).view(M, N)
    tg.gemm_fp8_blockscaled_ex(qa, sa, qb, sb, c, split_parts=parts, workspace=ws)
    torch.cuda.synchronize()
    assert int(buf[0]) == CANARY_BF16 and int(buf[M * N + 1]) == CANARY_BF16
    return c


def _check(qa, sa, qb, sb, c):
    y, d = og.gemm_fp8_blockscaled_bits(wl.bits_u8(qa), sa.cpu().numpy(), wl.bits_u8(qb),
                                        sb.cpu().numpy())
    r = og.compare(c.float().cpu().double().numpy(), y, d, TOL_FP8)
    assert r["ok"], r
    return r


@pytest.mark.parametrize("shape,parts", [
    ((600, 700, 2048), 0),    # automatic: 9 tiles, 2 ranges of 8 groups
    ((256, 256, 16384), 0),   # automatic: 1 tile, 8 ranges of 16 groups
    ((600, 700, 2048), 1),    # never split
    ((600, 700, 2048), 2),
    ((600, 700, 2048), 3),    # uneven ranges: 5, 5, 6 groups
    ((600, 700, 2048), 5),
    ((513, 1000, 384), 3),    # one group per range
    ((300, 323, 1040), 4),    # N % 4 != 0 (last-row patch in the last range) and a partial last group
    ((97, 131, 1024), 8),     # ragged single tile in eight ranges
    ((1, 8, 2048), 8),        # one row
])
def test_fp8_split_matches_oracle(shape, parts):
    dev = _dev()
    M, N, K = shape
    print(f"[gpu] fp8 split M={M} N={N} K={K} parts={parts}", flush=True)
    qa, sa, qb, sb = wl.fp8_inputs(wl.WORKLOADS["fp8"], device=dev, M=M, N=N, K=K)
    c = _run(qa, sa, qb, sb, parts)
    _check(qa, sa, qb, sb, c)


def test_fp8_split_repeats_bit_identical():
    """Arrival order of the ranges does not change the bits, and each call
    leaves the per-tile counters at zero (a stale counter would make the wrong
    workgroup finish the tile on the next call)."""
    dev = _dev()
    M, N, K = 600, 700, 2048
    print(f"[gpu] fp8 split repeats M={M} N={N} K={K}", flush=True)
    qa, sa, qb, sb = wl.fp8_inputs(wl.WORKLOADS["fp8"], device=dev, M=M, N=N, K=K)
    ws = _workspace(M, N, K, 8, dev)
    n_count = 256  # the counter region of 9 split tiles, rounded up to 256 bytes
    first = _run(qa, sa, qb, sb, 8, ws).clone()
    _check(qa, sa, qb, sb, first)
    for _ in range(4):
        again = _run(qa, sa, qb, sb, 8, ws)
        assert torch.equal(first.view(torch.int16), again.view(torch.int16))
        assert int(ws[:n_count].count_nonzero()) == 0


def test_fp8_split_without_workspace_runs_unsplit():
    """No workspace: every tile runs whole (within tolerance of the split
    run); a short or unaligned workspace is rejected."""
    dev = _dev()
    M, N, K = 600, 700, 2048
    print(f"[gpu] fp8 split without workspace M={M} N={N} K={K}", flush=True)
    qa, sa, qb, sb = wl.fp8_inputs(wl.WORKLOADS["fp8"], device=dev, M=M, N=N, K=K)
    c0 = _run(qa, sa, qb, sb, 4, None)
    _check(qa, sa, qb, sb, c0)
    c1 = _run(qa, sa, qb, sb, 1, None)
    assert torch.equal(c0.view(torch.int16), c1.view(torch.int16))
    need = tg.gemm_fp8_workspace_size(M, N, K, 4)
    c = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    with pytest.raises(tg.TgemmError):
        tg.gemm_fp8_blockscaled_ex(qa, sa, qb, sb, c, split_parts=4,
                                   workspace=torch.zeros(need - 256, dtype=torch.uint8, device=dev))
    big = torch.zeros(need + 16, dtype=torch.uint8, device=dev)
    with pytest.raises(tg.TgemmError):
        tg.gemm_fp8_blockscaled_ex(qa, sa, qb, sb, c, split_parts=4, workspace=big[4:need + 4])


def test_fp8_full_size_split_against_unsplit():
    """The full FP8 shape with its last round (128 tiles after three full
    rounds) forced into two K halves; sampled rows of every tile row match
    the oracle, and the whole output stays within a few bf16 ulps of the
    unsplit run."""
    dev = _dev()
    w = wl.WORKLOADS["fp8"]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    if cus == 256:  # MI355X: 896 tiles = 3 full rounds + 128 tiles
        assert tg.gemm_fp8_split_plan(w.M, w.N, w.K, cus, 2) == (768, 128, 2)
    print(f"[gpu] fp8 full split vs unsplit M={w.M} N={w.N} K={w.K}", flush=True)
    qa, sa, qb, sb = wl.fp8_inputs(w, device=dev)
    c_auto = _run(qa, sa, qb, sb, 2)
    c_one = _run(qa, sa, qb, sb, 1)
    rows = sorted({min(w.M - 1, r) for t in range(0, w.M, 256) for r in (t, t + 255, t + 101)})
    sel = torch.as_tensor(rows, device=dev)
    y, d = og.gemm_fp8_blockscaled_bits(wl.bits_u8(qa[sel]), sa[sel].cpu().numpy(), wl.bits_u8(qb),
                                        sb.cpu().numpy())
    for c in (c_auto, c_one):
        r = og.compare(c[sel].float().cpu().double().numpy(), y, d, TOL_FP8)
        assert r["ok"], r
    # both are roundings of fp32 sums of the same products: at most a few bf16 ulps apart
    diff = (c_auto.float() - c_one.float()).abs()
    scale = torch.maximum(c_auto.float().abs(), c_one.float().abs())
    assert bool((diff <= scale * 2.0 ** -6 + 1e-3).all())
