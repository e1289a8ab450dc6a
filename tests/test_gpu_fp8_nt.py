"""GPU parity of the FP8 block-scaled GEMM with a K-contiguous weight
(gemm_fp8_blockscaled_nt; needs an MI355X).

The weight arrives as Bt [N, K], the layout nn.Linear keeps (GEMM
compute-cost page, section 5.2: operands in the layout the kernel reads).
Every case is checked against the fp64 oracle on B = Btᵀ at the FP8
tolerance, and, where N % 4 == 0, against gemm_fp8_blockscaled on the
transposed weight bit for bit (the same MFMA operands, schedule and tile
split; for N % 4 != 0 the [K, N] kernel adds the last B row's final bytes
after its main loop, a different summation order).
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


def _out(M, N, dev):
    buf = torch.full((M * N + 2,), CANARY_BF16, dtype=torch.int16, device=dev)
    return buf, buf[1:M * N + 1].view(torch.bfloat16).view(M, N)


def _check_guards(buf, M, N):
    assert int(buf[0]) == CANARY_BF16 and int(buf[M * N + 1]) == CANARY_BF16


def _oracle(qa, sa, qb, sb, c, rows=None):
    sel = slice(None) if rows is None else torch.as_tensor(rows, device=qa.device)
    y, d = og.gemm_fp8_blockscaled_bits(wl.bits_u8(qa[sel]), sa[sel].cpu().numpy(), wl.bits_u8(qb),
                                        sb.cpu().numpy())
    r = og.compare(c[sel].float().cpu().double().numpy(), y, d, TOL_FP8)
    assert r["ok"], r


@pytest.mark.parametrize("shape", [(256, 128, 128), (300, 264, 384), (300, 260, 208), (17, 129, 144),
                                   (513, 1000, 1024), (1, 8, 16), (40, 5, 128), (33, 130, 96),
                                   (70, 67, 208), (300, 323, 1040), (600, 700, 2048),
                                   # N < 4: the [K, N] call runs its byte-wise kernel
                                   (19, 3, 160), (7, 1, 48)])
def test_fp8_nt_matches_oracle_and_kn_path(shape):
    dev = _dev()
    M, N, K = shape
    print(f"[gpu] fp8 nt M={M} N={N} K={K}", flush=True)
    qa, sa, qb, sb = wl.fp8_inputs(wl.WORKLOADS["fp8"], device=dev, M=M, N=N, K=K)
    bt = qb.t().contiguous()
    buf, c = _out(M, N, dev)
    tg.gemm_fp8_blockscaled_nt(qa, sa, bt, sb, c)
    torch.cuda.synchronize()
    _check_guards(buf, M, N)
    _oracle(qa, sa, qb, sb, c)
    if N % 4 == 0:  # both calls on the direct kernel, same tile split and order
        c_kn = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        tg.gemm_fp8_blockscaled(qa, sa, qb, sb, c_kn)
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.int16), c_kn.view(torch.int16))


def test_fp8_nt_unaligned_operands():
    """A and Bt at odd byte offsets, C at an odd element offset."""
    dev = _dev()
    M, N, K = 97, 131, 256
    print(f"[gpu] fp8 nt unaligned M={M} N={N} K={K}", flush=True)
    qa, sa, qb, sb = wl.fp8_inputs(wl.WORKLOADS["fp8"], device=dev, M=M, N=N, K=K)
    bt = qb.t().contiguous()
    ra = torch.zeros(M * K + 3, dtype=torch.uint8, device=dev)
    ra[3:].copy_(qa.view(torch.uint8).reshape(-1))
    rb = torch.zeros(N * K + 5, dtype=torch.uint8, device=dev)
    rb[5:].copy_(bt.view(torch.uint8).reshape(-1))
    a_u = ra[3:].view(torch.float8_e4m3fn).view(M, K)
    b_u = rb[5:].view(torch.float8_e4m3fn).view(N, K)
    buf, c = _out(M, N, dev)
    tg.gemm_fp8_blockscaled_nt(a_u, sa, b_u, sb, c)
    torch.cuda.synchronize()
    _check_guards(buf, M, N)
    _oracle(qa, sa, qb, sb, c)


def test_fp8_nt_k_not_multiple_of_16_is_unsupported():
    dev = _dev()
    M, N, K = 16, 16, 200
    qa, sa, qb, sb = wl.fp8_inputs(wl.WORKLOADS["fp8"], device=dev, M=M, N=N, K=K)
    c = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    with pytest.raises(tg.TgemmError):
        tg.gemm_fp8_blockscaled_nt(qa, sa, qb.t().contiguous(), sb, c)


@pytest.mark.parametrize("name", ["fp8", "fp8_ragged"])
def test_fp8_nt_full_size(name):
    """The full FP8 shapes: sampled rows of every tile row within the
    oracle's tolerance, and (N % 4 == 0) bit-equal to the [K, N] call on the
    whole output."""
    dev = _dev()
    w = wl.WORKLOADS[name]
    print(f"[gpu] fp8 nt full {name} M={w.M} N={w.N} K={w.K}", flush=True)
    qa, sa, qb, sb = wl.fp8_inputs(w, device=dev)
    bt = qb.t().contiguous()
    c = torch.empty(w.M, w.N, dtype=torch.bfloat16, device=dev)
    tg.gemm_fp8_blockscaled_nt(qa, sa, bt, sb, c)
    c_kn = torch.empty_like(c)
    tg.gemm_fp8_blockscaled(qa, sa, qb, sb, c_kn)
    torch.cuda.synchronize()
    if w.N % 4 == 0:
        assert torch.equal(c.view(torch.int16), c_kn.view(torch.int16))
    rows = sorted({min(w.M - 1, r) for t in range(0, w.M, 256) for r in (t, t + 255, t + 53)})
    _oracle(qa, sa, qb, sb, c, rows)
