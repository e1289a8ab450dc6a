"""GPU: the allocation-free split entry point (gemm_bf16_noalloc) against
gemm_bf16_ex with a caller workspace (needs an MI355X).

gemm_bf16_noalloc runs the same small-M K split as gemm_bf16_ex, with the
partials in the library's fixed device scratch array instead of a caller
workspace.  Two calls in a row (the second on a smaller problem, so the
array holds the first call's partials when the second starts) must each
equal the workspace call bit for bit and match the fp64 oracle; free device
memory must not change across calls; a split larger than the scratch must
be rejected before anything is enqueued, and problems that do not split
must run without touching it.
"""

import pytest
import torch

import tiled_gemm_04_amd as tg
import workloads as wl
from oracle import gemm as og

pytestmark = pytest.mark.gpu

TOL_F32, TOL_BF16 = 1e-5, 8e-3


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


def _case(M, N, K, seed, dev, epi, out):
    a = wl.bf16((M, K), "normal", 1.0, seed, 1, dev)
    b = wl.bf16((K, N), "normal", 0.05, seed, 2, dev)
    bias = wl.bf16((N,), "normal", 0.5, seed, 3, dev) if epi != tg.EPI_NONE else None
    need = tg.gemm_bf16_workspace_size(M, N, K)
    assert 0 < need <= tg.NOALLOC_SCRATCH_BYTES, need
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    return a, b, bias, ws, torch.empty(M, N, dtype=out, device=dev), torch.empty(M, N, dtype=out, device=dev)


def test_noalloc_matches_workspace_call_on_two_calls_in_a_row():
    dev = _dev()
    cases = [((64, 4096, 4096), 131, tg.EPI_BIAS_GELU_TANH, torch.bfloat16),
             ((8, 2048, 2048), 132, tg.EPI_BIAS, torch.float32)]   # the second is smaller
    built = [_case(*shape, seed, dev, epi, out) for shape, seed, epi, out in cases]
    for (shape, _, epi, out), (a, b, bias, ws, c_ref, c_na) in zip(cases, built):
        print(f"[gpu] noalloc M={shape[0]} N={shape[1]} K={shape[2]} epi={epi} out={out}", flush=True)
        tg.gemm_bf16_ex(a, b, bias, c_ref, epilogue=epi, workspace=ws)
        tg.gemm_bf16_noalloc(a, b, bias, c_na, epilogue=epi)
        torch.cuda.synchronize()
        raw = torch.int16 if out == torch.bfloat16 else torch.int32
        assert torch.equal(c_na.view(raw), c_ref.view(raw))
        y, d = og.gemm_bf16_bits(wl.bits_u16(a), wl.bits_u16(b), None if bias is None else wl.bits_u16(bias), epi)
        r = og.compare(c_na.float().cpu().double().numpy(), y, d, TOL_F32 if out == torch.float32 else TOL_BF16)
        assert r["ok"], r


def test_noalloc_allocates_nothing_and_repeats_bit_identically():
    dev = _dev()
    a, b, bias, ws, c_ref, c = _case(16, 4096, 4096, 133, dev, tg.EPI_BIAS, torch.bfloat16)
    print("[gpu] noalloc memory", flush=True)
    tg.gemm_bf16_noalloc(a, b, bias, c_ref, epilogue=tg.EPI_BIAS)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(10):
        tg.gemm_bf16_noalloc(a, b, bias, c, epilogue=tg.EPI_BIAS)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0, (free0, free1)
    assert torch.equal(c.view(torch.int16), c_ref.view(torch.int16))


def test_noalloc_rejects_splits_beyond_its_scratch_and_runs_unsplit_shapes():
    dev = _dev()
    M, N, K = 64, 51200, 4096   # 100 stripes: 3 chunks x 64 x 51200 fp32 = 39.3 MB
    assert tg.gemm_bf16_workspace_size(M, N, K) > tg.NOALLOC_SCRATCH_BYTES
    a = wl.bf16((M, K), "normal", 1.0, 134, 1, dev)
    b = wl.bf16((K, N), "normal", 0.05, 134, 2, dev)
    c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    print("[gpu] noalloc rejects and unsplit shapes", flush=True)
    with pytest.raises(tg.TgemmError) as ei:
        tg.gemm_bf16_noalloc(a, b, None, c)
    assert ei.value.status == tg.TGEMM_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool(torch.isnan(c.float()).all())   # nothing was enqueued
    # Shapes that do not split run without scratch, equal to gemm_bf16.
    for (m, n, k) in ((8, 66048, 256), (300, 264, 200)):
        assert tg.gemm_bf16_workspace_size(m, n, k) == 0
        x = wl.bf16((m, k), "normal", 1.0, 135, 1, dev)
        w = wl.bf16((k, n), "normal", 0.05, 135, 2, dev)
        c1 = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
        c2 = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
        tg.gemm_bf16(x, w, None, c1)
        tg.gemm_bf16_noalloc(x, w, None, c2)
        torch.cuda.synchronize()
        assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))
