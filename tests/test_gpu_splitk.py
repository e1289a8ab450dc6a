"""GPU parity of the split-K path of the small-M kernel, and of the caller
workspaces every split path takes (needs an MI355X).

With few 512-column stripes (N below 65536) and M <= 64, gemm_bf16_ex with a
workspace splits K into chunks whose fp32 partial sums a second kernel adds
in a fixed order before the bias, the epilogue and the single rounding; the
shapes below all take that path (N = 1000 .. 4104: 2 .. 9 stripes).  Without
a workspace (and always through gemm_bf16) the same problems run unsplit.
Checked against the fp64 oracle at the bf16 path's tolerances, and bit for
bit run to run.  The library allocates nothing: the free device memory is
the same before and after split calls of all three split paths.
"""

import threading

import pytest
import torch

import tiled_gemm_04_amd as tg
import workloads as wl
from oracle import gemm as og

pytestmark = pytest.mark.gpu

TOL_F32, TOL_BF16, TOL_FP8 = 1e-5, 8e-3, 1.5e-2


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


def _inputs(M, N, K, seed, dev, epi=tg.EPI_NONE):
    a = wl.bf16((M, K), "normal", 1.0, seed, 1, dev)
    b = wl.bf16((K, N), "normal", 0.05, seed, 2, dev)
    bias = wl.bf16((N,), "normal", 0.5, seed, 3, dev) if epi != tg.EPI_NONE else None
    return a, b, bias


def _workspace(M, N, K, dev, fill=0xFF):
    need = tg.gemm_bf16_workspace_size(M, N, K)
    assert need > 0 and need % 256 == 0, need
    return torch.full((need,), fill, dtype=torch.uint8, device=dev)


def _oracle_check(a, b, bias, epi, c):
    y, d = og.gemm_bf16_bits(wl.bits_u16(a), wl.bits_u16(b), None if bias is None else wl.bits_u16(bias), epi)
    tol = TOL_F32 if c.dtype == torch.float32 else TOL_BF16
    r = og.compare(c.float().cpu().double().numpy(), y, d, tol)
    assert r["ok"], r


def _check(M, N, K, seed, epi=tg.EPI_NONE, out=torch.bfloat16):
    dev = _dev()
    a, b, bias = _inputs(M, N, K, seed, dev, epi)
    assert "splitk" in tg.gemm_bf16_kernel_name(M, N, K, epi, tg.OUT_BF16, with_workspace=True)
    assert "splitk" not in tg.gemm_bf16_kernel_name(M, N, K, epi, tg.OUT_BF16)
    ws = _workspace(M, N, K, dev)
    c = torch.full((M, N), float("nan"), dtype=out, device=dev)
    print(f"[gpu] splitk M={M} N={N} K={K} epi={epi} out={out}", flush=True)
    tg.gemm_bf16_ex(a, b, bias, c, epilogue=epi, workspace=ws)
    torch.cuda.synchronize()
    _oracle_check(a, b, bias, epi, c)
    return a, b, bias, c, ws


@pytest.mark.parametrize("shape", [(1, 4096, 4096), (8, 4096, 14336), (16, 2048, 1000), (33, 4096, 4096),
                                   (64, 4104, 4096), (1, 1000, 8192), (5, 3000, 2056)])
def test_splitk_shapes(shape):
    M, N, K = shape
    _check(M, N, K, 111 + M)


@pytest.mark.parametrize("epi", [tg.EPI_BIAS, tg.EPI_BIAS_GELU_TANH])
@pytest.mark.parametrize("out", [torch.bfloat16, torch.float32])
def test_splitk_epilogues(epi, out):
    _check(12, 4096, 4096, 112, epi, out)


def test_splitk_deterministic_and_unsplit_without_workspace():
    a, b, bias, c1, ws = _check(4, 4096, 4096, 113, tg.EPI_BIAS, torch.float32)
    c2 = torch.empty_like(c1)
    tg.gemm_bf16_ex(a, b, bias, c2, epilogue=tg.EPI_BIAS, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int32), c2.view(torch.int32))
    # gemm_bf16 (no workspace) runs the unsplit kernel: within tolerance,
    # and a different summation order
    c3 = torch.empty_like(c1)
    tg.gemm_bf16(a, b, bias, c3, epilogue=tg.EPI_BIAS)
    torch.cuda.synchronize()
    _oracle_check(a, b, bias, tg.EPI_BIAS, c3)


def test_splitk_rejects_short_or_unaligned_workspace():
    dev = _dev()
    M, N, K = 8, 4096, 4096
    print("[gpu] split-K workspace rejects", flush=True)
    a, b, _ = _inputs(M, N, K, 116, dev)
    c = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    need = tg.gemm_bf16_workspace_size(M, N, K)
    with pytest.raises(tg.TgemmError):
        tg.gemm_bf16_ex(a, b, None, c, workspace=torch.empty(need - 256, dtype=torch.uint8, device=dev))
    big = torch.empty(need + 16, dtype=torch.uint8, device=dev)
    with pytest.raises(tg.TgemmError):
        tg.gemm_bf16_ex(a, b, None, c, workspace=big[8:need + 8])
    assert tg.gemm_bf16_workspace_size(M, 128256, K) == 0      # wide weight: no split
    assert tg.gemm_bf16_workspace_size(65, N, K) == 0          # tiled kernel: no split
    assert tg.gemm_bf16_workspace_size(-1, N, K) == -1


def test_splitk_on_two_streams():
    """Concurrent calls on two streams, each with its own workspace."""
    dev = _dev()
    M, N, K = 8, 4096, 4096
    a1, a2 = wl.bf16((M, K), "normal", 1.0, 114, 1, dev), wl.bf16((M, K), "normal", 1.0, 115, 1, dev)
    b = wl.bf16((K, N), "normal", 0.05, 114, 2, dev)
    c1, c2 = torch.empty(M, N, dtype=torch.float32, device=dev), torch.empty(M, N, dtype=torch.float32, device=dev)
    w1, w2 = _workspace(M, N, K, dev), _workspace(M, N, K, dev)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(5):
        tg.gemm_bf16_ex(a1, b, None, c1, workspace=w1, stream=s1)
        tg.gemm_bf16_ex(a2, b, None, c2, workspace=w2, stream=s2)
    torch.cuda.synchronize()
    for a, c in ((a1, c1), (a2, c2)):
        _oracle_check(a, b, None, tg.EPI_NONE, c)


def test_split_calls_from_two_host_threads_on_one_stream():
    """Two Python threads enqueue split calls of different N (bf16 split-K
    and the int8 head's split) on the same stream, each with its own
    workspace; every result matches a single-threaded run bit for bit."""
    dev = _dev()
    M, K = 8, 4096
    print("[gpu] split calls from two host threads on one stream", flush=True)
    a, b1, _ = _inputs(M, 4096, K, 117, dev)
    _, b2, _ = _inputs(M, 2048, K, 118, dev)
    q, s = wl.w8_weights(K, 3072, 119, dev)
    stream = torch.cuda.current_stream()
    ref1 = torch.empty(M, 4096, dtype=torch.float32, device=dev)
    ref2 = torch.empty(M, 2048, dtype=torch.float32, device=dev)
    ref3 = torch.empty(M, 3072, dtype=torch.float32, device=dev)
    w1, w2 = _workspace(M, 4096, K, dev), _workspace(M, 2048, K, dev)
    w3 = torch.empty(tg.gemm_wq_workspace_size(M, 3072, K), dtype=torch.uint8, device=dev)
    tg.gemm_bf16_ex(a, b1, None, ref1, workspace=w1)
    tg.gemm_bf16_ex(a, b2, None, ref2, workspace=w2)
    tg.gemm_bf16_w8(a, q, s, None, ref3, workspace=w3)
    torch.cuda.synchronize()
    outs = {k: [torch.empty_like(r) for _ in range(20)] for k, r in ((1, ref1), (2, ref2), (3, ref3))}
    errors = []

    def worker(kind):
        try:
            ws = {1: _workspace(M, 4096, K, dev), 2: _workspace(M, 2048, K, dev),
                  3: torch.empty(w3.numel(), dtype=torch.uint8, device=dev)}[kind]
            for c in outs[kind]:
                if kind == 1:
                    tg.gemm_bf16_ex(a, b1, None, c, workspace=ws, stream=stream)
                elif kind == 2:
                    tg.gemm_bf16_ex(a, b2, None, c, workspace=ws, stream=stream)
                else:
                    tg.gemm_bf16_w8(a, q, s, None, c, workspace=ws, stream=stream)
        except Exception as e:  # reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(k,)) for k in (1, 2, 3)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for kind, ref in ((1, ref1), (2, ref2), (3, ref3)):
        for c in outs[kind]:
            assert torch.equal(c.view(torch.int32), ref.view(torch.int32)), kind


def test_split_paths_allocate_no_device_memory():
    """Free device memory (as the driver reports it) is unchanged across
    split calls of the small-M bf16 kernel, the int8 head and the FP8 tile
    scheduler, once the caller's buffers exist; the split results equal
    the same calls' earlier results."""
    dev = _dev()
    M, N, K = 8, 4096, 4096
    print("[gpu] split paths allocate nothing", flush=True)
    a, b, _ = _inputs(M, N, K, 120, dev)
    q, s = wl.w8_weights(K, N, 121, dev)
    qa, sa, qb, sb = wl.fp8_inputs(wl.WORKLOADS["fp8"], device=dev, M=600, N=700, K=2048)
    c1 = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    c2 = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    c3 = torch.empty(600, 700, dtype=torch.bfloat16, device=dev)
    w1 = _workspace(M, N, K, dev)
    w2 = torch.empty(tg.gemm_wq_workspace_size(M, N, K), dtype=torch.uint8, device=dev)
    n3 = tg.gemm_fp8_workspace_size(600, 700, 2048)
    assert n3 > 0
    w3 = torch.zeros(n3, dtype=torch.uint8, device=dev)
    refs = []
    for _ in range(2):
        tg.gemm_bf16_ex(a, b, None, c1, workspace=w1)
        tg.gemm_bf16_w8(a, q, s, None, c2, workspace=w2)
        tg.gemm_fp8_blockscaled_ex(qa, sa, qb, sb, c3, workspace=w3)
        torch.cuda.synchronize()
        refs.append([c1.clone(), c2.clone(), c3.clone()])
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(10):
        tg.gemm_bf16_ex(a, b, None, c1, workspace=w1)
        tg.gemm_bf16_w8(a, q, s, None, c2, workspace=w2)
        tg.gemm_fp8_blockscaled_ex(qa, sa, qb, sb, c3, workspace=w3)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0, (free0, free1)
    for got, ref in zip((c1, c2, c3), refs[0]):
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    y, d = og.gemm_fp8_blockscaled_bits(wl.bits_u8(qa), sa.cpu().numpy(), wl.bits_u8(qb), sb.cpu().numpy())
    r = og.compare(c3.float().cpu().double().numpy(), y, d, TOL_FP8)
    assert r["ok"], r
