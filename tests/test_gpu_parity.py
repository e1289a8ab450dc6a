"""GPU parity: the HIP kernels against the fp64 CPU oracle (needs an MI355X).

Every case draws seeded inputs, runs one library call through the C ABI on
the GPU, decodes the exact input bits on the CPU, and compares element by
element with max |c - y| / (sum_k |a||b| + |bias|) <= tol: 1e-5 for fp32
output, 8e-3 for bf16 output, 1.5e-2 for the FP8 path.  Output buffers are
pre-filled with a NaN canary and surrounded by guard rows / columns that must
come back untouched.  The self-check list of the DeepGEMM page (section 4.4:
small sizes element by element, non-aligned sizes such as 67 x 50, random
and all-ones inputs) and its edge-tile advice (section 4.1) shape the cases.
At the full workload sizes the oracle evaluates sampled rows (both edges of
every M tile and one random row of every 32-row block) or sampled columns for
the thin-M shapes.
"""

import numpy as np
import pytest
import torch

import tiled_gemm_04_amd as tg
import workloads as wl
from oracle import gemm as og

pytestmark = pytest.mark.gpu

TOL_F32, TOL_BF16, TOL_FP8 = 1e-5, 8e-3, 1.5e-2
CANARY_BF16 = 0x7FC1  # a NaN bit pattern the kernels never write
CANARY_F32 = 0x7FC00001


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


def _rand_bf16(shape, seed, dev, dist="normal", sigma=1.0):
    return wl.bf16(shape, dist, sigma, seed, 0, dev)


def _guarded_out(M, N, dtype, dev, pad_cols=5):
    """C as an [M, N] view (row stride N + pad) inside a canary-filled buffer."""
    ldc = N + pad_cols
    if dtype == torch.bfloat16:
        big = torch.full((M + 2, ldc), CANARY_BF16, dtype=torch.int16, device=dev).view(torch.bfloat16)
    else:
        big = torch.full((M + 2, ldc), CANARY_F32, dtype=torch.int32, device=dev).view(torch.float32)
    return big, big[1:M + 1, :N]


def _guards_intact(big, M, N):
    raw = big.view(torch.int16 if big.dtype == torch.bfloat16 else torch.int32)
    canary = CANARY_BF16 if big.dtype == torch.bfloat16 else CANARY_F32
    ok = bool((raw[0] == canary).all()) and bool((raw[M + 1] == canary).all())
    ok = ok and bool((raw[1:M + 1, N:] == canary).all())
    return ok


def _tol(dtype):
    return TOL_F32 if dtype == torch.float32 else TOL_BF16


def run_and_check_bf16(a, b, bias, epi, out_dtype, algo, rows=None, label=""):
    dev = a.device
    M, K = a.shape
    N = b.shape[1]
    big, c = _guarded_out(M, N, out_dtype, dev)
    print(f"[gpu] bf16 {label} M={M} N={N} K={K} epi={epi} out={out_dtype} algo={algo}", flush=True)
    tg.gemm_bf16_ex(a, b, bias, c, epilogue=epi, algo=algo)
    torch.cuda.synchronize()
    assert _guards_intact(big, M, N), "kernel wrote outside C"
    sel = slice(None) if rows is None else torch.as_tensor(rows, device=dev)
    a_s = a[sel] if rows is not None else a
    y, d = og.gemm_bf16_bits(wl.bits_u16(a_s), wl.bits_u16(b),
                             None if bias is None else wl.bits_u16(bias), epi)
    got = (c[sel] if rows is not None else c).float().cpu().double().numpy()
    r = og.compare(got, y, d, _tol(out_dtype))
    assert r["ok"], f"{label}: {r}"
    return r


# ----------------------------------------------------------- small cases ---

@pytest.mark.parametrize("algo", [tg.ALGO_TILED, tg.ALGO_THIN])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_tiny_workload(algo, out_dtype):
    dev = _dev()
    w = wl.WORKLOADS["tiny"]
    a, b, _ = wl.bf16_inputs(w, device=dev)
    run_and_check_bf16(a, b, None, tg.EPI_NONE, out_dtype, algo, label="tiny")


@pytest.mark.parametrize("shape", [(32, 32, 32), (67, 50, 9), (67, 50, 64), (50, 67, 200)])
@pytest.mark.parametrize("fill", ["random", "ones"])
def test_self_check_shapes(shape, fill):
    dev = _dev()
    M, N, K = shape
    if fill == "ones":
        a = torch.ones(M, K, dtype=torch.bfloat16, device=dev)
        b = torch.ones(K, N, dtype=torch.bfloat16, device=dev)
    else:
        a = _rand_bf16((M, K), 11, dev)
        b = _rand_bf16((K, N), 12, dev)
    algos = [tg.ALGO_TILED] + ([tg.ALGO_THIN] if M <= 64 else [])
    for algo in algos:
        for out_dtype in (torch.float32, torch.bfloat16):
            run_and_check_bf16(a, b, None, tg.EPI_NONE, out_dtype, algo, label=f"self-check {fill}")


EDGE = [1, 2, 15, 16, 17, 31, 33, 63, 65, 67, 127, 129, 255, 257]
EDGE_CASES = [(m, n, k) for m, n, k in zip(EDGE, EDGE[::-1], EDGE[3:] + EDGE[:3])]
EDGE_CASES += [(129, 257, 64), (257, 129, 136), (256, 256, 72), (511, 300, 520), (300, 511, 8)]


@pytest.mark.parametrize("shape", EDGE_CASES)
def test_edge_sweep(shape):
    dev = _dev()
    M, N, K = shape
    a = _rand_bf16((M, K), 21, dev)
    b = _rand_bf16((K, N), 22, dev)
    bias = _rand_bf16((N,), 23, dev, sigma=0.5)
    run_and_check_bf16(a, b, bias, tg.EPI_BIAS, torch.bfloat16, tg.ALGO_TILED, label="edge")
    if M <= 64:
        run_and_check_bf16(a, b, bias, tg.EPI_BIAS, torch.float32, tg.ALGO_THIN, label="edge")


@pytest.mark.parametrize("epi", [tg.EPI_NONE, tg.EPI_BIAS, tg.EPI_BIAS_GELU_TANH])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_epilogues_and_outputs(epi, out_dtype):
    dev = _dev()
    for (M, N, K), algo in (((300, 264, 200), tg.ALGO_TILED), ((48, 1000, 520), tg.ALGO_THIN),
                            ((513, 384, 128), tg.ALGO_TILED)):
        a = _rand_bf16((M, K), 31, dev)
        b = _rand_bf16((K, N), 32, dev, sigma=0.1)
        bias = _rand_bf16((N,), 33, dev, sigma=0.5)
        run_and_check_bf16(a, b, bias if epi else None, epi, out_dtype, algo, label="epilogue")


@pytest.mark.parametrize("M", [1, 2, 8, 15, 16, 17, 31, 32, 33, 48, 63, 64])
def test_thin_and_tiled_agree_with_oracle(M):
    dev = _dev()
    a = _rand_bf16((M, 520), 41, dev)
    b = _rand_bf16((520, 1000), 42, dev, sigma=0.02)
    for algo in (tg.ALGO_THIN, tg.ALGO_TILED):
        run_and_check_bf16(a, b, None, tg.EPI_NONE, torch.bfloat16, algo, label="thin-vs-tiled")


def test_strided_and_unaligned_operands():
    dev = _dev()
    M, N, K = 200, 136, 96
    a_big = _rand_bf16((M, K + 9), 51, dev)
    b_big = _rand_bf16((K, N + 3), 52, dev)
    # strided, 16-byte aligned rows (vectorised path)
    a1 = _rand_bf16((M, K + 8), 53, dev)[:, :K]
    run_and_check_bf16(a1, b_big[:, :N].contiguous(), None, tg.EPI_NONE, torch.float32,
                       tg.ALGO_TILED, label="lda=K+8")
    # odd row strides and a base offset of one element (general path)
    a2 = a_big[:, 1:K + 1]
    b2 = b_big[:, :N]
    for algo in (tg.ALGO_TILED,):
        run_and_check_bf16(a2, b2, None, tg.EPI_NONE, torch.float32, algo, label="unaligned")
    run_and_check_bf16(a2[:40], b2, None, tg.EPI_NONE, torch.bfloat16, tg.ALGO_THIN, label="unaligned thin")


def test_tiled_weight_beyond_2gib_takes_slice_windows():
    """A [K, N] weight whose rows are 4 MiB apart (row stride 2^21
    elements): its K rows span 2.7 GB, more than one buffer window can
    address, so the tiled kernels build a window per slice instead of one
    over all of K.  Every tile shape (16 x 16 x 32 on 256 x 256, 32 x 32 x 16
    on 256 x 128 and 128 x 128) matches the oracle and, bit for bit, the
    same product with the weight packed (one window over all of K)."""
    dev = _dev()
    M, N, K, ldb = 300, 520, 640, 1 << 21
    assert (K - 1) * ldb * 2 >= 1 << 31
    a = _rand_bf16((M, K), 61, dev)
    b0 = _rand_bf16((K, N), 62, dev, sigma=0.05)
    bias = _rand_bf16((N,), 63, dev, sigma=0.5)
    bbuf = torch.empty((K - 1) * ldb + N, dtype=torch.bfloat16, device=dev)
    b = bbuf.as_strided((K, N), (ldb, 1))
    b.copy_(b0)
    for algo in (tg.ALGO_TILED_256x256, tg.ALGO_TILED_256x128, tg.ALGO_TILED_128x128):
        run_and_check_bf16(a, b, bias, tg.EPI_BIAS_GELU_TANH, torch.bfloat16, algo, label=f"ldb=2^21 algo={algo}")
        c_far = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        c_packed = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        tg.gemm_bf16_ex(a, b, bias, c_far, epilogue=tg.EPI_BIAS_GELU_TANH, algo=algo)
        tg.gemm_bf16_ex(a, b0, bias, c_packed, epilogue=tg.EPI_BIAS_GELU_TANH, algo=algo)
        torch.cuda.synchronize()
        assert torch.equal(c_far.view(torch.int16), c_packed.view(torch.int16)), algo
    del bbuf, b
    torch.cuda.empty_cache()


@pytest.mark.parametrize("algo", [tg.ALGO_TILED, tg.ALGO_THIN])
def test_k_zero_is_bias_only(algo):
    dev = _dev()
    M, N = 40, 72
    a = torch.empty(M, 0, dtype=torch.bfloat16, device=dev)
    b = torch.empty(0, N, dtype=torch.bfloat16, device=dev)
    bias = _rand_bf16((N,), 61, dev)
    run_and_check_bf16(a, b, bias, tg.EPI_BIAS_GELU_TANH, torch.float32, algo, label="K=0")
    run_and_check_bf16(a, b, None, tg.EPI_NONE, torch.bfloat16, algo, label="K=0")


def test_deterministic_bits():
    dev = _dev()
    a = _rand_bf16((1024, 1024), 71, dev)
    b = _rand_bf16((1024, 1536), 72, dev)
    c1 = torch.empty(1024, 1536, dtype=torch.bfloat16, device=dev)
    c2 = torch.empty_like(c1)
    tg.gemm_bf16(a, b, None, c1)
    tg.gemm_bf16(a, b, None, c2)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))


# ------------------------------------------------------------------ FP8 -----

def run_and_check_fp8(qa, sa, qb, sb, rows=None, label=""):
    dev = qa.device
    M, K = qa.shape
    N = qb.shape[1]
    print(f"[gpu] fp8 {label} M={M} N={N} K={K}", flush=True)
    big, c = _guarded_out(M, N, torch.bfloat16, dev, pad_cols=0)
    c = c.contiguous() if not c.is_contiguous() else c
    tg.gemm_fp8_blockscaled(qa, sa, qb, sb, c)
    torch.cuda.synchronize()
    raw = big.view(torch.int16)
    assert bool((raw[0] == CANARY_BF16).all()) and bool((raw[M + 1] == CANARY_BF16).all())
    sel = slice(None) if rows is None else torch.as_tensor(rows, device=dev)
    y, d = og.gemm_fp8_blockscaled_bits(wl.bits_u8(qa[sel]), sa[sel].cpu().numpy(), wl.bits_u8(qb),
                                        sb.cpu().numpy())
    got = c[sel].float().cpu().double().numpy()
    r = og.compare(got, y, d, TOL_FP8)
    assert r["ok"], f"{label}: {r}"
    return r


@pytest.mark.parametrize("shape", [(256, 128, 128), (300, 264, 384), (300, 260, 200),
                                   (17, 129, 136), (513, 1000, 1024), (1, 8, 16),
                                   # N % 4 != 0: the last B row's final bytes (1, 2, 3 of them)
                                   (40, 5, 128), (33, 130, 96), (70, 67, 208), (300, 323, 256),
                                   # N < 4 runs on the general kernel
                                   (19, 3, 160), (7, 1, 48), (9, 2, 16)])
def test_fp8_small_shapes(shape):
    dev = _dev()
    M, N, K = shape
    qa, sa, qb, sb = wl.fp8_inputs(wl.WORKLOADS["fp8"], device=dev, M=M, N=N, K=K)
    run_and_check_fp8(qa, sa, qb, sb, label="small")


@pytest.mark.parametrize("shape", [(300, 264, 384), (97, 131, 256)])
def test_fp8_unaligned_operands(shape):
    """A and B at odd byte offsets, C at an odd element offset: the direct
    kernel's byte-addressed loads and 2-byte stores."""
    dev = _dev()
    M, N, K = shape
    qa, sa, qb, sb = wl.fp8_inputs(wl.WORKLOADS["fp8"], device=dev, M=M, N=N, K=K)
    ra = torch.zeros(M * K + 3, dtype=torch.uint8, device=dev)
    ra[3:].copy_(qa.view(torch.uint8).reshape(-1))
    rb = torch.zeros(K * N + 1, dtype=torch.uint8, device=dev)
    rb[1:].copy_(qb.view(torch.uint8).reshape(-1))
    a_u = ra[3:].view(torch.float8_e4m3fn).view(M, K)
    b_u = rb[1:].view(torch.float8_e4m3fn).view(K, N)
    cbuf = torch.full((M * N + 2,), CANARY_BF16, dtype=torch.int16, device=dev)
    c = cbuf[1:M * N + 1].view(torch.bfloat16).view(M, N)
    print(f"[gpu] fp8 unaligned M={M} N={N} K={K}", flush=True)
    tg.gemm_fp8_blockscaled(a_u, sa, b_u, sb, c)
    torch.cuda.synchronize()
    assert int(cbuf[0]) == CANARY_BF16 and int(cbuf[M * N + 1]) == CANARY_BF16
    y, d = og.gemm_fp8_blockscaled_bits(wl.bits_u8(qa), sa.cpu().numpy(), wl.bits_u8(qb),
                                        sb.cpu().numpy())
    r = og.compare(c.float().cpu().double().numpy(), y, d, TOL_FP8)
    assert r["ok"], r


def test_fp8_integer_codes_exact():
    dev = _dev()
    M, N, K = 64, 128, 256
    g = torch.Generator(device=dev).manual_seed(81)
    ia = torch.randint(-4, 5, (M, K), generator=g, device=dev).float()
    ib = torch.randint(-4, 5, (K, N), generator=g, device=dev).float()
    qa, qb = ia.to(torch.float8_e4m3fn), ib.to(torch.float8_e4m3fn)
    sa = torch.ones(M, 2, device=dev)
    sb = torch.ones(2, 1, device=dev)
    c = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    tg.gemm_fp8_blockscaled(qa, sa, qb, sb, c)
    torch.cuda.synchronize()
    exact = (ia.double() @ ib.double()).cpu()
    # integers up to |256 * 16| = 4096 are exact in bf16 only up to 256; compare rounded
    assert torch.equal(c.cpu().float(), exact.float().to(torch.bfloat16).float())


def test_fp8_wide_weight_takes_slice_windows():
    """A [K, N] FP8 weight of 1.9 GB (K = 2048, N = 917504): its per-lane
    offsets over all of K pass 2^31, so the kernel builds windows per slice
    instead of one over all of K.  The weight repeats one random 1024-column
    block (and its scales) 896 times, so every 1024-column block of the
    output must equal, bit for bit, the product with that one block -- which
    takes the whole-K windows and is checked against the oracle."""
    dev = _dev()
    M, K, n_small, reps = 256, 2048, 1024, 896
    N = n_small * reps
    assert (K + 384) * N >= 1 << 31
    qa, sa, qb, sb = wl.fp8_inputs(wl.WORKLOADS["fp8"], device=dev, M=M, N=n_small, K=K)
    c_small = torch.empty(M, n_small, dtype=torch.bfloat16, device=dev)
    tg.gemm_fp8_blockscaled(qa, sa, qb, sb, c_small)
    torch.cuda.synchronize()
    y, d = og.gemm_fp8_blockscaled_bits(wl.bits_u8(qa), sa.cpu().numpy(), wl.bits_u8(qb), sb.cpu().numpy())
    assert og.compare(c_small.float().cpu().double().numpy(), y, d, TOL_FP8)["ok"]
    qb_big = qb.view(torch.uint8).repeat(1, reps).view(torch.float8_e4m3fn)
    sb_big = sb.repeat(1, reps).contiguous()
    c_big = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    print(f"[gpu] fp8 wide weight M={M} N={N} K={K}", flush=True)
    tg.gemm_fp8_blockscaled(qa, sa, qb_big, sb_big, c_big)
    torch.cuda.synchronize()
    blocks = c_big.view(torch.int16).view(M, reps, n_small)
    assert bool((blocks == c_small.view(torch.int16).unsqueeze(1)).all())
    del qb_big, c_big, blocks
    torch.cuda.empty_cache()


# ------------------------------------------------------- full workloads ----

def _tile_rows(M, tile=256, block=32, seed=93):
    """Both edge rows of every output tile, plus one seeded random row in
    every 32-row block (the row extent of one MFMA accumulator block), so
    every block of every wave tile is sampled."""
    rng = np.random.default_rng(seed)
    rows = set()
    for t0 in range(0, M, tile):
        rows.update({t0, min(M - 1, t0 + tile - 1)})
    for b0 in range(0, M, block):
        rows.add(int(rng.integers(b0, min(M, b0 + block))))
    return sorted(rows)


@pytest.mark.parametrize("name", ["square", "ffn_up", "ffn_down"])
def test_full_size_bf16_workloads(name):
    dev = _dev()
    w = wl.WORKLOADS[name]
    if name == "ffn_down":
        a = wl.ffn_hidden(w.M, w.K, w.seed, dev)
        _, b, bias = wl.bf16_inputs(w, device=dev)
    else:
        a, b, bias = wl.bf16_inputs(w, device=dev)
    run_and_check_bf16(a, b, bias, w.epilogue, torch.bfloat16, tg.ALGO_AUTO,
                       rows=_tile_rows(w.M), label=name)


def test_full_size_thin_workloads():
    dev = _dev()
    w = wl.WORKLOADS["thin_m64"]
    x, W, _ = wl.bf16_inputs(w, device=dev)
    g = torch.Generator().manual_seed(91)
    cols = torch.cat([torch.arange(0, 256), torch.randint(256, w.N - 256, (1536,), generator=g),
                      torch.arange(w.N - 256, w.N)]).to(dev)
    Wc = W[:, cols].contiguous()
    Wbits = wl.bits_u16(Wc)
    for M in (1, 8, 32, 64):
        xm = x[:M].contiguous()
        big, c = _guarded_out(M, w.N, torch.bfloat16, dev)
        print(f"[gpu] thin M={M} N={w.N} K={w.K}", flush=True)
        tg.gemm_bf16(xm, W, None, c)
        torch.cuda.synchronize()
        assert _guards_intact(big, M, w.N)
        y, d = og.gemm_bf16_bits(wl.bits_u16(xm), Wbits)
        r = og.compare(c[:, cols].float().cpu().double().numpy(), y, d, TOL_BF16)
        assert r["ok"], f"thin M={M}: {r}"


@pytest.mark.parametrize("name", ["fp8", "fp8_ragged"])
def test_full_size_fp8_workloads(name):
    dev = _dev()
    w = wl.WORKLOADS[name]
    qa, sa, qb, sb = wl.fp8_inputs(w, device=dev)
    run_and_check_fp8(qa, sa, qb, sb, rows=_tile_rows(w.M), label=name)
