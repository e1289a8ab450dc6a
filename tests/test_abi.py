"""The C ABI library on the host: it loads, exports what include/tgemm.h
declares, and rejects bad arguments before any HIP call (no GPU needed:
every call here returns during validation, so nothing is enqueued).
"""

import ctypes
import os
import subprocess

import pytest

from tiled_gemm_04_amd import binding

pytestmark = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH),
                                reason="libtgemm.so not built (python -m tiled_gemm_04_amd.build)")

INV, UNS, OK = binding.TGEMM_ERR_INVALID, binding.TGEMM_ERR_UNSUPPORTED, binding.TGEMM_OK
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails or M/N is 0 first
NULL = ctypes.c_void_p(0)


def test_every_declared_function_is_exported():
    names = binding.header_functions()
    assert {"gemm_bf16", "gemm_fp8_blockscaled", "gemm_bf16_ex", "quantize_fp8_1x128",
            "quantize_fp8_128x128", "gemm_bf16_w8", "gemm_w8_kernel_name", "gemm_bf16_w4",
            "gemm_w4_kernel_name", "gemm_bf16_logsoftmax", "gemm_logsoftmax_workspace_size"} <= set(names)
    L = binding.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported


def test_version_and_status_strings():
    assert binding.gemm_abi_version() == 2
    assert binding.gemm_status_string(0) == "ok"
    assert "invalid" in binding.gemm_status_string(INV)
    assert binding.gemm_status_string(99) == "unknown status"


def _bf16(A=FAKE, B=FAKE, bias=FAKE, C=FAKE, M=64, N=64, K=64, lda=64, ldb=64, ldc=64, epi=0,
          out=1, algo=None):
    L = binding.lib()
    if algo is None:
        return L.gemm_bf16(A, B, bias, C, M, N, K, lda, ldb, ldc, epi, out, NULL)
    return L.gemm_bf16_ex(A, B, bias, C, M, N, K, lda, ldb, ldc, epi, out, algo, NULL, 0, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), INV), (dict(N=-5), INV), (dict(K=-1), INV),
    (dict(M=1 << 31, lda=64), INV),
    (dict(C=NULL), INV), (dict(A=NULL), INV), (dict(B=NULL), INV),
    (dict(epi=3), INV), (dict(epi=-1), INV), (dict(out=2), INV),
    (dict(epi=1, bias=NULL), INV), (dict(epi=2, bias=NULL), INV),
    (dict(lda=63), INV), (dict(ldb=10), INV), (dict(ldc=0), INV),
    (dict(algo=6), INV), (dict(algo=2, M=65), UNS),
    (dict(M=0), OK), (dict(N=0, ldb=1, ldc=1), OK), (dict(M=0, A=NULL, C=NULL), OK),
])
def test_bf16_validation(kw, status):
    assert _bf16(**kw) == status


def test_bf16_k_zero_needs_no_operands_but_needs_c():
    # K == 0 with NULL A/B is valid (empty sum); C must still be given.
    assert _bf16(A=NULL, B=NULL, C=NULL, K=0, lda=1) == INV


def test_fp8_validation():
    L = binding.lib()
    f = ctypes.c_void_p
    assert L.gemm_fp8_blockscaled(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 4, 4, NULL) == INV
    assert L.gemm_fp8_blockscaled(FAKE, NULL, FAKE, FAKE, FAKE, 4, 4, 4, NULL) == INV
    assert L.gemm_fp8_blockscaled(FAKE, FAKE, FAKE, NULL, FAKE, 4, 4, 4, NULL) == INV
    assert L.gemm_fp8_blockscaled(FAKE, FAKE, FAKE, FAKE, NULL, 4, 4, 4, NULL) == INV
    assert L.gemm_fp8_blockscaled(NULL, NULL, NULL, NULL, NULL, 0, 4, 4, NULL) == OK
    del f


def _w8(X=FAKE, Q=FAKE, S=FAKE, bias=FAKE, C=FAKE, M=8, N=64, K=64, ldx=64, ldq=64, ldc=64, epi=0,
        out=1, fn="gemm_bf16_w8"):
    return getattr(binding.lib(), fn)(X, Q, S, bias, C, M, N, K, ldx, ldq, ldc, epi, out, NULL, 0, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), INV), (dict(K=-1), INV), (dict(C=NULL), INV), (dict(X=NULL), INV),
    (dict(Q=NULL), INV), (dict(S=NULL), INV), (dict(epi=1, bias=NULL), INV), (dict(out=2), INV),
    (dict(ldx=63), INV), (dict(ldq=10), INV),
    (dict(M=65), UNS), (dict(N=66, ldq=66, ldc=66), UNS), (dict(K=60, ldx=64), UNS),
    (dict(ldq=66), UNS),
    (dict(M=0), OK), (dict(N=0, ldq=1, ldc=1), OK),
])
@pytest.mark.parametrize("fn", ["gemm_bf16_w8", "gemm_bf16_w4"])
def test_w8_validation(kw, status, fn):
    assert _w8(fn=fn, **kw) == status


def test_w8_kernel_names():
    # narrow weights: the split pair only when a workspace is given
    assert binding.gemm_w8_kernel_name(8, 14336, 4096) == "tgemm_w8_thin_m16"
    assert binding.gemm_w8_kernel_name(8, 14336, 4096, with_workspace=True) == \
        "tgemm_w8_thin_splitk_m16+tgemm_splitk_reduce"
    assert binding.gemm_w4_kernel_name(40, 4096, 4096, with_workspace=True) == \
        "tgemm_w4_thin_splitk_m48+tgemm_splitk_reduce"
    assert binding.gemm_w8_kernel_name(1, 128256, 4096, with_workspace=True) == "tgemm_w8_thin_m16"
    assert binding.gemm_w8_kernel_name(1, 128256, 4096) == "tgemm_w8_thin_m16"
    assert binding.gemm_w8_kernel_name(64, 128256, 4096) == "tgemm_w8_thin_m64"
    assert binding.gemm_w8_kernel_name(65, 128256, 4096) is None
    assert binding.gemm_w8_kernel_name(8, 130, 4096) is None
    assert binding.gemm_w4_kernel_name(1, 128256, 4096) == "tgemm_w4_thin_m16"
    assert binding.gemm_w4_kernel_name(33, 128256, 4096) == "tgemm_w4_thin_m48"
    assert binding.gemm_w4_kernel_name(64, 128256, 4096) == "tgemm_w4_thin_m64"
    assert binding.gemm_w4_kernel_name(65, 128256, 4096) is None
    assert binding.gemm_w4_kernel_name(8, 128256, 4092) is None


@pytest.mark.parametrize("fn", ["quantize_fp8_1x128", "quantize_fp8_128x128"])
def test_quantize_validation(fn):
    q = getattr(binding.lib(), fn)
    assert q(FAKE, FAKE, FAKE, -1, 8, 8, NULL) == INV
    assert q(FAKE, FAKE, FAKE, 8, -1, 8, NULL) == INV
    assert q(FAKE, FAKE, FAKE, 1 << 31, 8, 8, NULL) == INV
    assert q(NULL, FAKE, FAKE, 8, 8, 8, NULL) == INV
    assert q(FAKE, NULL, FAKE, 8, 8, 8, NULL) == INV
    assert q(FAKE, FAKE, NULL, 8, 8, 8, NULL) == INV
    assert q(FAKE, FAKE, FAKE, 8, 8, 7, NULL) == INV  # row stride below the row length
    assert q(NULL, NULL, NULL, 0, 8, 8, NULL) == OK
    assert q(NULL, NULL, NULL, 8, 0, 8, NULL) == OK


def test_kernel_selection_table():
    name = binding.gemm_bf16_kernel_name
    assert name(4096, 4096, 4096) == "tgemm_bf16_tiled_256x256x32"
    assert name(2048, 16384, 4096) == "tgemm_bf16_tiled_256x256x32"
    assert name(2048, 4096, 16384) == "tgemm_bf16_tiled_256x128x64"
    assert name(64, 128256, 4096) == "tgemm_bf16_thin_m64"
    assert name(1, 128256, 4096) == "tgemm_bf16_thin_m16"
    assert name(1, 128256, 4096, with_workspace=True) == "tgemm_bf16_thin_m16"
    assert name(8, 4096, 4096) == "tgemm_bf16_thin_m16"
    assert name(8, 4096, 4096, with_workspace=True) == "tgemm_bf16_thin_splitk_m16+tgemm_splitk_reduce"
    assert name(64, 4096, 4096, with_workspace=True) == "tgemm_bf16_thin_splitk_m64+tgemm_splitk_reduce"
    assert name(64, 64, 64, algo=binding.ALGO_TILED).startswith("tgemm_bf16_tiled")
    assert name(65, 64, 64, algo=binding.ALGO_THIN) is None
    assert name(-1, 64, 64) is None
    assert name(4096, 4096, 4096, algo=binding.ALGO_TILED_128x128) == "tgemm_bf16_tiled_128x128x64"
    assert name(4096, 4096, 4096, algo=binding.ALGO_TILED_256x128) == "tgemm_bf16_tiled_256x128x64"
    assert name(64, 64, 64, algo=binding.ALGO_TILED_256x256) == "tgemm_bf16_tiled_256x256x32"
    assert binding.gemm_fp8_kernel_name(4096, 14336, 4096) == "tgemm_fp8_bs_256x256x128"
    assert binding.gemm_fp8_kernel_name(4097, 14335, 4096) == "tgemm_fp8_bs_256x256x128"
    assert binding.gemm_fp8_kernel_name(64, 64, 200).startswith("tgemm_fp8_bs_general")
    assert binding.gemm_fp8_kernel_name(64, 3, 256).startswith("tgemm_fp8_bs_general")


def test_logsoftmax_workspace_size_and_validation():
    L = binding.lib()
    assert L.gemm_logsoftmax_workspace_size(1, 128256, binding.OUT_F32) == 2048  # 251 * 8, to 256
    assert L.gemm_logsoftmax_workspace_size(1, 128256, binding.OUT_BF16) == 2048 + 128256 * 4
    assert L.gemm_logsoftmax_workspace_size(64, 512, binding.OUT_F32) == 512
    assert L.gemm_logsoftmax_workspace_size(-1, 8, binding.OUT_F32) == -1
    assert L.gemm_logsoftmax_workspace_size(1, 8, 7) == -1
    ws = 256 + 4 * 512 * 4

    def call(X=FAKE, W=FAKE, bias=NULL, C=FAKE, M=4, N=512, K=64, ldx=64, ldw=512, ldc=512, out=1,
             work=FAKE, work_bytes=ws):
        return L.gemm_bf16_logsoftmax(X, W, bias, C, M, N, K, ldx, ldw, ldc, out, work, work_bytes, NULL)

    assert call(M=0) == OK
    assert call(N=0, ldw=1, ldc=1) == INV              # empty distribution
    assert call(M=-1) == INV
    assert call(out=2) == INV
    assert call(C=NULL) == INV
    assert call(X=NULL) == INV
    assert call(work=NULL) == INV
    assert call(work_bytes=256 + 4 * 512 * 4 - 1) == INV
    assert call(out=0, work_bytes=255) == INV
    assert call(ldx=63) == INV


def test_nt_validation():
    L = binding.lib()

    def call(A=FAKE, B=FAKE, bias=FAKE, C=FAKE, M=64, N=64, K=64, lda=64, ldb=64, ldc=64, epi=0, out=1):
        return L.gemm_bf16_nt(A, B, bias, C, M, N, K, lda, ldb, ldc, epi, out, NULL)

    assert call(ldb=63) == INV                  # ldb < K for a [N, K] weight
    assert call(K=60, lda=64, ldb=64) == UNS   # K % 8
    assert call(lda=66) == UNS                 # lda % 8
    assert call(M=0) == OK and call(N=0, ldc=1) == OK
    assert call(C=NULL) == INV and call(B=NULL) == INV
    assert call(epi=1, bias=NULL) == INV
    assert binding.gemm_bf16_nt_kernel_name(4096, 4096, 4096) == "tgemm_bf16_tiled_bt_256x256x32"
    assert binding.gemm_bf16_nt_kernel_name(2048, 4096, 16384) == "tgemm_bf16_tiled_bt_256x128x64"
    assert binding.gemm_bf16_nt_kernel_name(64, 64, 60) is None
    assert binding.gemm_bf16_nt_kernel_name(1, 128256, 4096) == "tgemm_bf16_thin_nt_m16"
    assert binding.gemm_bf16_nt_kernel_name(64, 128256, 4096) == "tgemm_bf16_thin_nt_m64"
    assert binding.gemm_bf16_nt_kernel_name(65, 128256, 4096).startswith("tgemm_bf16_tiled_bt")


def test_strided_batched_validation():
    L = binding.lib()

    def call(A=FAKE, B=FAKE, bias=NULL, C=FAKE, M=64, N=64, K=64, lda=64, ldb=64, ldc=64, sa=4096,
             sb=4096, sc=4096, batch=3, layout=0, epi=0, out=1):
        return L.gemm_bf16_strided_batched(A, B, bias, C, M, N, K, lda, ldb, ldc, sa, sb, sc, batch,
                                           layout, epi, out, NULL)

    assert call(batch=-1) == INV
    assert call(sa=-1) == INV and call(sb=-8) == INV and call(sc=-8) == INV
    assert call(layout=2) == INV
    assert call(sc=64 * 63) == INV                     # outputs of problems 0 and 1 overlap
    assert call(batch=0) == OK and call(M=0) == OK
    assert call(batch=70000) == UNS
    assert call(layout=1, K=60, lda=64, ldb=64) == UNS  # [N, K] weights need K % 8 == 0
    assert call(C=NULL) == INV
    assert call(sa=1 << 61, batch=8) == INV            # whole-batch extent overflows


def test_fp8_ex_validation():
    L = binding.lib()
    for parts in (-1, 9):
        assert L.gemm_fp8_blockscaled_ex(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 4, parts, NULL, 0, NULL) == INV
    assert L.gemm_fp8_blockscaled_ex(NULL, NULL, NULL, NULL, NULL, 0, 4, 4, 2, NULL, 0, NULL) == OK
    assert L.gemm_fp8_blockscaled_ex(FAKE, NULL, FAKE, FAKE, FAKE, 4, 4, 4, 2, NULL, 0, NULL) == INV
    assert L.gemm_fp8_workspace_size(-1, 4, 4, 0) == -1
    assert L.gemm_fp8_workspace_size(4, 4, 4, 9) == -1
    assert L.gemm_fp8_workspace_size(0, 4, 4, 0) == 0


def test_workspace_sizes_and_validation():
    """Size queries (host only) and the rejection of a short or unaligned
    workspace before anything is enqueued."""
    L = binding.lib()
    # M = 8, N = K = 4096: 8 stripes; S = min(256/8, KT/4 = 32, K/(8M) = 64) = 32 chunks
    assert L.gemm_bf16_workspace_size(8, 4096, 4096, 0) == 32 * 8 * 4096 * 4
    assert L.gemm_bf16_workspace_size(8, 128256, 4096, 0) == 0      # 251 stripes: no split
    assert L.gemm_bf16_workspace_size(65, 4096, 4096, 0) == 0       # tiled kernel
    assert L.gemm_bf16_workspace_size(8, 4096, 4096, binding.ALGO_TILED) == 0
    assert L.gemm_bf16_workspace_size(-1, 4096, 4096, 0) == -1
    assert L.gemm_bf16_workspace_size(8, 4096, 4096, 9) == -1
    assert L.gemm_wq_workspace_size(-1, 4, 4) == -1
    assert L.gemm_wq_workspace_size(8, 128256, 4096) == 0
    need = L.gemm_bf16_workspace_size(8, 4096, 4096, 0)

    def call(ws, nbytes):
        return L.gemm_bf16_ex(FAKE, FAKE, NULL, FAKE, 8, 4096, 4096, 4096, 4096, 4096, 0, 1, 0, ws, nbytes, NULL)

    assert call(FAKE, need - 1) == INV
    assert call(ctypes.c_void_p(0x1008), need) == INV     # not 16-byte aligned
    wq = L.gemm_wq_workspace_size(8, 4096, 4096)
    assert wq > 0 and wq % 256 == 0
    assert L.gemm_bf16_w8(FAKE, FAKE, FAKE, NULL, FAKE, 8, 4096, 4096, 4096, 4096, 4096, 0, 1, FAKE, wq - 1,
                          NULL) == INV


def _tiles(M, N):
    return -(-M // 256) * -(-N // 256)


@pytest.mark.parametrize("M,N,K,cus,want", [
    # 896 tiles on 256 units: 3 full rounds + 128 tiles -> no split
    (4096, 14336, 4096, 256, (896, 0, 1)),
    (4097, 14335, 4096, 256, (952, 0, 1)),
    (8192, 8192, 4096, 256, (1024, 0, 1)),
    # one tile, 32 groups: four ranges of eight groups
    (256, 256, 4096, 256, (0, 1, 4)),
    # one tile, 128 groups: eight ranges (cap)
    (256, 256, 16384, 256, (0, 1, 8)),
    # fewer than 16 groups: no split
    (256, 256, 1920, 256, (1, 0, 1)),
    (256, 256, 256, 256, (1, 0, 1)),
    # 9 tiles, 16 groups: two ranges
    (600, 700, 2048, 256, (0, 9, 2)),
    # 64 tiles = a quarter of the units: 256 / 64 = 4 ranges
    (2048, 2048, 4096, 256, (0, 64, 4)),
    # 65 or more tiles: no split
    (16640, 256, 4096, 256, (65, 0, 1)),
    (4096, 2048, 4096, 256, (128, 0, 1)),
    (2560, 2560, 4096, 256, (100, 0, 1)),
    # unknown compute-unit count -> no split
    (256, 256, 4096, 0, (1, 0, 1)),
    # the general kernel (K not a multiple of 16) never splits
    (256, 256, 4100, 256, (1, 0, 1)),
])
def test_fp8_split_plan_automatic(M, N, K, cus, want):
    got = binding.gemm_fp8_split_plan(M, N, K, cus)
    assert got == want
    whole, split, parts = got
    assert whole + split == _tiles(M, N)
    if parts > 1:
        # the split tiles fit one round of workgroups, each range >= 8 groups
        assert whole == 0 and split * parts <= cus and parts * 8 <= -(-K // 128)


@pytest.mark.parametrize("forced,K,want_parts", [(1, 4096, 1), (2, 4096, 2), (8, 4096, 8),
                                                 (5, 384, 3), (3, 384, 3), (2, 128, 1)])
def test_fp8_split_plan_forced(forced, K, want_parts):
    whole, split, parts = binding.gemm_fp8_split_plan(600, 700, K, 256, forced)
    assert parts == want_parts
    assert whole + split == _tiles(600, 700)
    assert (split == 0) == (parts == 1)


def test_fp8_split_plan_forced_multi_round():
    # a forced split takes the last round of a longer grid
    assert binding.gemm_fp8_split_plan(4096, 14336, 4096, 256, 2) == (768, 128, 2)
    assert binding.gemm_fp8_split_plan(4097, 14335, 4096, 256, 3) == (768, 184, 3)


def test_fp8_split_plan_validation():
    L = binding.lib()
    i = ctypes.c_int32()
    p = ctypes.byref(i)
    assert L.gemm_fp8_split_plan(-1, 4, 4, 256, 0, p, p, p) == INV
    assert L.gemm_fp8_split_plan(4, 4, 4, -1, 0, p, p, p) == INV
    assert L.gemm_fp8_split_plan(4, 4, 4, 256, 9, p, p, p) == INV
    assert L.gemm_fp8_split_plan(4, 4, 4, 256, 0, None, p, p) == INV


def test_bf16_quant_fp8_validation():
    L = binding.lib()
    S = ctypes.c_void_p(0x2000)
    # M, N, K, lda, ldb, epilogue, algo
    assert L.gemm_bf16_quant_fp8(FAKE, FAKE, NULL, FAKE, S, -1, 8, 8, 8, 8, 0, 0, NULL) == INV
    assert L.gemm_bf16_quant_fp8(FAKE, FAKE, NULL, FAKE, S, 8, 8, 8, 4, 8, 0, 0, NULL) == INV   # lda < K
    assert L.gemm_bf16_quant_fp8(FAKE, FAKE, NULL, FAKE, S, 8, 8, 8, 8, 8, 1, 0, NULL) == INV   # bias missing
    assert L.gemm_bf16_quant_fp8(FAKE, FAKE, NULL, FAKE, S, 8, 8, 8, 8, 8, 3, 0, NULL) == INV   # epilogue
    assert L.gemm_bf16_quant_fp8(FAKE, FAKE, NULL, NULL, S, 8, 8, 8, 8, 8, 0, 0, NULL) == INV   # Q
    assert L.gemm_bf16_quant_fp8(FAKE, FAKE, NULL, FAKE, NULL, 8, 8, 8, 8, 8, 0, 0, NULL) == INV  # S
    assert L.gemm_bf16_quant_fp8(FAKE, FAKE, NULL, FAKE, S, 8, 8, 8, 8, 8, 0, 9, NULL) == INV   # algo
    assert L.gemm_bf16_quant_fp8(FAKE, FAKE, NULL, FAKE, S, 8, 8, 8, 8, 8, 0, 2, NULL) == UNS   # thin
    assert L.gemm_bf16_quant_fp8(FAKE, FAKE, NULL, FAKE, S, 8, 12, 8, 8, 12, 0, 0, NULL) == UNS  # N % 8
    assert L.gemm_bf16_quant_fp8(FAKE, FAKE, NULL, FAKE, S, 8, 8, 12, 12, 8, 0, 0, NULL) == UNS  # K % 8
    assert L.gemm_bf16_quant_fp8(ctypes.c_void_p(0x1002), FAKE, NULL, FAKE, S, 8, 8, 8, 8, 8, 0, 0, NULL) == UNS
    assert L.gemm_bf16_quant_fp8(NULL, NULL, NULL, NULL, NULL, 0, 8, 8, 8, 8, 0, 0, NULL) == OK


def test_fp8_nt_validation():
    L = binding.lib()
    assert L.gemm_fp8_blockscaled_nt(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 4, 16, NULL) == INV
    assert L.gemm_fp8_blockscaled_nt(FAKE, NULL, FAKE, FAKE, FAKE, 4, 4, 16, NULL) == INV
    assert L.gemm_fp8_blockscaled_nt(FAKE, FAKE, FAKE, FAKE, NULL, 4, 4, 16, NULL) == INV
    assert L.gemm_fp8_blockscaled_nt(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 24, NULL) == UNS  # K % 16
    assert L.gemm_fp8_blockscaled_nt(NULL, NULL, NULL, NULL, NULL, 0, 4, 16, NULL) == OK


def test_wq_logsoftmax_validation():
    L = binding.lib()
    WS = ctypes.c_void_p(0x3000)
    for f in (L.gemm_bf16_w8_logsoftmax, L.gemm_bf16_w4_logsoftmax):
        # X, Q, S, bias, C, M, N, K, ldx, ldq, ldc, out, ws, ws_bytes
        assert f(FAKE, FAKE, FAKE, NULL, FAKE, 2, 0, 64, 64, 0, 0, 1, WS, 1 << 20, NULL) == INV  # N == 0
        assert f(FAKE, FAKE, FAKE, NULL, FAKE, 2, 512, 64, 64, 512, 512, 1, NULL, 1 << 20, NULL) == INV
        assert f(FAKE, FAKE, FAKE, NULL, FAKE, 2, 512, 64, 64, 512, 512, 1, WS, 16, NULL) == INV  # short
        assert f(FAKE, FAKE, NULL, NULL, FAKE, 2, 512, 64, 64, 512, 512, 1, WS, 1 << 20, NULL) == INV  # S
        assert f(FAKE, FAKE, FAKE, NULL, FAKE, 65, 512, 64, 64, 512, 512, 1, WS, 1 << 24, NULL) == UNS  # M
        assert f(FAKE, FAKE, FAKE, NULL, FAKE, 2, 510, 64, 64, 512, 512, 1, WS, 1 << 20, NULL) == UNS  # N % 4
        assert f(NULL, NULL, NULL, NULL, NULL, 0, 512, 64, 64, 512, 512, 1, NULL, 0, NULL) == OK


def test_probe_validation():
    L = binding.lib()
    out = ctypes.c_void_p(0x4000)
    assert L.gemm_probe_mfma(5, 10, out, 1 << 20, 1, NULL) == INV      # unknown probe
    assert L.gemm_probe_mfma(0, -1, out, 1 << 20, 1, NULL) == INV      # negative iters
    assert L.gemm_probe_mfma(0, 1 << 40, out, 1 << 20, 1, NULL) == INV  # oversized iters
    assert L.gemm_probe_mfma(1, 10, NULL, 1 << 20, 1, NULL) == INV     # no output
    assert L.gemm_probe_stream_read(FAKE, 24, out, 1 << 20, NULL) == INV             # bytes % 16
    assert L.gemm_probe_stream_read(ctypes.c_void_p(0x1008), 32, out, 1 << 20, NULL) == INV  # unaligned
    assert L.gemm_probe_stream_read(NULL, 32, out, 1 << 20, NULL) == INV
    assert L.gemm_probe_out_elems(7) == -1
    assert L.gemm_probe_mfma_flop(7, 10) < 0
