"""ctypes binding of libtgemm.so (argument marshalling only).

The functions here carry the C ABI's names.  Each takes torch tensors that
already live on the GPU, checks dtype / device / layout, derives sizes and
row strides, passes raw device pointers and the current HIP stream to the
library, and raises on a non-zero status.  No arithmetic of the GEMM happens
here; torch is used only for device memory and streams.

If libtgemm.so has not been built, every call raises -- there is no fallback.
"""

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtgemm.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "tgemm.h")

TGEMM_OK = 0
TGEMM_ERR_INVALID = 1
TGEMM_ERR_UNSUPPORTED = 2
TGEMM_ERR_LAUNCH = 3
TGEMM_ERR_SCRATCH = 4
NOALLOC_SCRATCH_BYTES = 32 << 20  # TGEMM_NOALLOC_SCRATCH_BYTES

EPI_NONE = 0
EPI_BIAS = 1
EPI_BIAS_GELU_TANH = 2

OUT_F32 = 0
OUT_BF16 = 1

B_KN = 0  # B [K, N]
B_NK = 1  # B [N, K]

ALGO_AUTO = 0
ALGO_TILED = 1
ALGO_THIN = 2
ALGO_TILED_256x256 = 3
ALGO_TILED_256x128 = 4
ALGO_TILED_128x128 = 5

_lib = None


class TgemmError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = lib().gemm_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{where}: status {status} ({msg})")


def lib():
    """Load libtgemm.so once; raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m tiled_gemm_04_amd.build` "
            "(the HIP library is required; there is no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.gemm_bf16.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, i32, vp]
    L.gemm_bf16.restype = i32
    L.gemm_bf16_ex.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, i32, i32, vp, i64, vp]
    L.gemm_bf16_ex.restype = i32
    L.gemm_bf16_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, i32, i32, vp]
    L.gemm_bf16_noalloc.restype = i32
    L.gemm_bf16_workspace_size.argtypes = [i64, i64, i64, i32]
    L.gemm_bf16_workspace_size.restype = i64
    L.gemm_fp8_workspace_size.argtypes = [i64, i64, i64, i32]
    L.gemm_fp8_workspace_size.restype = i64
    L.gemm_wq_workspace_size.argtypes = [i64, i64, i64]
    L.gemm_wq_workspace_size.restype = i64
    L.gemm_fp8_blockscaled.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp]
    L.gemm_fp8_blockscaled.restype = i32
    L.gemm_fp8_blockscaled_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, i64, vp]
    L.gemm_fp8_blockscaled_ex.restype = i32
    L.gemm_fp8_split_plan.argtypes = [i64, i64, i64, i32, i32, ctypes.POINTER(i32),
                                      ctypes.POINTER(i32), ctypes.POINTER(i32)]
    L.gemm_fp8_split_plan.restype = i32
    for f in ("gemm_bf16_w8_logsoftmax", "gemm_bf16_w4_logsoftmax"):
        getattr(L, f).argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, vp, i64, vp]
        getattr(L, f).restype = i32
    L.gemm_probe_out_elems.argtypes = [i32]
    L.gemm_probe_out_elems.restype = i64
    L.gemm_probe_mfma_flop.argtypes = [i32, i64]
    L.gemm_probe_mfma_flop.restype = ctypes.c_double
    L.gemm_probe_mfma.argtypes = [i32, i64, vp, i64, ctypes.c_uint64, vp]
    L.gemm_probe_mfma.restype = i32
    L.gemm_probe_stream_read.argtypes = [vp, i64, vp, i64, vp]
    L.gemm_probe_stream_read.restype = i32
    L.gemm_fp8_blockscaled_nt.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp]
    L.gemm_fp8_blockscaled_nt.restype = i32
    L.gemm_bf16_quant_fp8.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, i32, vp]
    L.gemm_bf16_quant_fp8.restype = i32
    L.gemm_bf16_w8.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, i32, vp, i64, vp]
    L.gemm_bf16_w8.restype = i32
    L.gemm_w8_kernel_name.argtypes = [i64, i64, i64, i32]
    L.gemm_w8_kernel_name.restype = ctypes.c_char_p
    L.gemm_bf16_strided_batched.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, i64,
                                            i64, i32, i32, i32, vp]
    L.gemm_bf16_strided_batched.restype = i32
    L.gemm_bf16_nt.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, i32, vp]
    L.gemm_bf16_nt.restype = i32
    L.gemm_bf16_nt_kernel_name.argtypes = [i64, i64, i64]
    L.gemm_bf16_nt_kernel_name.restype = ctypes.c_char_p
    L.gemm_bf16_logsoftmax.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, vp, i64, vp]
    L.gemm_bf16_logsoftmax.restype = i32
    L.gemm_logsoftmax_workspace_size.argtypes = [i64, i64, i32]
    L.gemm_logsoftmax_workspace_size.restype = i64
    L.gemm_bf16_w4.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, i32, vp, i64, vp]
    L.gemm_bf16_w4.restype = i32
    L.gemm_w4_kernel_name.argtypes = [i64, i64, i64, i32]
    L.gemm_w4_kernel_name.restype = ctypes.c_char_p
    L.quantize_fp8_1x128.argtypes = [vp, vp, vp, i64, i64, i64, vp]
    L.quantize_fp8_1x128.restype = i32
    L.quantize_fp8_128x128.argtypes = [vp, vp, vp, i64, i64, i64, vp]
    L.quantize_fp8_128x128.restype = i32
    L.gemm_bf16_kernel_name.argtypes = [i64, i64, i64, i32, i32, i32, i32]
    L.gemm_bf16_kernel_name.restype = ctypes.c_char_p
    L.gemm_fp8_kernel_name.argtypes = [i64, i64, i64]
    L.gemm_fp8_kernel_name.restype = ctypes.c_char_p
    L.gemm_status_string.argtypes = [i32]
    L.gemm_status_string.restype = ctypes.c_char_p
    L.gemm_abi_version.argtypes = []
    L.gemm_abi_version.restype = i32
    _lib = L
    return L


def header_functions():
    """Names of the functions include/tgemm.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:gemm|quantize)_\w+)\s*\(", text)))


def _stream_ptr(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _row_major(t, name):
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.stride(1) != 1 and t.shape[1] > 1:
        raise ValueError(f"{name} must have unit inner stride")
    return max(t.stride(0), t.shape[1], 1)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else ctypes.c_void_p(0)


def _check_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on the GPU")


def _workspace(ws):
    """(pointer, bytes) of an optional workspace tensor (None: NULL, 0)."""
    if ws is None:
        return ctypes.c_void_p(0), 0
    _check_cuda(ws)
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return _ptr(ws), ws.numel() * ws.element_size()


def gemm_bf16_workspace_size(M, N, K, algo=ALGO_AUTO):
    """Bytes of workspace gemm_bf16_ex needs to split this problem (0: none)."""
    return int(lib().gemm_bf16_workspace_size(M, N, K, int(algo)))


def gemm_fp8_workspace_size(M, N, K, split_parts=0):
    """Bytes of workspace gemm_fp8_blockscaled_ex needs on the current device
    (0: it would not split).  Allocate it zero-filled (arrival counters)."""
    return int(lib().gemm_fp8_workspace_size(M, N, K, int(split_parts)))


def gemm_wq_workspace_size(M, N, K):
    """Bytes of workspace gemm_bf16_w8 / gemm_bf16_w4 need to split (0: none)."""
    return int(lib().gemm_wq_workspace_size(M, N, K))


def gemm_bf16_ex(A, B, bias, C, epilogue=EPI_NONE, algo=ALGO_AUTO, workspace=None, stream=None):
    """C[M,N] = epilogue(A[M,K] @ B[K,N] + bias[N]) on the GPU (writes C in place).

    A, B: bfloat16, row-major (unit inner stride, any row stride).
    bias: bfloat16 [N] contiguous, or None for EPI_NONE.
    C: float32 or bfloat16 [M, N], row-major.
    workspace: None (never split) or a device tensor of at least
    gemm_bf16_workspace_size(M, N, K, algo) bytes for the small-M K split.
    """
    _check_cuda(A, B, bias, C)
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise ValueError("A and B must be bfloat16")
    if C.dtype == torch.float32:
        out = OUT_F32
    elif C.dtype == torch.bfloat16:
        out = OUT_BF16
    else:
        raise ValueError("C must be float32 or bfloat16")
    if bias is not None and (bias.dtype != torch.bfloat16 or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous bfloat16 vector")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K or tuple(C.shape) != (M, N) or (bias is not None and bias.numel() != N):
        raise ValueError(f"shape mismatch A{tuple(A.shape)} B{tuple(B.shape)} C{tuple(C.shape)}")
    wp, wb = _workspace(workspace)
    st = lib().gemm_bf16_ex(_ptr(A), _ptr(B), _ptr(bias), _ptr(C), M, N, K,
                            _row_major(A, "A"), _row_major(B, "B"), _row_major(C, "C"),
                            int(epilogue), out, int(algo), wp, wb, _stream_ptr(stream))
    if st != TGEMM_OK:
        raise TgemmError(st, "gemm_bf16_ex")
    return C


def gemm_bf16_noalloc(A, B, bias, C, epilogue=EPI_NONE, algo=ALGO_AUTO, stream=None):
    """gemm_bf16_ex with the small-M K split in the library's fixed device
    scratch (no workspace argument, nothing allocated); raises TgemmError
    (status TGEMM_ERR_SCRATCH) when the split needs more than
    NOALLOC_SCRATCH_BYTES.  Calls that overlap on one GPU share the scratch."""
    _check_cuda(A, B, bias, C)
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise ValueError("A and B must be bfloat16")
    if C.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("C must be float32 or bfloat16")
    if bias is not None and (bias.dtype != torch.bfloat16 or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous bfloat16 vector")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K or tuple(C.shape) != (M, N) or (bias is not None and bias.numel() != N):
        raise ValueError(f"shape mismatch A{tuple(A.shape)} B{tuple(B.shape)} C{tuple(C.shape)}")
    out = OUT_F32 if C.dtype == torch.float32 else OUT_BF16
    st = lib().gemm_bf16_noalloc(_ptr(A), _ptr(B), _ptr(bias), _ptr(C), M, N, K,
                                 _row_major(A, "A"), _row_major(B, "B"), _row_major(C, "C"),
                                 int(epilogue), out, int(algo), _stream_ptr(stream))
    if st != TGEMM_OK:
        raise TgemmError(st, "gemm_bf16_noalloc")
    return C


def gemm_bf16(A, B, bias, C, epilogue=EPI_NONE, stream=None):
    """gemm_bf16 of the C ABI: the library picks the kernel family (no workspace)."""
    _check_cuda(A, B, bias, C)
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise ValueError("A and B must be bfloat16")
    if C.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("C must be float32 or bfloat16")
    if bias is not None and (bias.dtype != torch.bfloat16 or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous bfloat16 vector")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K or tuple(C.shape) != (M, N) or (bias is not None and bias.numel() != N):
        raise ValueError(f"shape mismatch A{tuple(A.shape)} B{tuple(B.shape)} C{tuple(C.shape)}")
    out = OUT_F32 if C.dtype == torch.float32 else OUT_BF16
    st = lib().gemm_bf16(_ptr(A), _ptr(B), _ptr(bias), _ptr(C), M, N, K,
                         _row_major(A, "A"), _row_major(B, "B"), _row_major(C, "C"),
                         int(epilogue), out, _stream_ptr(stream))
    if st != TGEMM_OK:
        raise TgemmError(st, "gemm_bf16")
    return C


def _fp8_operands(A, sA, B, sB, C):
    _check_cuda(A, sA, B, sB, C)
    if A.dtype != torch.float8_e4m3fn or B.dtype != torch.float8_e4m3fn:
        raise ValueError("A and B must be float8_e4m3fn")
    if sA.dtype != torch.float32 or sB.dtype != torch.float32 or C.dtype != torch.bfloat16:
        raise ValueError("scales must be float32 and C bfloat16")
    for t, n in ((A, "A"), (B, "B"), (sA, "sA"), (sB, "sB"), (C, "C")):
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous (packed row-major)")
    M, K = A.shape
    K2, N = B.shape
    G, H = (K + 127) // 128, (N + 127) // 128
    if K2 != K or tuple(C.shape) != (M, N) or tuple(sA.shape) != (M, G) or tuple(sB.shape) != (G, H):
        raise ValueError("shape mismatch")
    return M, N, K


def gemm_fp8_blockscaled(A, sA, B, sB, C, stream=None):
    """C[M,N] (bf16) = sum_g sA[:,g] sB[g,n/128] (A_g @ B_g) with e4m3fn A, B.

    A: float8_e4m3fn [M, K] contiguous; sA: float32 [M, ceil(K/128)] contiguous;
    B: float8_e4m3fn [K, N] contiguous; sB: float32 [ceil(K/128), ceil(N/128)];
    C: bfloat16 [M, N] contiguous.  A sparse last round of 256 x 256 tiles
    runs as 128-row halves (bit-identical); never split along K.
    """
    M, N, K = _fp8_operands(A, sA, B, sB, C)
    st = lib().gemm_fp8_blockscaled(_ptr(A), _ptr(sA), _ptr(B), _ptr(sB), _ptr(C), M, N, K,
                                    _stream_ptr(stream))
    if st != TGEMM_OK:
        raise TgemmError(st, "gemm_fp8_blockscaled")
    return C


def gemm_fp8_blockscaled_ex(A, sA, B, sB, C, split_parts=0, workspace=None, stream=None):
    """gemm_fp8_blockscaled_ex of the C ABI: split_parts 0 automatic, 1 never
    (whole 256 x 256 tiles only), 2..8 K ranges per tile of the last round;
    workspace None (never split along K)
    or a zero-initialised device tensor of at least
    gemm_fp8_workspace_size(M, N, K, split_parts) bytes (its arrival counters
    are left zero by every call, so it can be reused as is)."""
    M, N, K = _fp8_operands(A, sA, B, sB, C)
    wp, wb = _workspace(workspace)
    st = lib().gemm_fp8_blockscaled_ex(_ptr(A), _ptr(sA), _ptr(B), _ptr(sB), _ptr(C), M, N, K,
                                       int(split_parts), wp, wb, _stream_ptr(stream))
    if st != TGEMM_OK:
        raise TgemmError(st, "gemm_fp8_blockscaled_ex")
    return C


def gemm_bf16_quant_fp8(A, B, bias, Q, S, epilogue=EPI_NONE, algo=ALGO_AUTO, stream=None):
    """Q, S = 1x128 FP8 quantisation of bf16(epilogue(A @ B + bias)), one kernel.

    A: bf16 [M, K] (row stride free); B: bf16 [K, N] (row stride free);
    bias: bf16 [N] or None; Q: float8_e4m3fn or uint8 [M, N] contiguous;
    S: float32 [M, ceil(N/128)] contiguous.
    """
    _check_cuda(A, B, Q, S, *([bias] if bias is not None else []))
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise ValueError("A and B must be bfloat16")
    if Q.dtype not in (torch.float8_e4m3fn, torch.uint8) or S.dtype != torch.float32:
        raise ValueError("Q must be float8_e4m3fn (or uint8) and S float32")
    if not Q.is_contiguous() or not S.is_contiguous():
        raise ValueError("Q and S must be contiguous (packed row-major)")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K or tuple(Q.shape) != (M, N) or tuple(S.shape) != (M, (N + 127) // 128):
        raise ValueError("shape mismatch")
    if bias is not None and (bias.dtype != torch.bfloat16 or bias.numel() != N):
        raise ValueError("bias must be bfloat16 [N]")
    st = lib().gemm_bf16_quant_fp8(_ptr(A), _ptr(B), _ptr(bias) if bias is not None else None,
                                   _ptr(Q), _ptr(S), M, N, K, _row_major(A, "A"), _row_major(B, "B"),
                                   int(epilogue), int(algo), _stream_ptr(stream))
    if st != TGEMM_OK:
        raise TgemmError(st, "gemm_bf16_quant_fp8")
    return Q, S


def gemm_fp8_blockscaled_nt(A, sA, Bt, sB, C, stream=None):
    """gemm_fp8_blockscaled with the weight K-contiguous: Bt float8_e4m3fn [N, K].

    A: float8_e4m3fn [M, K]; sA: float32 [M, ceil(K/128)]; sB: float32
    [ceil(K/128), ceil(N/128)]; C: bfloat16 [M, N]; all contiguous.
    """
    _check_cuda(A, sA, Bt, sB, C)
    if A.dtype != torch.float8_e4m3fn or Bt.dtype != torch.float8_e4m3fn:
        raise ValueError("A and Bt must be float8_e4m3fn")
    if sA.dtype != torch.float32 or sB.dtype != torch.float32 or C.dtype != torch.bfloat16:
        raise ValueError("scales must be float32 and C bfloat16")
    for t, n in ((A, "A"), (Bt, "Bt"), (sA, "sA"), (sB, "sB"), (C, "C")):
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous (packed row-major)")
    M, K = A.shape
    N, K2 = Bt.shape
    G, H = (K + 127) // 128, (N + 127) // 128
    if K2 != K or tuple(C.shape) != (M, N) or tuple(sA.shape) != (M, G) or tuple(sB.shape) != (G, H):
        raise ValueError("shape mismatch")
    st = lib().gemm_fp8_blockscaled_nt(_ptr(A), _ptr(sA), _ptr(Bt), _ptr(sB), _ptr(C), M, N, K,
                                       _stream_ptr(stream))
    if st != TGEMM_OK:
        raise TgemmError(st, "gemm_fp8_blockscaled_nt")
    return C


PROBE_MFMA_BF16, PROBE_MFMA_FP8, PROBE_STREAM_READ = 0, 1, 2


def gemm_probe_out_elems(probe):
    """Number of 32-bit outputs the probe writes on the current device."""
    return int(lib().gemm_probe_out_elems(int(probe)))


def gemm_probe_mfma_flop(probe, iters):
    return float(lib().gemm_probe_mfma_flop(int(probe), int(iters)))


def gemm_probe_mfma(probe, iters, out, seed=1, stream=None):
    """MFMA-only loop on seeded random register operands (probe PROBE_MFMA_BF16
    or PROBE_MFMA_FP8); out: float32 tensor of at least gemm_probe_out_elems()."""
    _check_cuda(out)
    if out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor")
    st = lib().gemm_probe_mfma(int(probe), int(iters), _ptr(out), out.numel(), int(seed), _stream_ptr(stream))
    if st != TGEMM_OK:
        raise TgemmError(st, "gemm_probe_mfma")
    return out


def gemm_probe_stream_read(src, out, stream=None):
    """Streaming read of src (16-byte aligned, size a multiple of 16 bytes);
    out: int32 tensor of at least gemm_probe_out_elems(PROBE_STREAM_READ)
    holding per-thread XORs of the 32-bit words read."""
    _check_cuda(src, out)
    if out.dtype != torch.int32 or not out.is_contiguous() or not src.is_contiguous():
        raise ValueError("out must be a contiguous int32 tensor and src contiguous")
    nbytes = src.numel() * src.element_size()
    st = lib().gemm_probe_stream_read(_ptr(src), nbytes, _ptr(out), out.numel(), _stream_ptr(stream))
    if st != TGEMM_OK:
        raise TgemmError(st, "gemm_probe_stream_read")
    return out


def gemm_fp8_split_plan(M, N, K, cus, split_parts=0):
    """(whole, split_tiles, parts) of the FP8 tile scheduler (host only)."""
    w, t, p = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    st = lib().gemm_fp8_split_plan(M, N, K, cus, split_parts, ctypes.byref(w), ctypes.byref(t),
                                   ctypes.byref(p))
    if st != TGEMM_OK:
        raise TgemmError(st, "gemm_fp8_split_plan")
    return w.value, t.value, p.value


def _batch_stride(t):
    return t.stride(0) if t.shape[0] > 1 else 0


def gemm_bf16_strided_batched(A, B, bias, C, b_layout=B_KN, epilogue=EPI_NONE, stream=None):
    """C[z] = epilogue(A[z] @ B[z] + bias) for every z of a batch, one launch.

    A: bfloat16 [batch, M, K]; B: bfloat16 [batch, K, N] (b_layout B_KN) or
    [batch, N, K] (B_NK, the product is then A[z] @ B[z].T); C: bfloat16 or
    float32 [batch, M, N]; each matrix with unit inner stride, any row and
    batch strides (an expanded tensor, batch stride 0, shares an operand).
    """
    _check_cuda(A, B, bias, C)
    if A.dim() != 3 or B.dim() != 3 or C.dim() != 3:
        raise ValueError("A, B and C must be 3-D [batch, rows, cols]")
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise ValueError("A and B must be bfloat16")
    if C.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("C must be bfloat16 or float32")
    if bias is not None and (bias.dtype != torch.bfloat16 or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous bfloat16 vector")
    batch, M, K = A.shape
    if b_layout == B_KN:
        K2, N = B.shape[1:]
    else:
        N, K2 = B.shape[1:]
    if K2 != K or tuple(C.shape) != (batch, M, N) or B.shape[0] != batch:
        raise ValueError("shape mismatch")
    lda, ldb, ldc = _row_major(A[0], "A"), _row_major(B[0], "B"), _row_major(C[0], "C")
    out = OUT_BF16 if C.dtype == torch.bfloat16 else OUT_F32
    st = lib().gemm_bf16_strided_batched(_ptr(A), _ptr(B), _ptr(bias), _ptr(C), M, N, K, lda, ldb, ldc,
                                         _batch_stride(A), _batch_stride(B), _batch_stride(C), batch,
                                         int(b_layout), int(epilogue), out, _stream_ptr(stream))
    if st != TGEMM_OK:
        raise TgemmError(st, "gemm_bf16_strided_batched")
    return C


def gemm_bf16_nt(A, Bt, bias, C, epilogue=EPI_NONE, stream=None):
    """C[M,N] = epilogue(A[M,K] @ Bt[N,K].T + bias[N]) on the GPU (writes C in
    place); Bt is the K-contiguous weight, as nn.Linear stores it."""
    _check_cuda(A, Bt, bias, C)
    for t, nm in ((A, "A"), (Bt, "Bt")):
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{nm} must be bfloat16")
    if C.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("C must be bfloat16 or float32")
    if bias is not None and (bias.dtype != torch.bfloat16 or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous bfloat16 vector")
    lda, ldb, ldc = _row_major(A, "A"), _row_major(Bt, "Bt"), _row_major(C, "C")
    M, K = A.shape
    N, K2 = Bt.shape
    if K2 != K or tuple(C.shape) != (M, N):
        raise ValueError("shape mismatch")
    out = OUT_BF16 if C.dtype == torch.bfloat16 else OUT_F32
    st = lib().gemm_bf16_nt(_ptr(A), _ptr(Bt), _ptr(bias), _ptr(C), M, N, K, lda, ldb, ldc,
                            int(epilogue), out, _stream_ptr(stream))
    if st != TGEMM_OK:
        raise TgemmError(st, "gemm_bf16_nt")
    return C


def gemm_bf16_nt_kernel_name(M, N, K):
    r = lib().gemm_bf16_nt_kernel_name(M, N, K)
    return None if r is None else r.decode()


def gemm_logsoftmax_workspace_size(M, N, out_dtype=OUT_BF16):
    return int(lib().gemm_logsoftmax_workspace_size(M, N, out_dtype))


def gemm_bf16_logsoftmax(X, W, bias, C, workspace=None, stream=None):
    """C[M,N] = log_softmax(X[M,K] @ W[K,N] + bias[N], over N) on the GPU.

    X, W: bfloat16 (unit inner stride); bias: bfloat16 [N] or None; C:
    bfloat16 or float32 [M, N] (unit inner stride), written in place.
    workspace: a 16-byte aligned device tensor of at least
    gemm_logsoftmax_workspace_size(M, N, out dtype) bytes, or None to allocate
    one here (torch's caching allocator).
    """
    _check_cuda(X, W, bias, C)
    if X.dtype != torch.bfloat16 or W.dtype != torch.bfloat16:
        raise ValueError("X and W must be bfloat16")
    if C.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("C must be bfloat16 or float32")
    if bias is not None and (bias.dtype != torch.bfloat16 or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous bfloat16 vector")
    ldx, ldw, ldc = _row_major(X, "X"), _row_major(W, "W"), _row_major(C, "C")
    M, K = X.shape
    K2, N = W.shape
    if K2 != K or tuple(C.shape) != (M, N) or (bias is not None and bias.numel() != N):
        raise ValueError("shape mismatch")
    out = OUT_BF16 if C.dtype == torch.bfloat16 else OUT_F32
    need = gemm_logsoftmax_workspace_size(M, N, out)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=X.device)
    _check_cuda(workspace)
    st = lib().gemm_bf16_logsoftmax(_ptr(X), _ptr(W), _ptr(bias), _ptr(C), M, N, K, ldx, ldw, ldc,
                                    out, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream_ptr(stream))
    if st != TGEMM_OK:
        raise TgemmError(st, "gemm_bf16_logsoftmax")
    return C


def _weight_only(name, bits, X, Q, S, bias, C, epilogue, workspace, stream):
    _check_cuda(X, Q, S, bias, C)
    qdt = torch.int8 if bits == 8 else torch.uint8
    if X.dtype != torch.bfloat16 or Q.dtype != qdt or S.dtype != torch.float32:
        raise ValueError(f"X must be bfloat16, Q {qdt} and S float32")
    if C.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("C must be bfloat16 or float32")
    if bias is not None and (bias.dtype != torch.bfloat16 or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous bfloat16 vector")
    ldx, ldq, ldc = _row_major(X, "X"), _row_major(Q, "Q"), _row_major(C, "C")
    M, K = X.shape
    Kq, N = Q.shape
    if bits == 4 and K % 2:
        raise ValueError("int4 codes pair up along K: K must be even")
    if Kq != (K if bits == 8 else K // 2) or tuple(C.shape) != (M, N) \
            or tuple(S.shape) != ((K + 127) // 128, N):
        raise ValueError("shape mismatch")
    if not S.is_contiguous():
        raise ValueError("S must be contiguous")
    out = OUT_BF16 if C.dtype == torch.bfloat16 else OUT_F32
    wp, wb = _workspace(workspace)
    st = getattr(lib(), name)(_ptr(X), _ptr(Q), _ptr(S), _ptr(bias), _ptr(C), M, N, K, ldx, ldq, ldc,
                              int(epilogue), out, wp, wb, _stream_ptr(stream))
    if st != TGEMM_OK:
        raise TgemmError(st, name)
    return C


def gemm_bf16_w8(X, Q, S, bias, C, epilogue=EPI_NONE, workspace=None, stream=None):
    """C[M,N] = epilogue(X[M,K] @ (Q[K,N] * S[k/128, N]) + bias[N]) on the GPU.

    X: bfloat16 [M, K] (unit inner stride); Q: int8 [K, N] (unit inner stride);
    S: float32 [ceil(K/128), N] contiguous; bias: bfloat16 [N] or None;
    C: bfloat16 or float32 [M, N] (unit inner stride), written in place.
    workspace: None (never split) or a device tensor of at least
    gemm_wq_workspace_size(M, N, K) bytes for the K split of narrow weights.
    """
    return _weight_only("gemm_bf16_w8", 8, X, Q, S, bias, C, epilogue, workspace, stream)


def gemm_bf16_w4(X, Q, S, bias, C, epilogue=EPI_NONE, workspace=None, stream=None):
    """gemm_bf16_w8 with int4 codes: Q is uint8 [K/2, N], byte (r, n) holding
    code (2r, n) in its low nibble and (2r+1, n) in its high nibble, each a
    4-bit two's-complement value."""
    return _weight_only("gemm_bf16_w4", 4, X, Q, S, bias, C, epilogue, workspace, stream)


def _weight_only_logsoftmax(name, bits, X, Q, S, bias, C, workspace, stream):
    _check_cuda(X, Q, S, bias, C)
    qdt = torch.int8 if bits == 8 else torch.uint8
    if X.dtype != torch.bfloat16 or Q.dtype != qdt or S.dtype != torch.float32:
        raise ValueError(f"X must be bfloat16, Q {qdt} and S float32")
    if C.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("C must be bfloat16 or float32")
    if bias is not None and (bias.dtype != torch.bfloat16 or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous bfloat16 vector")
    ldx, ldq, ldc = _row_major(X, "X"), _row_major(Q, "Q"), _row_major(C, "C")
    M, K = X.shape
    Kq, N = Q.shape
    if bits == 4 and K % 2:
        raise ValueError("int4 codes pair up along K: K must be even")
    if Kq != (K if bits == 8 else K // 2) or tuple(C.shape) != (M, N) \
            or tuple(S.shape) != ((K + 127) // 128, N) or (bias is not None and bias.numel() != N):
        raise ValueError("shape mismatch")
    if not S.is_contiguous():
        raise ValueError("S must be contiguous")
    out = OUT_BF16 if C.dtype == torch.bfloat16 else OUT_F32
    need = gemm_logsoftmax_workspace_size(M, N, out)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=X.device)
    _check_cuda(workspace)
    st = getattr(lib(), name)(_ptr(X), _ptr(Q), _ptr(S), _ptr(bias), _ptr(C), M, N, K, ldx, ldq, ldc,
                              out, _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _stream_ptr(stream))
    if st != TGEMM_OK:
        raise TgemmError(st, name)
    return C


def gemm_bf16_w8_logsoftmax(X, Q, S, bias, C, workspace=None, stream=None):
    """C[M,N] = log_softmax(X @ (Q * S[k/128, n]) + bias, over N): the int8 LM head
    of gemm_bf16_w8 with the fused log-softmax of gemm_bf16_logsoftmax."""
    return _weight_only_logsoftmax("gemm_bf16_w8_logsoftmax", 8, X, Q, S, bias, C, workspace, stream)


def gemm_bf16_w4_logsoftmax(X, Q, S, bias, C, workspace=None, stream=None):
    """gemm_bf16_w8_logsoftmax with int4 codes packed two per byte along K."""
    return _weight_only_logsoftmax("gemm_bf16_w4_logsoftmax", 4, X, Q, S, bias, C, workspace, stream)


def gemm_w8_kernel_name(M, N, K, with_workspace=False):
    r = lib().gemm_w8_kernel_name(M, N, K, int(bool(with_workspace)))
    return None if r is None else r.decode()


def gemm_w4_kernel_name(M, N, K, with_workspace=False):
    r = lib().gemm_w4_kernel_name(M, N, K, int(bool(with_workspace)))
    return None if r is None else r.decode()


def _quantize(name, X, Q, S, group_rows, stream):
    _check_cuda(X, Q, S)
    if X.dtype != torch.bfloat16:
        raise ValueError("X must be bfloat16")
    if Q.dtype not in (torch.float8_e4m3fn, torch.uint8) or S.dtype != torch.float32:
        raise ValueError("Q must be float8_e4m3fn (or uint8 codes) and S float32")
    ld = _row_major(X, "X")
    R, Cn = X.shape
    if not Q.is_contiguous() or not S.is_contiguous():
        raise ValueError("Q and S must be contiguous (packed row-major)")
    G = (R + 127) // 128 if group_rows else R
    if tuple(Q.shape) != (R, Cn) or tuple(S.shape) != (G, (Cn + 127) // 128):
        raise ValueError("shape mismatch")
    st = getattr(lib(), name)(_ptr(X), _ptr(Q), _ptr(S), R, Cn, ld, _stream_ptr(stream))
    if st != TGEMM_OK:
        raise TgemmError(st, name)
    return Q, S


def quantize_fp8_1x128(X, Q, S, stream=None):
    """FP8 codes and per-(row, 128-column group) scales of X on the GPU.

    X: bfloat16 [M, K] with unit inner stride; Q: float8_e4m3fn (or uint8)
    [M, K] contiguous; S: float32 [M, ceil(K/128)] contiguous.  Written in
    place; returns (Q, S).
    """
    return _quantize("quantize_fp8_1x128", X, Q, S, False, stream)


def quantize_fp8_128x128(W, Q, S, stream=None):
    """FP8 codes and per-128x128-block scales of W on the GPU.

    W: bfloat16 [K, N] with unit inner stride; Q: float8_e4m3fn (or uint8)
    [K, N] contiguous; S: float32 [ceil(K/128), ceil(N/128)] contiguous.
    """
    return _quantize("quantize_fp8_128x128", W, Q, S, True, stream)


def gemm_bf16_kernel_name(M, N, K, epilogue=EPI_NONE, out_dtype=OUT_BF16, algo=ALGO_AUTO,
                          with_workspace=False):
    r = lib().gemm_bf16_kernel_name(M, N, K, epilogue, out_dtype, algo, int(bool(with_workspace)))
    return None if r is None else r.decode()


def gemm_fp8_kernel_name(M, N, K):
    r = lib().gemm_fp8_kernel_name(M, N, K)
    return None if r is None else r.decode()


def gemm_status_string(status):
    return lib().gemm_status_string(status).decode()


def gemm_abi_version():
    return lib().gemm_abi_version()
