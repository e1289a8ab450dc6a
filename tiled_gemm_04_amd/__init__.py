"""tgemm: bf16 and FP8 block-scaled GEMM for AMD MI355X (gfx950).

The compute path is the HIP library libtgemm.so (sources in csrc/, C ABI in
include/tgemm.h); this package only builds it and marshals torch tensors into
its calls.
"""

from .binding import (  # noqa: F401
    ALGO_AUTO, ALGO_THIN, ALGO_TILED, ALGO_TILED_128x128, ALGO_TILED_256x128, ALGO_TILED_256x256,
    B_KN, B_NK, EPI_BIAS, EPI_BIAS_GELU_TANH, EPI_NONE, OUT_BF16, OUT_F32,
    PROBE_MFMA_BF16, PROBE_MFMA_FP8, PROBE_STREAM_READ,
    NOALLOC_SCRATCH_BYTES, TGEMM_ERR_SCRATCH,
    TgemmError, gemm_abi_version, gemm_bf16, gemm_bf16_ex, gemm_bf16_kernel_name, gemm_bf16_noalloc,
    gemm_bf16_logsoftmax, gemm_bf16_nt, gemm_bf16_nt_kernel_name, gemm_bf16_quant_fp8,
    gemm_bf16_strided_batched, gemm_bf16_w4, gemm_bf16_w4_logsoftmax, gemm_bf16_w8,
    gemm_bf16_w8_logsoftmax, gemm_bf16_workspace_size, gemm_fp8_blockscaled, gemm_fp8_blockscaled_ex,
    gemm_fp8_blockscaled_nt, gemm_fp8_kernel_name, gemm_fp8_split_plan, gemm_fp8_workspace_size,
    gemm_logsoftmax_workspace_size, gemm_probe_mfma, gemm_probe_mfma_flop, gemm_probe_out_elems,
    gemm_probe_stream_read, gemm_status_string, gemm_w4_kernel_name, gemm_w8_kernel_name,
    gemm_wq_workspace_size, lib, quantize_fp8_1x128, quantize_fp8_128x128,
)
