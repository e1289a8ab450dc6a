"""GPU: the two load pipelines of the small-M kernels agree bit for bit
(needs an MI355X).

The [K, N] and K-contiguous small-M kernels bring the weight to LDS either
through registers (non-temporal loads, when the grid has at least three
quarters as many workgroups as the device has compute units) or with direct
loads into LDS (smaller grids).  Both place the same bytes in LDS and run the
same MFMA sequence, so they must agree exactly.  A single call on a narrow
weight runs the direct pipeline; the same problem repeated over a strided
batch (operands shared through batch stride 0) fills the grid and runs the
register-staged one.  Every batch entry must equal the single call bit for
bit, and the single call must match the fp64 oracle.  K is below eight
32-row slices, so the single [K, N] call is not split along K.
"""

import pytest
import torch

import tiled_gemm_04_amd as tg
import workloads as wl
from oracle import gemm as og

pytestmark = pytest.mark.gpu

TOL_F32, TOL_BF16 = 1e-5, 8e-3
BATCH = 8


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("M", [1, 17, 64])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_register_and_direct_pipelines_agree(layout, M, out_dtype):
    dev = _dev()
    N, K = 20000, 200  # N and K both ragged against the kernels' tiles
    cols_per_wg = 512 if layout == "kn" else 256
    wgs = -(-N // cols_per_wg)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert 4 * wgs < 3 * cus <= 4 * wgs * BATCH, (wgs, cus)
    seed = 9600 + M + (0 if layout == "kn" else 1)
    print(f"[gpu] thin pipelines layout={layout} M={M} N={N} K={K} out={out_dtype}", flush=True)
    a = wl.bf16((M, K), "normal", 1.0, seed, 1, dev)
    b = wl.bf16((K, N), "normal", 0.05, seed, 2, dev)
    bias = wl.bf16((N,), "normal", 0.5, seed, 3, dev)
    b_op = b if layout == "kn" else b.t().contiguous()
    single = torch.empty(M, N, dtype=out_dtype, device=dev)
    batched = torch.empty(BATCH, M, N, dtype=out_dtype, device=dev)
    if layout == "kn":
        tg.gemm_bf16(a, b_op, bias, single, epilogue=tg.EPI_BIAS)
    else:
        tg.gemm_bf16_nt(a, b_op, bias, single, epilogue=tg.EPI_BIAS)
    tg.gemm_bf16_strided_batched(a.unsqueeze(0).expand(BATCH, M, K), b_op.unsqueeze(0).expand(BATCH, *b_op.shape),
                                 bias, batched, b_layout=tg.B_KN if layout == "kn" else tg.B_NK,
                                 epilogue=tg.EPI_BIAS)
    torch.cuda.synchronize()
    raw = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
    for z in range(BATCH):
        assert torch.equal(batched[z].view(raw), single.view(raw)), z
    y, d = og.gemm_bf16_bits(wl.bits_u16(a), wl.bits_u16(b), wl.bits_u16(bias), tg.EPI_BIAS)
    r = og.compare(single.float().cpu().double().numpy(), y, d, TOL_F32 if out_dtype == torch.float32 else TOL_BF16)
    assert r["ok"], r
