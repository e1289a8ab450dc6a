"""The attainable-ceiling probes on an MI355X: they run, give finite and
reproducible results, the stream read sees every byte (the XOR of its
outputs equals the host's XOR of the buffer), and the measured rates sit
below the published peaks (2.5 PFLOP/s bf16, 5 PFLOP/s fp8, 8 TB/s)."""

import numpy as np
import pytest
import torch

import tiled_gemm_04_amd as tg

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


def _time(fn, reps=3):
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / reps


@pytest.mark.parametrize("probe,peak_tflops", [(tg.PROBE_MFMA_BF16, 2500.0), (tg.PROBE_MFMA_FP8, 5000.0)])
def test_mfma_probe_runs_reproducibly_below_peak(probe, peak_tflops):
    dev = _dev()
    n = tg.gemm_probe_out_elems(probe)
    assert n > 0
    print(f"[gpu] probe mfma {probe} outputs={n}", flush=True)
    out = torch.full((n,), float("nan"), dtype=torch.float32, device=dev)
    iters = 200
    sec = _time(lambda: tg.gemm_probe_mfma(probe, iters, out, seed=7))
    first = out.clone()
    tg.gemm_probe_mfma(probe, iters, out, seed=7)
    torch.cuda.synchronize()
    assert torch.isfinite(first).all()
    assert torch.equal(first, out)
    tflops = tg.gemm_probe_mfma_flop(probe, iters) / sec / 1e12
    print(f"[gpu] probe mfma {probe}: {tflops:.0f} TFLOP/s", flush=True)
    assert 0.2 * peak_tflops < tflops < 1.05 * peak_tflops


def test_stream_read_probe_sees_every_word():
    dev = _dev()
    nbytes = (512 << 20) + 48  # beyond the 256 MB last-level cache, with a tail past whole rows
    g = torch.Generator(device=dev).manual_seed(5)
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), generator=g, dtype=torch.int32, device=dev)
    n = tg.gemm_probe_out_elems(tg.PROBE_STREAM_READ)
    out = torch.zeros(n, dtype=torch.int32, device=dev)
    print(f"[gpu] probe stream read {nbytes} bytes outputs={n}", flush=True)
    sec = _time(lambda: tg.gemm_probe_stream_read(src, out))
    want = np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == want
    gbs = nbytes / sec / 1e9
    print(f"[gpu] probe stream read: {gbs:.0f} GB/s", flush=True)
    assert gbs < 8000.0 * 1.05
