"""The entry points inside a captured HIP graph (needs an MI355X).

The library allocates nothing, issues no memset and never synchronises, so a
sequence of its calls can be captured once and replayed.  The graph below
holds the tiled bf16 GEMM with bias + tanh-GeLU, the small-M split-K with a
caller workspace, the FP8 GEMM with its last round split in a workspace
(whose arrival counters every call returns to zero), the log-softmax LM
head, the int8 head split along K in a caller workspace (two launches), the
FP8 GEMM with its last round as half tiles (no workspace), the 1 x 128
FP8 quantiser and the allocation-free entry point (the same small-M split in
the library's fixed scratch).  It is replayed four times with eager library calls and host
synchronisations in between; every replay must reproduce the eager results
bit for bit, which in turn are checked against the fp64 oracle.
"""

import pytest
import torch

import tiled_gemm_04_amd as tg
import workloads as wl
from oracle import gemm as og
from oracle import quant as oq

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


def _bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).clone()


def test_captured_sequence_replays_bit_for_bit():
    dev = _dev()
    print("[gpu] graph capture and replay", flush=True)
    # tiled bf16 with bias + tanh-GeLU (several tiles, a ragged edge)
    a1 = wl.bf16((600, 512), "normal", 1.0, 141, 1, dev)
    b1 = wl.bf16((512, 700), "normal", 0.05, 141, 2, dev)
    bias1 = wl.bf16((700,), "normal", 0.5, 141, 3, dev)
    c1 = torch.empty(600, 700, dtype=torch.bfloat16, device=dev)
    # small-M split-K in a caller workspace
    a2 = wl.bf16((8, 4096), "normal", 1.0, 142, 1, dev)
    b2 = wl.bf16((4096, 4096), "normal", 0.05, 142, 2, dev)
    c2 = torch.empty(8, 4096, dtype=torch.float32, device=dev)
    ws2 = torch.empty(tg.gemm_bf16_workspace_size(8, 4096, 4096), dtype=torch.uint8, device=dev)
    assert ws2.numel() > 0
    # FP8 with a split last round (counters at the head of the workspace)
    qa, sa, qb, sb = wl.fp8_inputs(wl.WORKLOADS["fp8"], device=dev, M=600, N=700, K=2048)
    c3 = torch.empty(600, 700, dtype=torch.bfloat16, device=dev)
    ws3 = torch.zeros(tg.gemm_fp8_workspace_size(600, 700, 2048), dtype=torch.uint8, device=dev)
    assert ws3.numel() > 0
    # log-softmax LM head
    x4 = wl.bf16((5, 1024), "normal", 1.0, 143, 1, dev)
    w4 = wl.bf16((1024, 20000), "normal", 0.05, 143, 2, dev)
    b4 = wl.bf16((20000,), "normal", 0.02, 143, 3, dev)
    c4 = torch.empty(5, 20000, dtype=torch.float32, device=dev)
    ws4 = torch.empty(tg.gemm_logsoftmax_workspace_size(5, 20000, tg.OUT_F32), dtype=torch.uint8, device=dev)
    # int8 head split along K in a caller workspace
    x5 = wl.bf16((8, 4096), "normal", 1.0, 144, 1, dev)
    q5, s5 = wl.w8_weights(4096, 4096, 144, dev)
    c5 = torch.empty(8, 4096, dtype=torch.float32, device=dev)
    ws5 = torch.empty(tg.gemm_wq_workspace_size(8, 4096, 4096), dtype=torch.uint8, device=dev)
    assert ws5.numel() > 0
    # FP8 with its last round as half tiles (9 tiles: all halved)
    qa6, sa6, qb6, sb6 = wl.fp8_inputs(wl.WORKLOADS["fp8"], device=dev, M=600, N=700, K=384)
    c6 = torch.empty(600, 700, dtype=torch.bfloat16, device=dev)
    # 1 x 128 FP8 quantiser
    x7 = wl.bf16((300, 1000), "normal", 1.0, 145, 1, dev)
    q7 = torch.empty(300, 1000, dtype=torch.uint8, device=dev)
    s7 = torch.empty(300, 8, dtype=torch.float32, device=dev)
    # the allocation-free entry point on the small-M split's inputs
    c8 = torch.empty(8, 4096, dtype=torch.float32, device=dev)

    def calls():
        tg.gemm_bf16(a1, b1, bias1, c1, epilogue=tg.EPI_BIAS_GELU_TANH)
        tg.gemm_bf16_ex(a2, b2, None, c2, workspace=ws2)
        tg.gemm_fp8_blockscaled_ex(qa, sa, qb, sb, c3, split_parts=0, workspace=ws3)
        tg.gemm_bf16_logsoftmax(x4, w4, b4, c4, workspace=ws4)
        tg.gemm_bf16_w8(x5, q5, s5, None, c5, workspace=ws5)
        tg.gemm_fp8_blockscaled(qa6, sa6, qb6, sb6, c6)
        tg.quantize_fp8_1x128(x7, q7, s7)
        tg.gemm_bf16_noalloc(a2, b2, None, c8)

    outs = (c1, c2, c3, c4, c5, c6, q7, s7, c8)
    calls()
    torch.cuda.synchronize()
    eager = [_bits(c) for c in outs]

    # The eager results against the oracle.
    y, d = og.gemm_bf16_bits(wl.bits_u16(a1), wl.bits_u16(b1), wl.bits_u16(bias1), tg.EPI_BIAS_GELU_TANH)
    assert og.compare(c1.float().cpu().double().numpy(), y, d, 8e-3)["ok"]
    y, d = og.gemm_bf16_bits(wl.bits_u16(a2), wl.bits_u16(b2))
    assert og.compare(c2.cpu().double().numpy(), y, d, 1e-5)["ok"]
    y, d = og.gemm_fp8_blockscaled_bits(wl.bits_u8(qa), sa.cpu().numpy(), wl.bits_u8(qb), sb.cpu().numpy())
    assert og.compare(c3.float().cpu().double().numpy(), y, d, 1.5e-2)["ok"]
    out, dmax, lse = og.gemm_bf16_logsoftmax_bits(wl.bits_u16(x4), wl.bits_u16(w4), wl.bits_u16(b4))
    assert og.compare(c4.cpu().double().numpy(), out, og.logsoftmax_bound(out, dmax, lse, "f32"), 1.0)["ok"]
    y, d = og.gemm_bf16_w8_bits(wl.bits_u16(x5), q5.cpu().numpy(), s5.cpu().numpy())
    assert og.compare(c5.cpu().double().numpy(), y, d, 1e-5)["ok"]
    y, d = og.gemm_fp8_blockscaled_bits(wl.bits_u8(qa6), sa6.cpu().numpy(), wl.bits_u8(qb6), sb6.cpu().numpy())
    assert og.compare(c6.float().cpu().double().numpy(), y, d, 1.5e-2)["ok"]
    y, d = og.gemm_bf16_bits(wl.bits_u16(a2), wl.bits_u16(b2))
    assert og.compare(c8.cpu().double().numpy(), y, d, 1e-5)["ok"]
    rq, rs = oq.quantise_rows_1x128(x7.float().cpu().numpy())
    assert (q7.cpu().numpy() == rq).all() and (s7.cpu().numpy().view("u4") == rs.view("u4")).all()

    # Capture (torch warms the stream up first; the library needs nothing).
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()

    for replay in range(4):
        for c in outs:
            c.view(torch.uint8).fill_(0xFF)  # a fill kernel, outside the graph
        graph.replay()
        torch.cuda.synchronize()
        for k, (c, ref) in enumerate(zip(outs, eager)):
            assert torch.equal(_bits(c), ref), (replay, k)
        # eager work between replays, on the same buffers
        tg.gemm_bf16(a1, b1, None, c1)
        tg.gemm_bf16_ex(a2, b2, None, c2, workspace=ws2)
        tg.gemm_bf16_w8(x5, q5, s5, None, c5, workspace=ws5)
        torch.cuda.synchronize()
    # the FP8 split left its counters at zero
    cnt = ws3[: 4 * ((600 + 255) // 256) * ((700 + 255) // 256)].view(torch.int32)
    assert int(cnt.abs().sum()) == 0
    del graph
