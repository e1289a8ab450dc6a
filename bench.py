"""Benchmark of the GEMM hot path on one MI355X; prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload square]
                    [--no-secondary] [--no-cpu-baseline]

A step is one library call on the headline workload (the square bf16 GEMM
M = N = K = 4096, bf16 output) with all inputs resident in HBM.  W untimed
warm-up steps, then exactly K timed steps between two synchronisations;
value = 2*M*N*K / (time per step), in TFLOP/s (the FLOP count of the GEMM
compute-cost page, section 3.1; rates and utilisation are the "three numbers"
of the DeepGEMM page, section 3.4).

Also reported in the same line:
  roofline      the dominant kernel's launch time from HIP events on the
                launch stream (mean over the timed region; median and min from
                a second pass with one event pair per call), as achieved
                TFLOP/s (or GB/s, from the mean) against the MI355X dense
                peak, plus HBM traffic from the committed rocprofv3 counter
                summary when it matches the current source;
  clocks        shader and memory clocks read from the driver's sysfs before,
                during (sampled by a thread while the steps run) and after the
                timed region;
  cpu_baseline  the fp64 CPU oracle (the plain triple loop in C) timed on this
                host on a bounded row sample of the same workload, with its
                thread count, the host's CPU count and model, and the oracle's
                single-thread time on the 64^3 workload (rank 0, one GPU only);
  secondary     the other workloads (FFN pair, thin-M LM head at M = 1, 8,
                32, 64, FP8 block-scaled and its ragged variant, ...), each
                timed the same way with its own roofline figure, after at
                least SECONDARY_WARM_MS of untimed back-to-back calls (the
                first tens of milliseconds of calls after the idle gap in
                which a workload's inputs are built run at lower clocks: on
                MI355X the first 20 FP8 calls averaged 276 us, those after
                the first hundred 224 us, on the same buffers);
  probes        reference rates of this machine (MFMA-only loops on random
                register operands, a streaming read), informational only.
"""

import argparse
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "GEMM TFLOPS & % MFMA peak (bf16/fp8); HBM GB/s % peak on thin-M LM head"
PROFILES = os.path.join(ROOT, "profiles")
SECONDARY_WARM_MS = 50.0    # untimed back-to-back calls before a secondary's timing


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="square",
                    help="headline workload (square, ffn_up, ffn_down, thin_m1..64, fp8, fp8_ragged, "
                         "tiny, quant_a, quant_b, w8_m1..64, w4_m1..64, lsm_m1..64, square_nt, ffn_up_nt, ffn_down_nt, thin_nt_m1..64, ffn_up_q8, fp8_nt, fp8_ragged_nt, w8_lsm_m1/m64, w4_lsm_m1/m64)")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--secondary-steps", type=int, default=50)
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the reference-rate probes (MFMA loops, HBM stream read)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (the reference kernel for "
                         "scaling HBM byte counters) and exit")
    return ap.parse_args()


def calibrate_copy(steps=5):
    """A plain copy of known size: 2^30 bytes read and 2^30 bytes written per call."""
    import torch

    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read_per_call": n,
                      "bytes_written_per_call": n, "calls": steps}), flush=True)


def source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "tiled_gemm_04_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "tiled": ["common.h", "launch.h", "gemm_bf16_tiled.hip"],
    "thin": ["common.h", "launch.h", "gemm_bf16_thin.hip"],
    "fp8": ["common.h", "launch.h", "gemm_fp8_blockscaled.hip"],
    "quant": ["common.h", "launch.h", "quant_fp8.hip"],
    "w8": ["common.h", "launch.h", "gemm_wq_thin.hip"],
    "w4": ["common.h", "launch.h", "gemm_wq_thin.hip"],
    "lsm": ["common.h", "launch.h", "gemm_bf16_thin.hip"],
    "nt": ["common.h", "launch.h", "gemm_bf16_tiled.hip", "gemm_bf16_thin.hip"],
    "q8": ["common.h", "launch.h", "gemm_bf16_tiled.hip"],
    "wq_lsm": ["common.h", "launch.h", "gemm_wq_thin.hip", "gemm_bf16_thin.hip"],
}

# Weight-only int8 LM head: the thin-M workloads' X [M, 4096] times int8
# codes Q [4096, 128256] with fp32 scales per (128 rows, column).
W8_CASES = {"w8_m1": 1, "w8_m8": 8, "w8_m32": 32, "w8_m64": 64,
            "w4_m1": 1, "w4_m8": 8, "w4_m32": 32, "w4_m64": 64,
            # the same heads with bias and log-softmax fused (two kernels per call)
            "w8_lsm_m1": 1, "w8_lsm_m64": 64, "w4_lsm_m1": 1, "w4_lsm_m64": 64}

# FP8 quantisers, timed on the FP8 workload's unquantised operands (bf16):
# activations A [4096, 4096] in 1 x 128 groups, weights B [4096, 14336] in
# 128 x 128 blocks.
NT_CASES = {"square_nt": "square", "ffn_up_nt": "ffn_up", "ffn_down_nt": "ffn_down",
            "thin_nt_m1": "thin_m1", "thin_nt_m8": "thin_m8", "thin_nt_m32": "thin_m32",
            "thin_nt_m64": "thin_m64"}
# The FFN up-projection with the FP8 1 x 128 activation quantiser in its
# epilogue (codes + scales out, no bf16 output).
Q8_CASES = {"ffn_up_q8": "ffn_up"}
# The FP8 workloads with the weight stored [N, K] (K-contiguous).
FP8_NT_CASES = {"fp8_nt": "fp8", "fp8_ragged_nt": "fp8_ragged"}
LSM_CASES = {"lsm_m1": 1, "lsm_m8": 8, "lsm_m32": 32, "lsm_m64": 64}
QUANT_CASES = {"quant_a": ("a", "tgemm_quant_fp8_1x128"), "quant_b": ("b", "tgemm_quant_fp8_128x128")}


def committed_traffic(workload, family):
    """HBM bytes per launch from profiles/<workload>_pmc.md, or None.

    The summary holds lines 'source_digest: <hex>' and
    'hbm_bytes_per_launch: <int>'; the figure is used only while the digest
    matches the kernel's current source.
    """
    path = os.path.join(PROFILES, f"{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    dig = re.search(r"source_digest:\s*([0-9a-f]+)", text)
    val = re.search(r"hbm_bytes_per_launch:\s*([0-9]+)", text)
    if not dig or not val or dig.group(1) != source_digest(KERNEL_SOURCES[family]):
        return None
    return int(val.group(1))


class Case:
    """One workload: inputs resident on the GPU and a launch closure."""

    def __init__(self, name, dev):
        import torch

        import tiled_gemm_04_amd as tg
        import workloads as wl

        self.name = name
        if name in QUANT_CASES:
            self._init_quant(name, dev)
            return
        if name in W8_CASES:
            self._init_w8(name, dev)
            return
        if name in LSM_CASES:
            self._init_lsm(name, dev)
            return
        if name in NT_CASES:
            self._init_nt(name, dev)
            return
        if name in Q8_CASES:
            self._init_q8(name, dev)
            return
        if name in FP8_NT_CASES:
            self._init_fp8_nt(name, dev)
            return
        w = wl.WORKLOADS[name]
        self.w = w
        self.M, self.N, self.K = w.M, w.N, w.K
        self.flops = 2 * w.M * w.N * w.K
        if w.fp8:
            qa, sa, qb, sb = wl.fp8_inputs(w, device=dev)
            c = torch.empty(w.M, w.N, dtype=torch.bfloat16, device=dev)
            self.launch = lambda: tg.gemm_fp8_blockscaled(qa, sa, qb, sb, c)
            self.family = "fp8"
            self.kernel = tg.gemm_fp8_kernel_name(w.M, w.N, w.K)
            self.bytes = w.M * w.K + w.K * w.N + 2 * w.M * w.N + 4 * (sa.numel() + sb.numel())
            self.bound, self.peak = "mfma", PEAK_FP8_TFLOPS
            self.dtype = "fp8_e4m3"
        else:
            if name == "ffn_down":
                a = wl.ffn_hidden(w.M, w.K, w.seed, dev)
                _, b, bias = wl.bf16_inputs(w, device=dev)
            else:
                a, b, bias = wl.bf16_inputs(w, device=dev)
            out = torch.float32 if w.out_f32 else torch.bfloat16
            c = torch.empty(w.M, w.N, dtype=out, device=dev)
            self.launch = lambda: tg.gemm_bf16(a, b, bias, c, epilogue=w.epilogue)
            self.kernel = tg.gemm_bf16_kernel_name(w.M, w.N, w.K, w.epilogue,
                                                   tg.OUT_F32 if w.out_f32 else tg.OUT_BF16)  # gemm_bf16: no workspace
            self.family = "thin" if "thin" in self.kernel else "tiled"
            out_bytes = 4 if w.out_f32 else 2
            self.bytes = 2 * (w.M * w.K + w.K * w.N) + out_bytes * w.M * w.N + (
                2 * w.N if bias is not None else 0)
            thin = self.family == "thin"
            self.bound = "hbm" if thin else "mfma"
            self.peak = PEAK_HBM_GBS if thin else PEAK_BF16_TFLOPS
            self.dtype = "bf16"
        self.inputs_for_oracle = None if w.fp8 else (a, b)

    def describe(self):
        if self.family == "quant":
            grouping = "1x128" if self.name == "quant_a" else "128x128"
            return f"{self.name}: Q, S = quantize_fp8_{grouping}(X[{self.M},{self.N}] bf16)"
        if self.family == "wq_lsm":
            code = "int8" if self.name.startswith("w8") else "int4, two per byte"
            return (f"{self.name}: C[{self.M},{self.N}] = log_softmax(X[{self.M},{self.K}] . "
                    f"(Q[{self.K},{self.N}] {code} * S) + bias[{self.N}]) over each row")
        if self.family == "w8":
            return (f"{self.name}: C[{self.M},{self.N}] = X[{self.M},{self.K}] . "
                    f"(Q[{self.K},{self.N}] int8 * S[{(self.K + 127) // 128},{self.N}])")
        if self.name in FP8_NT_CASES:
            return (f"{self.name}: C[{self.M},{self.N}] = A[{self.M},{self.K}] . Bt[{self.N},{self.K}]^T "
                    f"(FP8 e4m3, 1x128 / 128x128 scales, weight K-contiguous)")
        if self.family == "q8":
            return (f"{self.name}: Q, S = quantize_fp8_1x128(gelu(A[{self.M},{self.K}] . "
                    f"B[{self.K},{self.N}] + bias)) in one kernel")
        if self.family == "nt":
            return (f"{self.name}: C[{self.M},{self.N}] = A[{self.M},{self.K}] . Bt[{self.N},{self.K}]^T "
                    f"(weight K-contiguous)")
        if self.family == "lsm":
            return (f"{self.name}: C[{self.M},{self.N}] = log_softmax(X[{self.M},{self.K}] . "
                    f"W[{self.K},{self.N}] + bias[{self.N}]) over each row")
        if self.family == "w4":
            return (f"{self.name}: C[{self.M},{self.N}] = X[{self.M},{self.K}] . "
                    f"(Q[{self.K},{self.N}] int4, two per byte * S[{(self.K + 127) // 128},{self.N}])")
        return f"{self.name}: C[{self.M},{self.N}] = A[{self.M},{self.K}] . B[{self.K},{self.N}]"

    def _init_w8(self, name, dev):
        import torch

        import tiled_gemm_04_amd as tg
        import workloads as wl

        w = wl.WORKLOADS["thin_m64"]
        M, N, K = W8_CASES[name], w.N, w.K
        x = wl.thin_x(w, M, dev)
        bits = 8 if name.startswith("w8") else 4
        q, s = (wl.w8_weights if bits == 8 else wl.w4_weights)(K, N, w.seed, dev)
        c = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        self.w = None
        self.M, self.N, self.K = M, N, K
        self.flops = 2 * M * N * K
        # X, the codes (K*N*bits/8 bytes), the scales and C, each once.
        self.bytes = 2 * M * K + q.numel() + 4 * s.numel() + 2 * M * N
        self.kernel = (tg.gemm_w8_kernel_name if bits == 8 else tg.gemm_w4_kernel_name)(M, N, K)
        self.family = "w8" if bits == 8 else "w4"
        if "_lsm_" in name:
            b = wl.bf16((N,), "normal", 0.02, w.seed, wl.T_BIAS, dev)
            ws = torch.empty(tg.gemm_logsoftmax_workspace_size(M, N, tg.OUT_BF16), dtype=torch.uint8,
                             device=dev)
            fn = tg.gemm_bf16_w8_logsoftmax if bits == 8 else tg.gemm_bf16_w4_logsoftmax
            self.launch = lambda: fn(x, q, s, b, c, workspace=ws)
            self.bytes += 2 * N  # the bias
            self.kernel = f"tgemm_wq_thin_lsm<{bits}, {(M + 15) // 16}>+tgemm_lsm_normalize"
            self.family = "wq_lsm"
        else:
            fn = tg.gemm_bf16_w8 if bits == 8 else tg.gemm_bf16_w4
            self.launch = lambda: fn(x, q, s, None, c)
        self.bound, self.peak = "hbm", PEAK_HBM_GBS
        self.dtype = "bf16 x int8" if bits == 8 else "bf16 x int4"
        self.inputs_for_oracle = None

    def _init_nt(self, name, dev):
        import torch

        import tiled_gemm_04_amd as tg
        import workloads as wl

        w = wl.WORKLOADS[NT_CASES[name]]
        a, b, bias = wl.bf16_inputs(w, device=dev)
        if w.name.startswith("thin"):
            a = wl.thin_x(w, w.M, dev)
        bt = b.t().contiguous()  # the same weight, stored [N, K]
        del b
        c = torch.empty(w.M, w.N, dtype=torch.bfloat16, device=dev)
        self.launch = lambda: tg.gemm_bf16_nt(a, bt, bias, c, epilogue=w.epilogue)
        self.w = None
        self.M, self.N, self.K = w.M, w.N, w.K
        self.flops = 2 * w.M * w.N * w.K
        self.bytes = 2 * (w.M * w.K + w.K * w.N) + 2 * w.M * w.N + (2 * w.N if w.epilogue else 0)
        self.kernel = tg.gemm_bf16_nt_kernel_name(w.M, w.N, w.K)
        self.family = "nt"
        thin = w.name.startswith("thin")
        self.bound, self.peak = ("hbm", PEAK_HBM_GBS) if thin else ("mfma", PEAK_BF16_TFLOPS)
        self.dtype = "bf16"
        self.inputs_for_oracle = None

    def _init_fp8_nt(self, name, dev):
        import torch

        import tiled_gemm_04_amd as tg
        import workloads as wl

        w = wl.WORKLOADS[FP8_NT_CASES[name]]
        qa, sa, qb, sb = wl.fp8_inputs(w, device=dev)
        bt = qb.t().contiguous()
        del qb
        c = torch.empty(w.M, w.N, dtype=torch.bfloat16, device=dev)
        self.launch = lambda: tg.gemm_fp8_blockscaled_nt(qa, sa, bt, sb, c)
        self.w = None
        self.M, self.N, self.K = w.M, w.N, w.K
        self.flops = 2 * w.M * w.N * w.K
        self.bytes = w.M * w.K + w.K * w.N + 2 * w.M * w.N + 4 * (sa.numel() + sb.numel())
        self.kernel = "tgemm_fp8_bs_nt_256x256x128"
        self.family = "fp8"
        self.bound, self.peak = "mfma", PEAK_FP8_TFLOPS
        self.dtype = "fp8_e4m3"
        self.inputs_for_oracle = None

    def _init_q8(self, name, dev):
        import torch

        import tiled_gemm_04_amd as tg
        import workloads as wl

        w = wl.WORKLOADS[Q8_CASES[name]]
        a, b, bias = wl.bf16_inputs(w, device=dev)
        G = (w.N + 127) // 128
        q = torch.empty(w.M, w.N, dtype=torch.uint8, device=dev)
        s = torch.empty(w.M, G, dtype=torch.float32, device=dev)
        self.launch = lambda: tg.gemm_bf16_quant_fp8(a, b, bias, q, s, epilogue=w.epilogue)
        self.w = None
        self.M, self.N, self.K = w.M, w.N, w.K
        self.flops = 2 * w.M * w.N * w.K
        # A, B, bias read once; codes (1 byte each) and scales written once.
        self.bytes = 2 * (w.M * w.K + w.K * w.N) + 2 * w.N + w.M * w.N + 4 * w.M * G
        self.kernel = tg.gemm_bf16_kernel_name(w.M, w.N, w.K, w.epilogue, tg.OUT_BF16).replace(
            "tgemm_bf16_tiled_", "tgemm_bf16_tiled_q8_")
        self.family = "q8"
        self.bound, self.peak = "mfma", PEAK_BF16_TFLOPS
        self.dtype = "bf16"
        self.inputs_for_oracle = None

    def _init_lsm(self, name, dev):
        import torch

        import tiled_gemm_04_amd as tg
        import workloads as wl

        w = wl.WORKLOADS["thin_m64"]
        M, N, K = LSM_CASES[name], w.N, w.K
        x = wl.thin_x(w, M, dev)
        _, wt, _ = wl.bf16_inputs(w, device=dev, rows=1)
        b = wl.bf16((N,), "normal", 0.02, w.seed, wl.T_BIAS, dev)
        c = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        ws = torch.empty(tg.gemm_logsoftmax_workspace_size(M, N), dtype=torch.uint8, device=dev)
        self.launch = lambda: tg.gemm_bf16_logsoftmax(x, wt, b, c, workspace=ws)
        self.w = None
        self.M, self.N, self.K = M, N, K
        self.flops = 2 * M * N * K
        # X, W, bias and the log-probabilities, each once (the logits never
        # leave the chip).
        self.bytes = 2 * M * K + 2 * K * N + 2 * N + 2 * M * N
        self.kernel = f"tgemm_bf16_thin_lsm<{(M + 15) // 16}>+tgemm_lsm_normalize"
        self.family = "lsm"
        self.bound, self.peak = "hbm", PEAK_HBM_GBS
        self.dtype = "bf16"
        self.inputs_for_oracle = None

    def _init_quant(self, name, dev):
        import torch

        import tiled_gemm_04_amd as tg
        import workloads as wl

        operand, self.kernel = QUANT_CASES[name]
        a, b = wl.fp8_sources_bf16(wl.WORKLOADS["fp8"], device=dev)
        x = a if operand == "a" else b
        del a, b
        R, C = x.shape
        q = torch.empty(R, C, dtype=torch.float8_e4m3fn, device=dev)
        if operand == "a":
            s = torch.empty(R, (C + 127) // 128, dtype=torch.float32, device=dev)
            self.launch = lambda: tg.quantize_fp8_1x128(x, q, s)
        else:
            s = torch.empty((R + 127) // 128, (C + 127) // 128, dtype=torch.float32, device=dev)
            self.launch = lambda: tg.quantize_fp8_128x128(x, q, s)
        self.w = None
        self.M, self.N, self.K = R, C, 0
        self.flops = 0
        self.bytes = 2 * R * C + R * C + 4 * s.numel()  # read bf16, write codes and scales
        self.family = "quant"
        self.bound, self.peak = "hbm", PEAK_HBM_GBS
        self.dtype = "bf16->fp8_e4m3"
        self.inputs_for_oracle = None

    def time(self, steps, warmup, clocks=False, warm_ms=0.0):
        """Timing of `steps` back-to-back calls after `warmup` untimed ones.

        warm_ms > 0: after those, untimed calls continue in batches of ten
        until warm_ms of wall-clock time has passed, so that the timing
        starts from the clocks of sustained load.

        The timed region (bracketed by two synchronisations) enqueues the
        calls with one pair of HIP events around all of them on the launch
        stream (torch's current stream, which the binding launches on):
        ms_per_step is its wall-clock time per call, kernel_ms_mean the
        events' time per call.  A second pass of `steps` calls, each between
        its own pair of events, gives the per-call median and minimum (an
        event pair per call adds queue gaps, so it is kept out of the timed
        region).  With clocks, the driver's shader / memory clock is sampled
        from sysfs by a thread before, during and after the timed region.
        """
        import threading

        import torch

        for _ in range(warmup):
            self.launch()
        torch.cuda.synchronize()
        if warm_ms > 0:
            t_warm = time.perf_counter()
            while (time.perf_counter() - t_warm) * 1e3 < warm_ms:
                for _ in range(10):
                    self.launch()
                torch.cuda.synchronize()
        region = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        samples, stop = [], threading.Event()

        def poll():
            while not stop.is_set():
                r = read_clocks()
                if r:
                    samples.append(r)
                stop.wait(0.0005)

        clk = {"before": read_clocks()} if clocks else None
        poller = threading.Thread(target=poll, daemon=True) if clocks else None
        torch.cuda.synchronize()
        if poller:
            poller.start()
        t0 = time.perf_counter()
        region[0].record()
        for _ in range(steps):
            self.launch()
        region[1].record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        if poller:
            stop.set()
            poller.join()
            clk["after"] = read_clocks()
            clk["during"] = summarize_clocks(samples)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for e0, e1 in ev:
            e0.record()
            self.launch()
            e1.record()
        torch.cuda.synchronize()
        per = [e0.elapsed_time(e1) for e0, e1 in ev]
        return {"ms_per_step": (t1 - t0) * 1e3 / steps,
                "kernel_ms_mean": region[0].elapsed_time(region[1]) / steps,
                "kernel_ms_median": statistics.median(per), "kernel_ms_min": min(per),
                "kernel_ms_per_call_mean": statistics.fmean(per), "clocks": clk}

    def roofline(self, t):
        """Roofline entry from a time() result: achieved from the mean kernel time."""
        def rate(ms):
            if self.bound == "hbm":
                return self.bytes / (ms * 1e-3) / 1e9
            return self.flops / (ms * 1e-3) / 1e12

        achieved = rate(t["kernel_ms_mean"])
        traffic = committed_traffic(self.name, self.family)
        return {"bound": self.bound, "achieved": round(achieved, 2), "peak": self.peak,
                "unit": "GB/s" if self.bound == "hbm" else "TFLOP/s",
                "frac": round(achieved / self.peak, 4), "traffic": traffic,
                "kernel": self.kernel, "kernel_ms_mean": round(t["kernel_ms_mean"], 5),
                "kernel_ms_median": round(t["kernel_ms_median"], 5),
                "kernel_ms_min": round(t["kernel_ms_min"], 5),
                "kernel_ms_timing": "mean: one HIP event pair around the timed region / steps; "
                                    "median and min: a second pass with one event pair per call",
                "achieved_at_median": round(rate(t["kernel_ms_median"]), 2),
                "algorithmic_bytes": self.bytes, "flop": self.flops}


def read_clocks():
    """Current shader and memory clocks (MHz) of the visible GPU from the
    amdgpu driver's sysfs files (the level marked '*' in pp_dpm_sclk /
    pp_dpm_mclk, and the hwmon sclk reading when present), or None.  With
    several cards listed, the one whose PCI address matches torch's device 0
    is used when torch reports it, else the first readable one."""
    cards = sorted(glob.glob("/sys/class/drm/card[0-9]*/device"))
    want = None
    try:
        import torch

        props = torch.cuda.get_device_properties(0)
        bus = getattr(props, "pci_bus_id", None)
        dom = getattr(props, "pci_domain_id", 0) or 0
        dev_ = getattr(props, "pci_device_id", None)
        if bus is not None and dev_ is not None:
            want = f"{dom:04x}:{bus:02x}:{dev_:02x}."
    except Exception:  # clocks are informational
        want = None
    for card in cards:
        real = os.path.realpath(card)
        if want is not None and want not in real:
            continue
        out = {}
        for key, fname in (("sclk_mhz", "pp_dpm_sclk"), ("mclk_mhz", "pp_dpm_mclk")):
            try:
                with open(os.path.join(card, fname)) as fh:
                    for line in fh:
                        if line.rstrip().endswith("*"):
                            m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                            if m:
                                out[key] = int(m.group(1))
            except OSError:
                pass
        for f in glob.glob(os.path.join(card, "hwmon", "hwmon*", "freq1_input")):
            try:
                with open(f) as fh:
                    out["sclk_hwmon_mhz"] = round(int(fh.read().strip()) / 1e6)
            except (OSError, ValueError):
                pass
        if out:
            out["card"] = os.path.basename(os.path.dirname(card))
            return out
    return None


def summarize_clocks(samples):
    """min / median / max of the sampled clocks and the sample count."""
    out = {"samples": len(samples)}
    for key in ("sclk_mhz", "mclk_mhz"):
        vals = sorted(r[key] for r in samples if key in r)
        if vals:
            out[key] = {"min": vals[0], "median": vals[len(vals) // 2], "max": vals[-1]}
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(case, dev, budget_s=12.0):
    """The fp64 oracle, as it stands, on a bounded sample of the headline workload.

    The oracle decodes the bf16 inputs and runs the plain k-ascending triple
    loop in C (oracle/contract.c) on its worker threads.  The sample is the
    first rows of A that take about a quarter of budget_s (the whole GEMM if
    it fits), repeated until about budget_s seconds have been spent.  Also
    timed: one call on the 64 x 64 x 64 workload with one thread.  Reported
    value: oracle FLOP/s in TFLOP/s.
    """
    import workloads as wl
    from oracle import gemm as og
    from oracle import native

    threads = native.default_threads()
    tiny = wl.WORKLOADS["tiny"]
    ta, tb, _ = wl.bf16_inputs(tiny, device=dev)
    ta_bits, tb_bits = wl.bits_u16(ta), wl.bits_u16(tb)
    og.gemm_bf16_bits(ta_bits, tb_bits, threads=1)  # builds / loads the library
    t0 = time.perf_counter()
    reps_tiny = 20
    for _ in range(reps_tiny):
        og.gemm_bf16_bits(ta_bits, tb_bits, threads=1)
    tiny_ms = (time.perf_counter() - t0) * 1e3 / reps_tiny

    a, b = case.inputs_for_oracle
    a_bits = wl.bits_u16(a)
    b_bits = wl.bits_u16(b)
    rows = min(case.M, 16)
    t0 = time.perf_counter()
    og.gemm_bf16_bits(a_bits[:rows], b_bits)
    probe = time.perf_counter() - t0
    while rows < case.M and probe < budget_s / 4:
        rows = min(case.M, rows * 2)
        t0 = time.perf_counter()
        og.gemm_bf16_bits(a_bits[:rows], b_bits)
        probe = time.perf_counter() - t0
    reps = max(1, int(budget_s // max(probe, 1e-3)))
    t0 = time.perf_counter()
    for _ in range(reps):
        og.gemm_bf16_bits(a_bits[:rows], b_bits)
    dt = time.perf_counter() - t0
    flops = 2 * rows * case.N * case.K * reps
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(dt, 3),
            "host_cpus": os.cpu_count(), "affinity_cpus": affinity, "cpu_model": cpu_model(),
            "single_thread_tiny_ms": round(tiny_ms, 3),
            "sample": f"{reps} x rows 0..{rows - 1} of the {case.M}x{case.N}x{case.K} {case.name} "
                      f"GEMM on {threads} threads (bf16 decode + plain fp64 k-ascending loop with "
                      f"|a||b| denominators); single_thread_tiny_ms: the 64x64x64 workload on one "
                      f"thread"}


def measure_probes(dev):
    """Reference rates of this machine (informational, not bounds): the library's
    MFMA-only loops on random register operands and its streaming read of a
    1 GiB buffer (beyond the 256 MB last-level cache), each the best of three
    timed calls after one warm-up, HIP events on the launch stream.  A tuned
    kernel can exceed them (the LM head reads faster than the stream probe)."""
    import torch

    import tiled_gemm_04_amd as tg

    def best(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1) / 1e3)
        return min(t)

    out = {}
    iters = 2000
    buf = torch.empty(tg.gemm_probe_out_elems(tg.PROBE_MFMA_BF16), dtype=torch.float32, device=dev)
    for key, probe in (("mfma_bf16_loop_tflops", tg.PROBE_MFMA_BF16),
                       ("mfma_fp8_loop_tflops", tg.PROBE_MFMA_FP8)):
        sec = best(lambda: tg.gemm_probe_mfma(probe, iters, buf))
        out[key] = round(tg.gemm_probe_mfma_flop(probe, iters) / sec / 1e12, 1)
    src = torch.ones(1 << 28, dtype=torch.int32, device=dev)  # 1 GiB
    xo = torch.empty(tg.gemm_probe_out_elems(tg.PROBE_STREAM_READ), dtype=torch.int32, device=dev)
    sec = best(lambda: tg.gemm_probe_stream_read(src, xo))
    out["stream_read_gbs"] = round((1 << 30) / sec / 1e9, 1)
    out["note"] = ("reference rates on this box (MFMA-only loops on random register operands, a "
                   "1 GiB streaming read), informational; not bounds")
    del buf, src, xo
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the GEMM is measured "
                                   "on one device's share (multi-GPU sharding is not built)"}))
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        calibrate_copy()
        return

    head = Case(args.workload, dev)
    t = head.time(args.steps, args.warmup, clocks=True)
    ms_step = t["ms_per_step"]
    value = head.flops / (ms_step * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head.dtype,
        "data": "synthetic (seeded, shapes and distributions of the source pages' workloads)",
        "config": {"workload": head.describe(), "M": head.M, "N": head.N, "K": head.K,
                   "kernel": head.kernel},
        "roofline": head.roofline(t),
        "clocks": t["clocks"],
        "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
    }
    del head.launch
    torch.cuda.empty_cache()

    if not args.no_secondary:
        sec = {}
        for name in ("ffn_up", "ffn_down", "thin_m1", "thin_m8", "thin_m32", "thin_m64", "fp8",
                     "fp8_ragged", "tiny", "quant_a", "quant_b", "w8_m1", "w8_m8", "w8_m32",
                     "w8_m64", "w4_m1", "w4_m8", "w4_m32", "w4_m64", "lsm_m1", "lsm_m8", "lsm_m32",
                     "lsm_m64", "square_nt", "ffn_up_nt", "ffn_down_nt", "thin_nt_m1",
                     "thin_nt_m8", "thin_nt_m32", "thin_nt_m64", "ffn_up_q8", "fp8_nt",
                     "fp8_ragged_nt", "w8_lsm_m1", "w8_lsm_m64", "w4_lsm_m1", "w4_lsm_m64"):
            if name == args.workload:
                continue
            c = Case(name, dev)
            tc = c.time(args.secondary_steps, 5, warm_ms=SECONDARY_WARM_MS)
            r = c.roofline(tc)
            sec[name] = {"ms_per_call": round(tc["ms_per_step"], 5),
                         "kernel_ms_mean": r["kernel_ms_mean"], "kernel_ms_median": r["kernel_ms_median"],
                         "kernel_ms_min": r["kernel_ms_min"],
                         "tflops": round(c.flops / (tc["kernel_ms_mean"] * 1e-3) / 1e12, 2),
                         "gbs": round(c.bytes / (tc["kernel_ms_mean"] * 1e-3) / 1e9, 1),
                         "bound": r["bound"], "frac": r["frac"], "kernel": c.kernel,
                         "traffic": r["traffic"]}
            del c
            torch.cuda.empty_cache()
        line["secondary"] = sec

    # The probes run last, so their heat and power draw do not colour the
    # measurements above.
    if not args.no_probes:
        line["probes"] = measure_probes(dev)

    if not args.no_cpu_baseline and head.inputs_for_oracle is not None:
        line["cpu_baseline"] = cpu_baseline(head, dev)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
