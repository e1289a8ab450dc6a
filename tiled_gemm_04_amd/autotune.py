"""Offline autotune sweep of the bf16 GEMM's kernel choice.

Usage: python -m tiled_gemm_04_amd.autotune [--out report.json] [--iters N]

For each problem shape it times every kernel the library can run for it
(the thin-M kernel when M <= 64, and the tiled kernel with each of its tile
shapes) through gemm_bf16_ex, next to the automatic choice (ALGO_AUTO), and
reports which is fastest and how far the automatic choice is from it.  The
shapes are the linear layers of the GEMM compute-cost page (section 2.1:
attention projections, the FFN pair, the LM head) at decode and prefill
batch sizes.  The sweep only measures; the shape table it checks lives in
the library (abi.cpp, pick_tiled_shape and the thin-M threshold).
"""

import argparse
import json

import torch

from . import binding as tg

SHAPES = [
    # (M, N, K)
    (1, 4096, 4096), (8, 4096, 4096), (64, 4096, 4096), (1, 14336, 4096), (16, 16384, 4096),
    (1, 4096, 14336), (32, 32768, 4096), (1, 65536, 4096), (128, 4096, 4096), (512, 4096, 4096),
    (2048, 4096, 4096), (4096, 4096, 4096), (8192, 4096, 4096),
    (128, 16384, 4096), (512, 16384, 4096), (2048, 16384, 4096),
    (128, 4096, 16384), (512, 4096, 16384), (2048, 4096, 16384),
    (64, 128256, 4096), (256, 128256, 4096),
    (1024, 1024, 1024), (1000, 3000, 500),
]

CANDIDATES = [
    ("thin", tg.ALGO_THIN), ("tiled_256x256", tg.ALGO_TILED_256x256),
    ("tiled_256x128", tg.ALGO_TILED_256x128), ("tiled_128x128", tg.ALGO_TILED_128x128),
]


def time_call(fn, iters, warmup=3, repeats=3):
    """Best over `repeats` of the mean over `iters` back-to-back calls (ms)."""
    for _ in range(warmup):
        fn()
    best = float("inf")
    for _ in range(repeats):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(iters):
            fn()
        e.record()
        torch.cuda.synchronize()
        best = min(best, s.elapsed_time(e) / iters)
    return best


def sweep(shapes=SHAPES, iters=10, seed=7):
    dev = torch.device("cuda")
    g = torch.Generator(device=dev).manual_seed(seed)
    rows = []
    for M, N, K in shapes:
        a = torch.randn(M, K, generator=g, device=dev).to(torch.bfloat16)
        b = (torch.randn(K, N, generator=g, device=dev) * 0.02).to(torch.bfloat16)
        c = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        flop = 2.0 * M * N * K
        # The automatic choice with the workspace its split-K asks for (the
        # candidates are timed as gemm_bf16 would run them, unsplit).
        need = tg.gemm_bf16_workspace_size(M, N, K)
        ws = torch.empty(need, dtype=torch.uint8, device=dev) if need > 0 else None
        times = {}
        for name, algo in CANDIDATES:
            if algo == tg.ALGO_THIN and M > 64:
                continue
            times[name] = time_call(lambda: tg.gemm_bf16_ex(a, b, None, c, algo=algo), iters)
        t_auto = time_call(lambda: tg.gemm_bf16_ex(a, b, None, c, algo=tg.ALGO_AUTO, workspace=ws), iters)
        best = min(times, key=times.get)
        auto_kernel = tg.gemm_bf16_kernel_name(M, N, K, with_workspace=ws is not None)
        rows.append({
            "M": M, "N": N, "K": K, "auto_kernel": auto_kernel, "auto_ms": round(t_auto, 5),
            "auto_tflops": round(flop / t_auto / 1e9, 1),
            "candidates_ms": {k: round(v, 5) for k, v in times.items()},
            "best": best, "best_ms": round(times[best], 5),
            "auto_vs_best": round(t_auto / times[best], 3),
        })
        del a, b, c, ws
        print(f"M={M:5d} N={N:6d} K={K:5d}  auto {auto_kernel:30s} {t_auto * 1e3:8.1f} us  "
              f"best {best:14s} {times[best] * 1e3:8.1f} us  ratio {t_auto / times[best]:.3f}", flush=True)
    return rows


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=None, help="write the report as JSON here")
    ap.add_argument("--iters", type=int, default=10)
    args = ap.parse_args(argv)
    rows = sweep(iters=args.iters)
    worst = max(r["auto_vs_best"] for r in rows)
    print(f"largest automatic-choice slowdown against the best candidate: {worst:.3f}x")
    if args.out:
        with open(args.out, "w") as fh:
            json.dump({"device": torch.cuda.get_device_name(0), "rows": rows}, fh, indent=1)


if __name__ == "__main__":
    main()
