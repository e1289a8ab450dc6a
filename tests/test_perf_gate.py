"""Performance regression gate: each headline workload must keep at least
the throughput floor committed in tests/perf_floors.json (about 80 % of what
one MI355X measured, so box-to-box spread does not trip it).

Opt-in: marked ``perf`` (run with ``pytest -m perf`` on a GPU); skipped
without one.  The timing is the benchmark's own for its secondary workloads
(bench.Case: warm-up calls, then untimed back-to-back calls for
bench.SECONDARY_WARM_MS, then one pair of HIP events around the timed
back-to-back launches, mean); HBM-bound workloads are measured in GB/s of
algorithmic bytes, MFMA-bound ones in TFLOP/s.
"""

import json
import os

import pytest
import torch

pytestmark = pytest.mark.perf

FLOORS = json.load(open(os.path.join(os.path.dirname(__file__), "perf_floors.json")))
WORKLOADS = sorted(k for k in FLOORS if not k.startswith("_"))


@pytest.mark.parametrize("name", WORKLOADS)
def test_throughput_floor(name):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench

    case = bench.Case(name, torch.device("cuda"))
    kern_ms = case.time(20, 3, warm_ms=bench.SECONDARY_WARM_MS)["kernel_ms_mean"]
    if case.bound == "hbm":
        value, unit = case.bytes / kern_ms / 1e6, "GB/s"
    else:
        value, unit = case.flops / kern_ms / 1e9, "TFLOP/s"
    print(f"[perf] {name}: {value:.1f} {unit} (floor {FLOORS[name]})", flush=True)
    del case
    torch.cuda.empty_cache()
    assert value >= FLOORS[name], f"{name}: {value:.1f} {unit} below the floor {FLOORS[name]}"
