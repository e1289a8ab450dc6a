"""bench.py's command-line contract, on the CPU.

The benchmark measures one GPU: asked for more (a --gpus count above one,
or a launcher's WORLD_SIZE above one) it prints one JSON line with an
"error" key and exits with status 2 before touching the GPU; with no GPU
visible it says so and exits with status 1 (it never falls back to the CPU).
"""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=300)
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    return r.returncode, lines


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), (["--gpus", "8", "--steps", "3"], None),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(args, env):
    rc, lines = _run(args, env)
    assert rc == 2
    assert len(lines) == 1
    msg = json.loads(lines[0])
    assert "one GPU" in msg["error"]


def test_no_gpu_is_an_error_not_a_cpu_run():
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible: bench.py would run the benchmark")
    rc, lines = _run(["--steps", "1", "--warmup", "0"])
    assert rc == 1
    assert json.loads(lines[-1]) == {"error": "no GPU visible"}
