"""bench.py's output contract on a GPU: one JSON line on stdout whose fields
agree with each other (throughput, step time, roofline fraction) for a small
and an 8-bit list, run as a separate process the way a driver runs it."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), *args, "--no-cpu-baseline"]
    print("case: bench", " ".join(args), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True,
                         timeout=110, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [l for l in res.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, res.stdout[-2000:]
    return json.loads(lines[0])


@pytest.mark.parametrize("args, workload, params", [
    (("--workload", "tiny", "--steps", "50", "--warmup", "5"), "tiny", 525_315),
    (("--workload", "lora_q8", "--steps", "10", "--warmup", "5"), "lora_q8", 24_313_856),
])
def test_bench_line_fields_agree(args, workload, params):
    d = _run(*args)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "kernel_ms"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == int(args[3]) and d["warmup"] == int(args[5])
    assert d["config"]["workload"] == workload and d["config"]["params"] == params
    assert d["higher_is_better"] is True and d["unit"] == "params/s"
    # value is whole-job params per second over the timed wall-clock steps
    assert d["value"] == pytest.approx(params / (d["ms_per_step"] / 1e3), rel=1e-6)
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-9)
    # achieved: algorithmic bytes over the event-timed average launch
    assert r["achieved"] == pytest.approx(
        r["algorithmic_bytes_per_launch"] / (d["kernel_ms"]["avg"] / 1e3) / 1e9, rel=1e-6)
    assert 0.0 < r["frac"] < 1.0
    assert r["traffic"] is None or isinstance(r["traffic"], int)
    k = d["kernel_ms"]
    assert 0.0 < k["per_step_min"] <= k["per_step_median"] <= k["per_step_max"]
