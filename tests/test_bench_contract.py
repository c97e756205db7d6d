"""bench.py's output contract: one JSON line with the fields the benchmark
driver reads, and a refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, timeout):
    return subprocess.run([sys.executable, "bench.py", *args], cwd=ROOT, capture_output=True,
                          text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused():
    """No GPU is touched: the library has no multi-GPU path, and the bench says so."""
    r = _bench("--gpus", "2", timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.gpu
def test_one_block_line_carries_the_contract_fields():
    """A one-block run of the default workload: every field of the line, the
    roofline object of the dominant kernel, and the determinism check."""
    print("case: bench.py --blocks 1 --steps 1 --warmup 0 --no-cpu-baseline", flush=True)
    r = _bench("--blocks", "1", "--steps", "1", "--warmup", "0", "--no-cpu-baseline",
               timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["value"] > 0 and d["unit"] == "s" and d["higher_is_better"] is False
    assert d["n_gpus"] == 1 and d["steps"] == 1 and d["warmup"] == 0
    assert abs(d["ms_per_step"] / 1e3 - d["value"]) <= 1e-5 + 1e-3 * d["value"]
    assert d["scaling"] in ("weak", "strong")
    assert d["vs_baseline"] is None          # no published number for this workload
    assert d["dtype"] == "bf16" and d["data"] == "synthetic"
    assert isinstance(d["config"]["workload"], str) and d["config"]["blocks"] == 1
    assert d["cpu_baseline"] is None         # skipped on request
    rf = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in rf, key
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2500.0
    assert 0 < rf["frac"] < 1
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert rf["traffic"] is None or rf["traffic"] > 0
    assert d["determinism"]["identical"] is True
    pr = d["protocol"]
    assert pr["forwards"] == 1 and pr["step1_ms"] > 0 and pr["median_steps_2_8_ms"] is None
