"""bench.py end to end on the GPU: one run on the tiny list, in a child
process, must print exactly one JSON line carrying every field of the
benchmark's contract (the step's metric and throughput, the roofline of the
dominant kernel, the oracle's CPU baseline and the workload's config)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(300)
def test_bench_prints_one_complete_json_line():
    r = subprocess.run(
        [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny",
         "--steps", "20", "--warmup", "2", "--cpu-steps", "1",
         "--no-ceiling"],
        capture_output=True, text=True, timeout=280, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup",
              "ms_per_step", "higher_is_better", "scaling", "vs_baseline",
              "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert (d["n_gpus"], d["steps"], d["warmup"]) == (1, 20, 2)
    assert d["unit"] == "params/s" and d["higher_is_better"] is True
    assert d["value"] > 0 and d["ms_per_step"] > 0
    # value is the whole job's params per second over the timed steps
    n = d["config"]["params"]
    assert abs(d["value"] - n / (d["ms_per_step"] * 1e-3)) <= 1e-6 * d["value"]
    assert d["config"]["workload"] == "tiny"
    rl = d["roofline"]
    assert rl["bound"] == "hbm" and rl["unit"] == "GB/s"
    assert rl["peak"] == 8000.0
    assert abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-12
    assert 0 < rl["frac"] < 1
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] == 1
    assert cb["value"] > 0 and cb["unit"] == "params/s"
    assert cb["steps"] == 1 and cb["sample"].startswith("1 whole steps")
