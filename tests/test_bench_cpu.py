"""bench.py's contract and bookkeeping, checked without a GPU: the one-GPU
refusal, the algorithmic bytes per parameter of every update rule and type
combination, the --no-decay selection on the GPT-2 layouts, and the lookup
of counter traffic (present only for the kernel source it was taken on)."""
import json
import os
import subprocess
import sys

import pytest

import bench
from mixed_precision_optimizer_mta_amd import workloads as WL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                        "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("name,update", [
    ("gpt2_124m", 28), ("gpt2_124m_bf16g", 26), ("gpt2_124m_f16amp", 26),
    ("gpt2_xl", 20), ("ragged", 22), ("tiny", 28)])
def test_update_bytes_per_param(name, update):
    # read w, g, m, v and write w, m, v, at each buffer's element size
    wl = WL.get(name)
    assert bench.update_bytes(wl, "adamw", False, None) == update
    assert bench.update_bytes(wl, "adam", False, None) == update
    gb = 4 if wl.gtype == WL.F32 else 2
    # zeroing writes g once more; a 16-bit weight copy writes 2 bytes
    assert bench.update_bytes(wl, "adamw", True, "bf16") == update + gb + 2


def test_other_rules_bytes_per_param():
    wl = WL.get("gpt2_124m")
    assert bench.update_bytes(wl, "sgd", False, None) == 12       # w, g; w
    assert bench.update_bytes(wl, "momentum", False, None) == 20  # + buf


@pytest.mark.parametrize("name,flagged,largest,smallest_kept", [
    ("gpt2_124m", 60, 3072, 589824), ("gpt2_xl", 240, 6400, 1638400)])
def test_no_decay_selects_the_biases_and_gains(name, flagged, largest,
                                               smallest_kept):
    # five 1-D tensors per layer (the [d, 2] layer-norm pair and four
    # biases), no weight matrix and no embedding
    sizes = WL.get(name).sizes
    picked = [n for n in sizes if n < bench.NO_DECAY_BELOW]
    layers = (len(sizes) - 2) // 9
    assert len(picked) == flagged == 5 * layers
    assert max(picked) == largest
    assert min(n for n in sizes if n >= bench.NO_DECAY_BELOW) == \
        smallest_kept


def test_traffic_is_reported_only_for_the_profiled_source(tmp_path,
                                                          monkeypatch):
    src = tmp_path / "kernels.hip"
    src.write_text("// one version of the kernels\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    sha = bench.kernel_source_sha()
    table = {"gpt2_124m": {"k_adamw": {"kernel_source_sha": sha,
                                       "bytes_per_launch": 123.0}}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(table))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("gpt2_124m", "k_adamw") == 123.0
    assert bench.measured_traffic("gpt2_124m", "k_sumsq") is None
    assert bench.measured_traffic("ragged", "k_adamw") is None
    src.write_text("// the kernels changed since the counters were taken\n")
    assert bench.measured_traffic("gpt2_124m", "k_adamw") is None


def test_traffic_keys():
    wl = WL.get("gpt2_124m")
    assert bench.traffic_key(wl, "adamw", False) == "gpt2_124m"
    assert bench.traffic_key(wl, "adam", False) == "gpt2_124m+adam"
    assert bench.traffic_key(wl, "sgd", True) == "gpt2_124m+sgd+zero"


def test_defaults_run_the_largest_single_gpu_workload():
    args = bench.make_parser().parse_args([])
    assert args.workload == "gpt2_xl"
    assert (args.gpus, args.torch_reference, args.probes) == (1, False,
                                                              False)
    assert args.cpu_steps is None
    # about 20 s of one host core, from the first step's time: a 14 s step
    # (the 1.56B packed list) is the whole sample, a 0.36 s one (the 124M
    # list) gives 56, a tiny list stops at 60
    assert bench.cpu_steps_after(14.4) == 1
    assert bench.cpu_steps_after(30.0) == 1
    assert bench.cpu_steps_after(0.36) == 56
    assert bench.cpu_steps_after(1e-4) == 60


def test_cpu_baseline_default_sample_is_timed_from_the_first_step():
    wl = WL.get("tiny")
    arena = WL.Arena(wl, "cpu")
    arena.fill_weights()
    arena.fill_grads(1)
    r = bench.cpu_baseline(arena, wl, None)
    assert 1 <= r["steps"] <= 60 and r["cores"] == 1
    assert r["sample"].startswith(f"{r['steps']} whole steps")
    r = bench.cpu_baseline(arena, wl, 3)
    assert r["steps"] == 3
