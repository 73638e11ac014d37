"""The C boundary used from C: tests/c/abi_demo (gcc, include/mta.h, no
Python) runs three deferred-unscale + clip + AdamW steps on the GPU; every
norm, coefficient and final w, m, v element it prints is checked against the
CPU oracle fed the same exact inputs (lockstep on the device coefficient,
the norm within 1e-6 relative, the rest bit for bit)."""
import os
import subprocess

import numpy as np
import pytest

import oracle as O

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c",
                   "abi_demo")
SIZES = [4096 * 2 + 5, 777, 1]


def _inputs(t=None):
    total = sum(SIZES)
    i = np.arange(total, dtype=np.int64)
    if t is None:
        return ((i * 37) % 101 - 50).astype(np.float32) / np.float32(1024)
    return ((i * 53 + t * 11) % 97 - 48).astype(np.float32) / np.float32(2048)


def _split(x):
    out, o = [], 0
    for n in SIZES:
        out.append(np.ascontiguousarray(x[o:o + n]))
        o += n
    return out


def test_c_program_matches_the_oracle():
    assert os.path.exists(EXE), (
        f"{EXE} is not built: run tests/c/build.py (or "
        "__graft_entry__.build()) first")
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    lines = r.stdout.strip().splitlines()
    steps = [ln.split() for ln in lines if ln.startswith("step")]
    assert len(steps) == 3
    ts = [O.Tensor(w, np.zeros(n, np.float32), np.zeros(n, np.float32),
                   np.zeros(n, np.float32))
          for w, n in zip(_split(_inputs()), SIZES)]
    for t, row in enumerate(steps, start=1):
        nrm = np.uint32(int(row[3], 16)).view(np.float32)
        coef = np.uint32(int(row[5], 16)).view(np.float32)
        for x, g in zip(ts, _split(_inputs(t))):
            x.g = g
        want = O.norm([x.g for x in ts], O.F32, 0.5)
        assert abs(float(nrm) - want) <= 1e-6 * want, (t, float(nrm), want)
        assert coef == O.clip_coef(0.05, nrm)
        assert coef < 1.0          # the clip is active in this run
        O.step_(ts, O.F32, 0, 0, 1e-3, 0.9, 0.999, 1e-8, 0.1, t, s=0.5,
                coef=coef)
    got = {}
    for ln in lines:
        parts = ln.split()
        if parts[0] in ("w", "m", "v"):
            got[(parts[0], int(parts[1]))] = np.array(
                [int(h, 16) for h in parts[2:]], dtype=np.uint32)
    for k, x in enumerate(ts):
        for name, buf in (("w", x.w), ("m", x.m), ("v", x.v)):
            assert np.array_equal(got[(name, k)], buf.view(np.uint32)), (
                name, k)
