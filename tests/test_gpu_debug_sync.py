"""MTA_DEBUG_SYNC=1: every call that launches work returns only after that
work is done, so a kernel failure is reported by the call that launched it
("Mica 7.7", section "Kernels ready at the start": the debug tier waits for
each kernel; section "Upgrading": without it a queued kernel's failure
surfaces when the program next waits on the device).  The variable is read once per
process, so each setting runs in a child process (tests/debug_sync_child.py)
that checks, after each call, whether the caller's stream is already idle,
and checks the results against the oracle.  Nothing here faults: the
contract is observed on calls that succeed."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

CHILD = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                     "debug_sync_child.py")
CALLS = ["mta_scale(in place)", "mta_clip_norm", "mta_adamw_step",
         "mta_amp_clip_norm", "mta_amp_adamw_step", "mta_amp_update"]


def _child(debug):
    env = dict(os.environ)
    env.pop("MTA_DEBUG_SYNC", None)
    if debug:
        env["MTA_DEBUG_SYNC"] = "1"
    r = subprocess.run([sys.executable, CHILD], env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    out = json.loads(r.stdout.strip().splitlines()[-1])
    assert out["parity"] is True
    return out["idle"]


def test_debug_sync_returns_with_the_stream_idle():
    idle = _child(debug=True)
    assert sorted(idle) == sorted(CALLS)
    assert all(idle.values()), idle


def test_without_debug_sync_calls_return_before_their_work_is_done():
    # the control: the same calls on the same list, without the variable;
    # the update kernels (about 0.1 ms of device work) are still running
    # when their calls return
    idle = _child(debug=False)
    assert sorted(idle) == sorted(CALLS)
    assert not idle["mta_adamw_step"] and not idle["mta_amp_adamw_step"], \
        idle
