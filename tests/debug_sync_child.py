"""Child process of test_gpu_debug_sync.py (not a test module itself).

Runs every device call of the library once on a side stream over a list
large enough that its kernels take tens of microseconds, and reports, for
each call, whether that stream was already idle when the call returned
(hipStreamQuery through torch.cuda.Stream.query).  Then checks the results
against the oracle: the in-place scale bit for bit, the norm within 1e-6
relative with the coefficient the clip rule gives for it, the AdamW update
bit for bit, and the loss-scaled calls (norm, found-inf flag, step, scale
update) likewise.  Prints one JSON line: {"idle": {call: bool, ...},
"parity": true}.  MTA_DEBUG_SYNC is read by the library from this process's
environment, which the parent sets.
"""
import json
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle as O  # noqa: E402
from mixed_precision_optimizer_mta_amd import AmpState  # noqa: E402
from mixed_precision_optimizer_mta_amd import workloads as WL  # noqa: E402
from parity_util import (check_amp_state, check_norm, compare,  # noqa: E402
                         make_list, oracle_grads, oracle_state)


def main():
    torch.cuda.set_device(0)
    side = torch.cuda.Stream()
    idle = {}
    # bf16 gradients, packed m, float32 v: 33M elements, about 0.1 ms of
    # device work for the update
    wl = WL.Workload("debug_sync", [4096 * 8000 + 13, 4096 * 50, 5],
                     WL.BF16, WL.MOM_BF16X2, WL.MOM_F32, steps=2,
                     g_mult=64.0, ident=81)
    arena = WL.Arena(wl, "cuda")
    arena.fill_weights()
    arena.fill_grads(1)
    torch.cuda.synchronize()
    ost = oracle_state(arena)
    nd = torch.zeros(1, device="cuda")
    cd = torch.zeros(1, device="cuda")
    with torch.cuda.stream(side):
        L = make_list(arena)
        side.synchronize()

        def call(name, fn):
            fn()
            idle[name] = bool(side.query())
            side.synchronize()

        # mta_scale in place: g = g * 2^-6 (exact on bfloat16)
        call("mta_scale(in place)", lambda: L.scale(2.0 ** -6, defer=False))
        for o in ost:
            O.scale_(o.g, wl.gtype, 2.0 ** -6)
        got = oracle_grads(arena)
        assert all(np.array_equal(a, o.g) for a, o in zip(got, ost))
        call("mta_clip_norm", lambda: L.clip_norm(1.0, nd, cd))
        check_norm(np.float32(nd.item()), np.float32(cd.item()),
                   O.norm([o.g for o in ost], wl.gtype), 1.0, "clip")
        call("mta_adamw_step", lambda: L.adamw_step(wl.hparams, 1, cd))
        O.step_(ost, wl.gtype, wl.mkind, wl.vkind, wl.lr, wl.beta1,
                wl.beta2, wl.eps, wl.weight_decay, 1,
                coef=np.float32(cd.item()))
        assert compare(arena, ost) == {"w": 0, "m": 0, "v": 0}
        # the loss-scaled calls: gradients hold 64 * g, scale 64
        amp_d = AmpState(64.0)
        amp_o = O.AmpState(64.0)
        side.synchronize()
        call("mta_amp_clip_norm",
             lambda: L.amp_clip_norm(1.0, amp_d, nd, cd))
        call("mta_amp_adamw_step",
             lambda: L.amp_adamw_step(wl.hparams, amp_d, cd))
        call("mta_amp_update", lambda: amp_d.update(2.0, 0.5, 2000))
        # the list's gradients were scaled by 2^-6 above: the oracle's
        # copies hold the same values
        _, _, found = O.amp_step_(ost, wl.gtype, wl.mkind, wl.vkind, amp_o,
                                  wl.lr, wl.beta1, wl.beta2, wl.eps,
                                  wl.weight_decay, 1.0,
                                  coef=np.float32(cd.item()))
        assert not found
        amp_o.update(2.0, 0.5, 2000)
        check_amp_state(amp_d.read(), amp_o, "amp")
        assert compare(arena, ost) == {"w": 0, "m": 0, "v": 0}
        L.close()
    print(json.dumps({"idle": idle, "parity": True,
                      "debug_sync": os.environ.get("MTA_DEBUG_SYNC")}),
          flush=True)


if __name__ == "__main__":
    main()
