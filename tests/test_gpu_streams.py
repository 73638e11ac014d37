"""Streams: every call runs on the caller's stream (the current torch stream
here) and returns without waiting.  A step on a side stream gives the same
bits as on the default stream; two lists stepped concurrently on two streams
give the same bits as the same steps run one after the other (each list owns
its norm scratch); the host does not block on a call.
"""
import numpy as np
import pytest
import torch

from mixed_precision_optimizer_mta_amd import workloads as WL

pytestmark = pytest.mark.gpu

from parity_util import make_list  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import mixed_precision_optimizer_mta_amd as M
    M.lib()
    yield
    torch.cuda.synchronize()


def _setup(ident, gtype=WL.BF16):
    wl = WL.Workload(f"streams{ident}", [4096 * 300 + 9, 4096 * 50, 77],
                     gtype, WL.MOM_BF16X2, WL.MOM_F32, steps=3,
                     scale=0.25, ident=ident)
    arena = WL.Arena(wl, "cuda")
    arena.fill_weights()
    return wl, arena


def _steps(wl, arena, L, nd, cd):
    for t in range(1, 4):
        arena.fill_grads(t)
        L.scale(wl.scale, defer=True)
        L.clip_norm(wl.max_norm, nd, cd)
        L.adamw_step(wl.hparams, t, cd)


def _state(arena):
    return [getattr(arena, b).clone() for b in "wmv"]


def _equal(a, b):
    for x, y in zip(a, b):
        ity = torch.int32 if x.dtype == torch.float32 else torch.int16
        assert torch.equal(x.view(ity), y.view(ity))


def test_side_stream_equals_default_stream():
    results = []
    for use_side in (False, True):
        wl, arena = _setup(71)
        nd = torch.zeros(1, device="cuda")
        cd = torch.zeros(1, device="cuda")
        side = torch.cuda.Stream()
        if use_side:
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                L = make_list(arena)
                _steps(wl, arena, L, nd, cd)
            torch.cuda.current_stream().wait_stream(side)
        else:
            L = make_list(arena)
            _steps(wl, arena, L, nd, cd)
        torch.cuda.synchronize()
        results.append(_state(arena) + [nd.clone(), cd.clone()])
        L.close()
    _equal(results[0][:3], results[1][:3])
    assert torch.equal(results[0][3], results[1][3])
    assert torch.equal(results[0][4], results[1][4])


def test_two_lists_on_two_streams_equal_sequential_runs():
    seq = []
    for ident in (72, 73):
        wl, arena = _setup(ident, WL.F32)
        L = make_list(arena)
        nd, cd = torch.zeros(1, device="cuda"), torch.zeros(1, device="cuda")
        _steps(wl, arena, L, nd, cd)
        torch.cuda.synchronize()
        seq.append(_state(arena))
        L.close()
    setups = [_setup(ident, WL.F32) for ident in (72, 73)]
    lists = [make_list(a) for _, a in setups]
    outs = [(torch.zeros(1, device="cuda"), torch.zeros(1, device="cuda"))
            for _ in setups]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for t in range(1, 4):
        for (wl, arena), s in zip(setups, streams):
            with torch.cuda.stream(s):
                arena.fill_grads(t)
        for (wl, arena), L, (nd, cd), s in zip(setups, lists, outs,
                                                streams):
            with torch.cuda.stream(s):
                L.scale(wl.scale, defer=True)
                L.clip_norm(wl.max_norm, nd, cd)
                L.adamw_step(wl.hparams, t, cd)
    torch.cuda.synchronize()
    for (wl, arena), want in zip(setups, seq):
        _equal(_state(arena), want)
    for L in lists:
        L.close()


def test_calls_return_before_the_work_is_done():
    # a step on a 1.5e8-element list takes ~1 ms on the device; issuing it
    # must take far less on the host (no hidden synchronization)
    import time
    wl = WL.Workload("async", [150_000_000], WL.F32, 0, 0, steps=1,
                     ident=74)
    arena = WL.Arena(wl, "cuda")
    arena.fill_weights()
    arena.fill_grads(1)
    L = make_list(arena)
    nd, cd = torch.zeros(1, device="cuda"), torch.zeros(1, device="cuda")
    L.clip_norm(1.0, nd, cd)
    L.adamw_step(wl.hparams, 1, cd)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), \
        torch.cuda.Event(enable_timing=True)
    ev0.record()
    h0 = time.perf_counter()
    for t in range(2, 12):
        L.clip_norm(1.0, nd, cd)
        L.adamw_step(wl.hparams, t, cd)
    host_ms = (time.perf_counter() - h0) * 1e3
    ev1.record()
    torch.cuda.synchronize()
    dev_ms = ev0.elapsed_time(ev1)
    assert host_ms < 0.5 * dev_ms, (host_ms, dev_ms)
    assert np.isfinite(nd.item())
    L.close()
