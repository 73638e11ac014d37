"""Stress of the norm's finishing protocol: every workgroup stores its
partial into its own atomic slot and takes a ticket; the last one reads every
slot (reloading one still empty) and re-arms them.  Hundreds of launches run
back to back with no host synchronization between them, on grids of 1, 2
and 8 workgroups per CU (up to 2048 slots); every result must be the same
bits (the grid and tile order are fixed per list) and match the oracle's
norm, and the loss-scaled variant must report the same found-inf flag each
time.
"""
import os

import numpy as np
import pytest
import torch

import oracle as O
from mixed_precision_optimizer_mta_amd import workloads as WL

pytestmark = pytest.mark.gpu

from parity_util import make_list, oracle_grads  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import mixed_precision_optimizer_mta_amd as M
    M.lib()
    yield
    torch.cuda.synchronize()


def _list_with_norm_grid(arena, bpc):
    key = "MTA_NORM_BLOCKS_PER_CU"
    old = os.environ.get(key)
    os.environ[key] = str(bpc)
    try:
        return make_list(arena)
    finally:
        if old is None:
            del os.environ[key]
        else:
            os.environ[key] = old


@pytest.mark.parametrize("gtype", [WL.F32, WL.BF16, WL.F16])
@pytest.mark.parametrize("bpc", [1, 2, 8])
def test_back_to_back_norms_are_identical_and_right(gtype, bpc):
    sizes = [4096 * 2100 + 77, 5000, 3, 4096 * 7]
    wl = WL.Workload("norm_stress", sizes, gtype, 0, 0, steps=1, g_sigma=0.02,
                     ident=61)
    arena = WL.Arena(wl, "cuda")
    arena.fill_grads(1)
    L = _list_with_norm_grid(arena, bpc)
    info = L.info()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert info["grid_norm"] == min(info["tiles"], cus * bpc)
    reps = 300
    norms = torch.full((reps,), -1.0, device="cuda")
    coefs = torch.full((reps,), -1.0, device="cuda")
    for i in range(reps):
        L.clip_norm(0.5, norms[i:i + 1], coefs[i:i + 1])
    torch.cuda.synchronize()
    bits = norms.view(torch.int32).cpu().numpy()
    assert (bits == bits[0]).all(), np.unique(bits)
    assert (coefs.view(torch.int32).cpu().numpy() ==
            coefs[:1].view(torch.int32).item()).all()
    want = O.norm(oracle_grads(arena), gtype, 1.0)
    got = float(norms[0].item())
    assert abs(got - want) <= 1e-6 * want, (got, want)
    L.close()


@pytest.mark.parametrize("bpc", [1, 8])
def test_back_to_back_loss_scaled_norms_with_and_without_overflow(bpc):
    from mixed_precision_optimizer_mta_amd import AmpState
    sizes = [4096 * 600 + 5, 999]
    wl = WL.Workload("norm_stress_amp", sizes, WL.F16, 0, 0, steps=1,
                     g_sigma=0.02, g_mult=64.0, ident=62)
    arena = WL.Arena(wl, "cuda")
    arena.fill_grads(1)
    L = _list_with_norm_grid(arena, bpc)
    amp = AmpState(64.0)
    reps = 200
    norms = torch.full((reps,), -1.0, device="cuda")
    coef = torch.zeros(1, device="cuda")
    for i in range(reps):
        L.amp_clip_norm(1.0, amp, norms[i:i + 1], coef)
    torch.cuda.synchronize()
    assert amp.read()["found_inf"] == 0.0
    bits = norms.view(torch.int32).cpu().numpy()
    assert (bits == bits[0]).all()
    want = O.norm(oracle_grads(arena), WL.F16, O.inv_scale(64.0))
    assert abs(float(norms[0].item()) - want) <= 1e-6 * want
    arena.g[arena.offsets[1] + 3] = float("inf")
    for i in range(reps):
        L.amp_clip_norm(1.0, amp, norms[i:i + 1], coef)
    torch.cuda.synchronize()
    assert amp.read()["found_inf"] == 1.0
    assert torch.isinf(norms).all()
    L.close()
