"""GPU invariants of the step beyond element-wise parity: every tile
updated once at tile counts around the update's dispatch runs, lists
longer than one per-tile launch, the norm's
launch shape changing only its summation order, deferred vs in-place
unscale on bfloat16 gradients, the independent (non-lockstep) protocol, a
tensor past 2^32 elements, and an informational cross-check against
PyTorch's own AdamW."""
import numpy as np
import pytest
import torch

import oracle as O
from mixed_precision_optimizer_mta_amd import MtaList
from mixed_precision_optimizer_mta_amd import workloads as WL

from parity_util import (compare, lockstep, opt_for, oracle_grads,
                         oracle_state, rule_lockstep)

pytestmark = pytest.mark.gpu


def _list(arena):
    wl = arena.wl
    return MtaList([], entries=arena.entries(), gtype=wl.gtype,
                   mkind=wl.mkind, vkind=wl.vkind)


def _ragged_small():
    rng = np.random.default_rng(91)
    sizes = [int(max(1, np.floor(2.0 ** (16 * x)))) for x in rng.random(120)]
    return WL.scaled_down(WL.get("ragged"), sizes + [4096 * 7 + 3],
                          name="ragged_inv")


@pytest.mark.parametrize("ntiles", [1, 255, 256, 257, 511, 512, 513, 2049])
def test_update_covers_every_tile_once(ntiles):
    # one workgroup per tile, tiles handed to the XCDs in runs of 8 * 32:
    # tile counts just below, at and above whole runs, a last tile of 4091
    # elements, and every element of w, m, v against the oracle (a tile
    # missed or updated twice would differ); nothing outside the tensor is
    # written
    wl = WL.Workload("cover", [ntiles * 4096 - 5, 3], WL.BF16, WL.MOM_BF16X2,
                     WL.MOM_F32, steps=2, ident=61)
    worst = lockstep(wl, 2, check_guards=True)
    assert worst == {"w": 0, "m": 0, "v": 0}, worst


@pytest.mark.parametrize("bpc", ["1", "7"])
def test_norm_grid_changes_only_summation_order(bpc, monkeypatch):
    wl = _ragged_small()
    arena = WL.Arena(wl, "cuda")
    arena.fill_weights()
    arena.fill_grads(1)
    nref = O.norm(oracle_grads(arena), wl.gtype)
    monkeypatch.setenv("MTA_NORM_BLOCKS_PER_CU", bpc)
    L = _list(arena)
    nd = torch.zeros(1, device="cuda")
    cd = torch.zeros(1, device="cuda")
    L.clip_norm(1.0, nd, cd)
    torch.cuda.synchronize()
    assert abs(nd.item() - nref) <= 1e-6 * nref
    assert np.float32(cd.item()) == O.clip_coef(1.0, np.float32(nd.item()))
    L.close()


def test_deferred_equals_in_place_for_bf16_with_power_of_two_scale():
    # multiplying a bfloat16 value by 2^-16 is exact (no underflow at these
    # magnitudes), so rewriting g in place and unscaling in registers agree
    wl = WL.scaled_down(WL.get("gpt2_124m_bf16g"),
                        WL.gpt2_sizes(1000, 64, 128, 2, 256))
    res = []
    for defer in (True, False):
        arena = WL.Arena(wl, "cuda")
        arena.fill_weights()
        arena.fill_grads(1)
        L = _list(arena)
        cd = torch.zeros(1, device="cuda")
        L.scale(2.0 ** -16, defer=defer)
        L.clip_norm(0.5, None, cd)
        L.adamw_step(wl.hparams, 1, cd)
        torch.cuda.synchronize()
        res.append((arena.w.clone(), arena.m.clone(), arena.v.clone(),
                    cd.item()))
        L.close()
    (w1, m1, v1, c1), (w2, m2, v2, c2) = res
    assert c1 == c2
    assert torch.equal(w1, w2) and torch.equal(m1, m2) and torch.equal(v1, v2)


@pytest.mark.parametrize("name", ["gpt2_124m", "gpt2_xl", "ragged"])
def test_independent_protocol(name):
    # the oracle uses its own norm and coefficient (not the device's); the
    # float64 device norm rounds to the same float32, so the bits still agree
    wl = WL.get(name)
    small = {"gpt2_124m": WL.gpt2_sizes(2000, 64, 128, 2, 256),
             "gpt2_xl": WL.gpt2_sizes(2000, 96, 64, 2, 384),
             "ragged": _ragged_small().sizes}[name]
    wl = WL.scaled_down(wl, small)
    arena = WL.Arena(wl, "cuda")
    arena.fill_weights()
    ost = oracle_state(arena)
    L = _list(arena)
    cd = torch.zeros(1, device="cuda")
    for t in (1, 2, 3):
        arena.fill_grads(t)
        for o, g in zip(ost, oracle_grads(arena)):
            o.g = g
        L.scale(wl.scale, defer=True)
        L.clip_norm(wl.max_norm, None, cd)
        L.adamw_step(wl.hparams, t, cd)
        torch.cuda.synchronize()
        O.step_(ost, wl.gtype, wl.mkind, wl.vkind, wl.lr, wl.beta1, wl.beta2,
                wl.eps, wl.weight_decay, t, s=wl.scale, max_norm=wl.max_norm)
        worst = compare(arena, ost, what=f"{name} independent t={t}")
        assert worst == {"w": 0, "m": 0, "v": 0}, worst
    L.close()


@pytest.mark.parametrize("cap", [1, 256, 300])
def test_lists_longer_than_one_launch(monkeypatch, cap):
    # a list with more tiles than one per-tile launch holds (2^24 - 256 of
    # them) is updated and scaled in consecutive launches over stretches of
    # its tile table; MTA_MAX_TILE_GRID lowers the cap so that a list of
    # about 700 tiles takes several (every tile a launch of its own at 1).
    # Every element against the oracle, for AdamW, Adam with zeroing, a
    # loss-scaled step and the in-place scale.
    monkeypatch.setenv("MTA_MAX_TILE_GRID", str(cap))
    sizes = [4096 * 690 + 5, 3, 4096 * 3 + 1, 300]
    wl = WL.Workload("chunks", sizes, WL.BF16, WL.MOM_BF16X2, WL.MOM_F32,
                     steps=2, ident=41)
    arena = WL.Arena(wl, "cuda")
    L = _list(arena)
    info = L.info()
    assert info["tiles"] == 691 + 1 + 4 + 1
    assert info["grid_update"] == min(info["tiles"], cap)
    L.close()
    del arena
    worst = lockstep(wl, 2)
    assert worst == {"w": 0, "m": 0, "v": 0}, worst
    rule_lockstep(wl, opt_for("adam", True), 2)
    amp = WL.scaled_down(WL.get("gpt2_124m_f16amp"), sizes, name="chunks_amp")
    worst = lockstep(amp, 3)
    assert worst == {"w": 0, "m": 0, "v": 0}, worst
    # the in-place scale
    arena = WL.Arena(wl, "cuda")
    arena.fill_grads(1)
    gs = oracle_grads(arena)
    L = _list(arena)
    for s in (0.3, 2.0 ** 12):
        L.scale(s, defer=False)
        torch.cuda.synchronize()
        for g in gs:
            O.scale_(g, wl.gtype, s)
        for a, b in zip(oracle_grads(arena), gs):
            assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    L.close()


def test_tensor_past_two_to_the_32_elements():
    # one tensor of 2^32 + 4099 elements (bf16 g, packed m and v): tile
    # numbers past 2^20 and element offsets past 2^32; g is a constant, so
    # the norm has a closed form; w, m, v are checked at sampled positions
    n = (1 << 32) + 4099
    wl = WL.Workload("huge", [n], WL.BF16, WL.MOM_BF16X2, WL.MOM_BF16X2,
                     steps=1, ident=31)
    arena = WL.Arena(wl, "cuda")
    arena.fill_weights()
    arena.g.fill_(0.25)
    rng = np.random.default_rng(5)
    idx = np.unique(np.concatenate([
        np.arange(8), n - 1 - np.arange(4100), (1 << 32) + np.arange(-8, 8),
        rng.integers(0, n, size=1 << 16)]))
    ost = oracle_state(arena, idx)
    L = _list(arena)
    nd = torch.zeros(1, device="cuda")
    cd = torch.zeros(1, device="cuda")
    L.scale(0.5, defer=True)
    L.clip_norm(1.0, nd, cd)
    L.adamw_step(wl.hparams, 1, cd)
    torch.cuda.synchronize()
    want = 0.125 * np.sqrt(float(n))          # |x| sqrt(n), x = 0.25 * 0.5
    assert abs(nd.item() - want) <= 1e-6 * want
    c = np.float32(cd.item())
    assert c == O.clip_coef(1.0, np.float32(nd.item()))
    O.step_(ost, wl.gtype, wl.mkind, wl.vkind, wl.lr, wl.beta1, wl.beta2,
            wl.eps, wl.weight_decay, 1, s=0.5, coef=c)
    worst = compare(arena, ost, idx, "huge")
    assert worst == {"w": 0, "m": 0, "v": 0}, worst
    L.close()
    del arena
    torch.cuda.empty_cache()


def test_informational_torch_adamw_on_the_gpu():
    # PyTorch's single-tensor AdamW on the GPU is not the pages' arithmetic
    # bit for bit (its kernels may fuse lerp and use reciprocals), so this
    # is a tolerance check only: a few ulp of the terms over 5 steps
    wl = WL.scaled_down(WL.get("gpt2_124m"), [4096 * 5 + 17, 1000])
    arena = WL.Arena(wl, "cuda")
    arena.fill_weights()
    params = [torch.nn.Parameter(arena.view("w", i).clone())
              for i in range(wl.count)]
    opt = torch.optim.AdamW(params, lr=wl.lr, betas=(wl.beta1, wl.beta2),
                            eps=wl.eps, weight_decay=wl.weight_decay,
                            foreach=False, fused=False)
    L = _list(arena)
    cd = torch.zeros(1, device="cuda")
    for t in range(1, 6):
        arena.fill_grads(t)
        for i, p in enumerate(params):
            p.grad = arena.view("g", i).clone()
        torch.nn.utils.clip_grad_norm_(params, wl.max_norm, foreach=False)
        opt.step()
        L.clip_norm(wl.max_norm, None, cd)
        L.adamw_step(wl.hparams, t, cd)
    torch.cuda.synchronize()
    for i, p in enumerate(params):
        ours = arena.view("w", i)
        err = (ours - p.detach()).abs().max().item()
        assert err <= 5 * 2.0 ** -24 * wl.lr * 10 + 4 * 2.0 ** -24 * 0.1, err
    L.close()
