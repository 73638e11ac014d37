"""GPU parity of per-tensor weight-decay flags (mta_list_set_no_decay).

One launch over a list whose flagged tensors take weight_decay = 0 must
update every tensor exactly as a step of its own, with its own weight decay,
would ("Mica 7.7", section "The whole model in one call": each group is
updated as a lone AdamWStep updates it).  The oracle therefore runs each
tensor as a list of one (oracle.opt_step_ / amp_opt_step_), with
weight_decay 0 for the flagged ones and the device's clip coefficient
(lockstep), and w, g, m, v are compared bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle as O
from mixed_precision_optimizer_mta_amd import workloads as WL

pytestmark = pytest.mark.gpu

from parity_util import (check_amp_state, check_norm, dev_bf16_bits,  # noqa: E402
                         oracle_grads)
from test_gpu_optimizers import (EDGE, compare_rule, make_rule_list,  # noqa: E402
                                 opt_for, oracle_rule_state)


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import mixed_precision_optimizer_mta_amd as M
    M.lib()
    yield
    torch.cuda.synchronize()


FLAGS = {
    "odd": lambda n: [i % 2 == 1 for i in range(n)],
    "ends": lambda n: [i in (0, n - 1) for i in range(n)],
    "all": lambda n: [True] * n,
    "none": lambda n: [False] * n,
}


def own_opt(opt, flag):
    """The rule a flagged tensor's lone step takes."""
    return dict(opt, weight_decay=0.0) if flag else opt


def nodecay_lockstep(wl, opt, flags, steps, offsets=None, copies=None,
                     copies_first=False, clear_at=None):
    """Steps of one list with these flags against per-tensor oracle steps.
    copies: None, or "bf16" / "f16" weight copies on every tensor (attached
    before the flags when copies_first).  clear_at: the step before which
    the flags are cleared (every tensor decays from then on)."""
    from mixed_precision_optimizer_mta_amd import MtaList  # noqa: F401
    arena = WL.Arena(wl, "cuda", offsets)
    arena.fill_weights()
    kind, zero = opt["kind"], bool(opt.get("zero_grad"))
    L = make_rule_list(arena, kind)
    ost = oracle_rule_state(arena, kind)
    dcopies = None
    if copies is not None:
        dt = torch.bfloat16 if copies == "bf16" else torch.float16
        ct = O.BF16 if copies == "bf16" else O.F16
        dcopies = [torch.zeros(n, dtype=dt, device="cuda") for n in wl.sizes]
        for o, n in zip(ost, wl.sizes):
            o.w16 = np.zeros(n, dtype=np.uint16)
            o.w16_type = ct
    if copies_first and dcopies is not None:
        L.set_weight_copies(dcopies)
    L.set_no_decay(flags)
    if not copies_first and dcopies is not None:
        L.set_weight_copies(dcopies)
    live = list(flags)
    nd = torch.full((1,), -1.0, device="cuda")
    cd = torch.full((1,), -1.0, device="cuda")
    for t in range(1, steps + 1):
        if clear_at is not None and t == clear_at:
            L.set_no_decay(None)
            live = [False] * wl.count
        arena.fill_grads(t)
        for o, g in zip(ost, oracle_grads(arena)):
            o.g = g
        if wl.scale != 1.0:
            L.scale(wl.scale, defer=True)
        L.clip_norm(wl.max_norm, nd, cd)
        L.step(opt, t, cd)
        torch.cuda.synchronize()
        what = f"{wl.name} {kind} t={t}"
        ng, coef = np.float32(nd.item()), np.float32(cd.item())
        check_norm(ng, coef, O.norm([o.g for o in ost], wl.gtype, wl.scale),
                   wl.max_norm, what)
        for o, f in zip(ost, live):
            O.opt_step_([o], own_opt(opt, f), wl.gtype, wl.mkind, wl.vkind,
                        t, s=wl.scale, coef=coef, zero=zero)
        compare_rule(arena, ost, kind, None, what)
        if dcopies is not None:
            for i, (c, o) in enumerate(zip(dcopies, ost)):
                assert np.array_equal(dev_bf16_bits(c), o.w16), (what, i)
    L.close()
    print(f"{wl.name} {kind}: {steps} steps with {sum(flags)} of "
          f"{wl.count} tensors undecayed, bitwise", flush=True)


@pytest.mark.parametrize("pattern", ["odd", "ends", "all", "none"])
@pytest.mark.parametrize("kind", ["adamw", "adam"])
def test_no_decay_patterns(kind, pattern):
    wl = WL.Workload(f"nodecay_{pattern}", EDGE, 0, 0, 0, steps=3,
                     g_sigma=0.3, ident=41)
    nodecay_lockstep(wl, opt_for(kind), FLAGS[pattern](wl.count), 3)


@pytest.mark.parametrize("gtype,mkind,vkind",
                         [(1, 1, 1), (2, 0, 0), (1, 1, 0), (0, 0, 1)])
@pytest.mark.parametrize("kind", ["adamw", "adam"])
def test_no_decay_types(kind, gtype, mkind, vkind):
    wl = WL.Workload("nodecay_types", EDGE, gtype, mkind, vkind, steps=3,
                     g_sigma=0.3, scale=0.5 if gtype else 1.0, ident=42)
    nodecay_lockstep(wl, opt_for(kind, zero=gtype == 2),
                     FLAGS["odd"](wl.count), 3)


@pytest.mark.parametrize("kind", ["sgd", "momentum"])
def test_no_decay_changes_nothing_without_decay(kind):
    # SGD and momentum have no decay: the flags leave the step as it was
    wl = WL.Workload("nodecay_plain", EDGE, 1, 0, 0, steps=2, g_sigma=0.3,
                     ident=43)
    nodecay_lockstep(wl, opt_for(kind, zero=True), FLAGS["odd"](wl.count), 2)


def test_no_decay_on_peeled_heads():
    # every buffer 1 element (mod 8) off: a head tile through the element
    # path, then vector tiles, each taking its tensor's flag
    sizes = [5000, 4096, 33, 9000, 5, 8200]
    offsets, pos = [], 0
    for n in sizes:
        offsets.append(pos + 1)
        pos += -(-(n + 1) // 8) * 8 + 8
    wl = WL.Workload("nodecay_heads", sizes, 1, 0, 0, steps=2, ident=44)
    nodecay_lockstep(wl, opt_for("adamw"), FLAGS["odd"](len(sizes)), 2,
                     offsets=offsets)


@pytest.mark.parametrize("copies_first", [False, True])
@pytest.mark.parametrize("copies", ["bf16", "f16"])
def test_no_decay_with_weight_copies(copies, copies_first):
    # either setting rewrites the tile table; each keeps the other's
    wl = WL.Workload("nodecay_copies", EDGE, 1, 1, 1, steps=2, g_sigma=0.3,
                     ident=45)
    nodecay_lockstep(wl, opt_for("adamw"), FLAGS["ends"](wl.count), 2,
                     copies=copies, copies_first=copies_first)


def test_no_decay_cleared():
    wl = WL.Workload("nodecay_clear", EDGE, 0, 0, 0, steps=3, g_sigma=0.3,
                     ident=46)
    nodecay_lockstep(wl, opt_for("adamw"), FLAGS["all"](wl.count), 3,
                     clear_at=2)


@pytest.mark.parametrize("kind", ["adamw", "adam"])
def test_no_decay_loss_scaled(kind):
    from mixed_precision_optimizer_mta_amd import AmpState
    wl = WL.Workload("nodecay_amp", EDGE, 2, 0, 0, steps=3, g_sigma=0.3,
                     ident=47)
    arena = WL.Arena(wl, "cuda")
    arena.fill_weights()
    L = make_rule_list(arena, kind)
    flags = FLAGS["odd"](wl.count)
    L.set_no_decay(flags)
    ost = oracle_rule_state(arena, kind)
    opt = opt_for(kind)
    amp_d, amp_o = AmpState(1024.0), O.AmpState(1024.0)
    nd = torch.full((1,), -1.0, device="cuda")
    cd = torch.full((1,), -1.0, device="cuda")
    for t in range(1, 4):
        arena.fill_grads(t)
        for o, g in zip(ost, oracle_grads(arena)):
            o.g = g
        L.amp_clip_norm(wl.max_norm, amp_d, nd, cd)
        L.amp_step(opt, amp_d, cd)
        amp_d.update(2.0, 0.5, 2)
        torch.cuda.synchronize()
        coef = np.float32(cd.item())
        s = O.inv_scale(amp_o.scale)
        check_norm(np.float32(nd.item()), coef,
                   O.norm([o.g for o in ost], wl.gtype, s), wl.max_norm,
                   f"amp t={t}")
        for o, f in zip(ost, flags):
            one = O.AmpState(amp_o.scale, amp_o.step, amp_o.tracker)
            _, _, found = O.amp_opt_step_([o], own_opt(opt, f), wl.gtype,
                                          wl.mkind, wl.vkind, one,
                                          wl.max_norm, coef=coef)
            assert not found
        amp_o.found_inf = np.float32(0.0)
        amp_o.update(2.0, 0.5, 2)
        check_amp_state(amp_d.read(), amp_o, f"amp t={t}")
        compare_rule(arena, ost, kind, None, f"nodecay amp {kind} t={t}")
    L.close()


@pytest.mark.timeout(300)
@pytest.mark.parametrize("kind", ["adamw", "adam"])
def test_no_decay_on_the_full_124m_list(kind):
    # the GPT-2 biases and layer-norm gains (the 60 tensors under 2^14
    # elements) flagged, as the 124M benchmark runs them with --no-decay:
    # every element of the full list against per-tensor oracle steps
    wl = WL.get("gpt2_124m")
    flags = [n < (1 << 14) for n in wl.sizes]
    assert sum(flags) == 60
    nodecay_lockstep(wl, opt_for(kind), flags, 2)


def test_no_decay_argument_checks():
    from mixed_precision_optimizer_mta_amd import MtaError
    wl = WL.Workload("nodecay_args", [9, 4096], 0, 0, 0, steps=1, ident=48)
    arena = WL.Arena(wl, "cuda")
    L = make_rule_list(arena, "adamw")
    with pytest.raises(ValueError):
        L.set_no_decay([True])             # one flag for two tensors
    import mixed_precision_optimizer_mta_amd._binding as B
    with pytest.raises(MtaError):
        B.mta_list_set_no_decay(None, None)  # no list
    L.set_no_decay([True, False])
    L.set_no_decay(None)
    L.close()
