"""Seeded random parity sweep: every knob of the library at once.

Each case draws a tensor list (counts, sizes from empty through tail tiles to
several tiles; aligned, shifted off 16-byte alignment, or back to back in
flat buffers; sometimes the gradient shifted against the other buffers), a
gradient type, moment kinds, an update rule, gradient zeroing, a deferred
unscale or a device loss scale, bfloat16 or float16 weight copies on a
random subset of tensors, no-decay flags on another random subset, a clip
threshold (from always clipping to never) and occasionally a non-finite
gradient, then runs two lockstep steps
through the C ABI against the oracle
and compares every buffer bit for bit (w, g, the rule's state buffers, the
copies), the norm (1e-6 relative), the clip coefficient (exact) and, under
loss scaling, the whole device state.
"""
import os

import numpy as np
import pytest
import torch

import oracle as O
from mixed_precision_optimizer_mta_amd import workloads as WL

pytestmark = pytest.mark.gpu

from parity_util import (bf16_ulp, check_amp_state, check_norm,  # noqa: E402
                         expected_tiles,
                         dev_bf16_bits, dev_f32, f32_ulp, grad_np, mom_np,
                         oracle_grads)


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import mixed_precision_optimizer_mta_amd as M
    M.lib()
    yield
    torch.cuda.synchronize()


def draw_case(seed):
    rng = np.random.default_rng([20261202, 91, seed])
    count = int(rng.integers(1, 9))
    sizes = []
    for _ in range(count):
        r = rng.random()
        if r < 0.05:
            sizes.append(0)
        elif r < 0.25:
            sizes.append(int(rng.integers(1, 18)))
        elif r < 0.5:
            sizes.append(int(4096 * rng.integers(1, 5) + rng.integers(-3, 4)))
        else:
            sizes.append(int(rng.integers(18, 20000)))
    kind = str(rng.choice(O.OPT_KINDS))
    c = dict(
        seed=seed, sizes=sizes, kind=kind,
        gtype=int(rng.integers(0, 3)),
        mkind=0 if kind == "momentum" else int(rng.integers(0, 2)),
        vkind=int(rng.integers(0, 2)),
        zero=bool(rng.random() < 0.4),
        amp=bool(rng.random() < 0.35),
        scale=float(rng.choice([1.0, 0.5, 2.0 ** -10, 3.0])),
        aligned=bool(rng.random() < 0.6),
        copies=bool(rng.random() < 0.35),
        max_norm=float(rng.choice([1e-3, 0.1, 1.0, 1e30])),
        bad_step=int(rng.choice([0, 0, 0, 0, 1, 2])),
        shifts=[int(x) for x in rng.integers(0, 8, count)],
        pick=[bool(x) for x in rng.random(count) < 0.6],
        copy_f16=bool(rng.random() < 0.5),
        flat=bool(rng.random() < 0.5),
        g_shift=int(rng.choice([0, 0, 0, 0, 0, 1, 2, 5])),
    )
    # drawn last, so the cases of the earlier draws stay as they were
    c["nodecay"] = bool(rng.random() < 0.35)
    c["nd_pick"] = [bool(x) for x in rng.random(count) < 0.5]
    return c


def run_case(c):
    import mixed_precision_optimizer_mta_amd as M
    from mixed_precision_optimizer_mta_amd import AmpState, MtaList
    kind, gtype, mkind, vkind = c["kind"], c["gtype"], c["mkind"], c["vkind"]
    adam = kind in ("adamw", "adam")
    has_m, has_v = kind != "sgd", adam
    wl = WL.Workload(f"random{c['seed']}", c["sizes"], gtype, mkind, vkind,
                     steps=2, g_sigma=0.05,
                     g_mult=256.0 if c["amp"] else 1.0,
                     scale=1.0 if c["amp"] else c["scale"],
                     max_norm=c["max_norm"], amp=c["amp"], amp_scale=256.0,
                     amp_interval=2, ident=50 + c["seed"] % 1000)
    offsets = None
    if not c["aligned"] and c["flat"]:
        offsets = [c["shifts"][0]]          # back to back
        for n in c["sizes"][:-1]:
            offsets.append(offsets[-1] + n)
    elif not c["aligned"]:
        offsets, pos = [], 0
        for n, sh in zip(c["sizes"], c["shifts"]):
            offsets.append(pos + sh)
            pos += -(-(n + sh) // 8) * 8 + 8
    arena = WL.Arena(wl, "cuda", offsets, g_shift=c["g_shift"])
    arena.fill_weights()
    ents = [(w, g, m if has_m else None, v if has_v else None, n)
            for (w, g, m, v, n) in arena.entries()]
    L = MtaList([], entries=ents, gtype=gtype, mkind=mkind, vkind=vkind)
    info = L.info()
    assert (info["tiles"], info["vector_tensors"]) == \
        expected_tiles(ents, gtype, mkind, vkind)
    plan = M.mta_list_plan(ents, gtype, mkind, vkind)
    for key in ("count", "elements", "tiles", "vector_tensors",
                "state_buffers", "norm_kept_tiles"):
        assert plan[key] == info[key], key
    copies = None
    picked = [p and c["copies"] for p in c["pick"]]
    if c["copies"]:
        copies = torch.zeros(arena.total, dtype=torch.float16 if
                             c["copy_f16"] else torch.bfloat16, device="cuda")
        L.set_weight_copies([copies[o:o + n] if p else None for o, n, p in
                             zip(arena.offsets, wl.sizes, picked)])
    flags = [f and c["nodecay"] for f in c["nd_pick"]]
    if c["nodecay"]:
        L.set_no_decay(flags)
    opt = dict(kind=kind, lr=1e-3 if adam else 0.05, beta1=0.9, beta2=0.99,
               eps=1e-8, weight_decay=0.05 if adam else 0.0, momentum=0.8,
               zero_grad=c["zero"])
    # the flagged tensors' own rule: the same step with weight_decay = 0
    opt_nd = dict(opt, weight_decay=0.0)
    ost = []
    for i, n in enumerate(wl.sizes):
        views = [arena.view(b, i) for b in "wgmv"]
        ost.append(O.Tensor(dev_f32(views[0]), grad_np(views[1], gtype),
                            mom_np(views[2], mkind) if has_m else None,
                            mom_np(views[3], vkind) if has_v else None,
                            np.zeros(n, np.uint16) if picked[i] else None,
                            O.F16 if c["copy_f16"] else O.BF16))
    amp_d = AmpState(wl.amp_scale) if c["amp"] else None
    amp_o = O.AmpState(wl.amp_scale) if c["amp"] else None
    nd = torch.full((1,), -1.0, device="cuda")
    cd = torch.full((1,), -1.0, device="cuda")
    nonempty = [i for i, n in enumerate(wl.sizes) if n > 0]
    for t in (1, 2):
        arena.fill_grads(t)
        if t == c["bad_step"] and nonempty:
            i = nonempty[c["seed"] % len(nonempty)]
            arena.view("g", i)[wl.sizes[i] // 2] = float("inf")
        for o, g in zip(ost, oracle_grads(arena)):
            o.g = g
        if c["amp"]:
            s = O.inv_scale(amp_o.scale)
            L.amp_clip_norm(wl.max_norm, amp_d, nd, cd)
            L.amp_step(opt, amp_d, cd)
            amp_d.update(wl.amp_growth, wl.amp_backoff, wl.amp_interval)
        else:
            s = wl.scale
            if s != 1.0:
                L.scale(s, defer=True)
            L.clip_norm(wl.max_norm, nd, cd)
            L.step(opt, t, cd)
        torch.cuda.synchronize()
        coef = np.float32(cd.item())
        what = f"case {c} t={t}"
        check_norm(np.float32(nd.item()), coef,
                   O.norm([o.g for o in ost], gtype, s), wl.max_norm, what)
        subs = [([o for o, f in zip(ost, flags) if not f], opt),
                ([o for o, f in zip(ost, flags) if f], opt_nd)]
        if c["amp"]:
            found = not np.isfinite(O.norm([o.g for o in ost], gtype, s))
            if found:                  # the whole step is skipped
                O.amp_opt_step_(ost, opt, gtype, mkind, vkind, amp_o,
                                wl.max_norm, coef=coef, zero=c["zero"])
            else:
                for sub, rule in subs:
                    if sub:
                        one = O.AmpState(amp_o.scale, amp_o.step,
                                         amp_o.tracker)
                        O.amp_opt_step_(sub, rule, gtype, mkind, vkind, one,
                                        wl.max_norm, coef=coef,
                                        zero=c["zero"])
                amp_o.found_inf = np.float32(0.0)
            amp_o.update(wl.amp_growth, wl.amp_backoff, wl.amp_interval)
            check_amp_state(amp_d.read(), amp_o, what)
        else:
            for sub, rule in subs:
                if sub:
                    O.opt_step_(sub, rule, gtype, mkind, vkind, t, s=s,
                                coef=coef, zero=c["zero"])
        for i, (o, n) in enumerate(zip(ost, wl.sizes)):
            if n == 0:
                continue
            w, g, m, v = (arena.view(b, i) for b in "wgmv")
            assert f32_ulp(dev_f32(w), o.w).max() == 0, (what, i, "w")
            assert np.array_equal(grad_np(g, gtype), o.g), (what, i, "g")
            for has, x, k, ob, name in ((has_m, m, mkind, o.m, "m"),
                                        (has_v, v, vkind, o.v, "v")):
                if not has:
                    continue
                if k == WL.MOM_BF16X2:
                    d = bf16_ulp(dev_bf16_bits(x), O.unpack_words(ob, n))
                else:
                    d = f32_ulp(dev_f32(x), ob)
                assert d.max() == 0, (what, i, name)
            if picked[i]:
                o16 = arena.offsets[i]
                assert np.array_equal(dev_bf16_bits(copies[o16:o16 + n]),
                                      o.w16), (what, i, "copy")
    L.close()


# MTA_RANDOM_CASES widens the sweep for a one-off run
@pytest.mark.parametrize(
    "seed", range(int(os.environ.get("MTA_RANDOM_CASES", "600"))))
def test_random_case(seed):
    run_case(draw_case(seed))
