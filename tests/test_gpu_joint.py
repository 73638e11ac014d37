"""One clip over several lists (mta_clip_norm_joint,
mta_amp_clip_norm_joint): lists with float32, bfloat16 and float16
gradients and their own deferred factors, against the oracle's joint norm
(1e-6 relative, the coefficient exact on the device norm), then every
list's update against the oracle bit for bit with the joint coefficient."""
import numpy as np
import pytest
import torch

import oracle as O
from mixed_precision_optimizer_mta_amd import (AmpState, MtaError,
                                               clip_norm_joint)
from mixed_precision_optimizer_mta_amd import workloads as WL

from parity_util import (check_norm, compare, in_groups, make_list,
                         oracle_grads, oracle_state)

pytestmark = pytest.mark.gpu


def lists_of(specs):
    """specs: [(sizes, gtype, mkind, vkind, scale, ident)] -> arenas."""
    out = []
    for sizes, g, m, v, scale, ident in specs:
        wl = WL.Workload(f"joint{ident}", sizes, g, m, v, steps=2,
                         g_sigma=0.05, scale=scale, ident=ident)
        a = WL.Arena(wl, "cuda")
        a.fill_weights()
        out.append(a)
    return out


SPECS = [([4096 * 3 + 5, 700], WL.F32, 0, 0, 1.0, 61),
         ([9000, 17, 4096], WL.BF16, 1, 0, 2.0 ** -8, 62),
         ([5000], WL.F16, 0, 1, 0.5, 63)]


@pytest.mark.parametrize("order", [(0, 1, 2), (2, 0, 1), (1,)])
def test_joint_clip_over_mixed_gradient_types(order):
    arenas = lists_of([SPECS[i] for i in order])
    lists = [make_list(a) for a in arenas]
    ost = [oracle_state(a) for a in arenas]
    nd = torch.zeros(1, device="cuda")
    cd = torch.zeros(1, device="cuda")
    max_norm = 0.5
    for t in (1, 2):
        parts = []
        for a, L, o in zip(arenas, lists, ost):
            a.fill_grads(t)
            for x, g in zip(o, oracle_grads(a)):
                x.g = g
            if a.wl.scale != 1.0:
                L.scale(a.wl.scale, defer=True)
            parts.append(([x.g for x in o], a.wl.gtype, a.wl.scale))
        clip_norm_joint(lists, max_norm, nd, cd)
        for a, L in zip(arenas, lists):
            L.adamw_step(a.wl.hparams, t, cd)
        torch.cuda.synchronize()
        coef = np.float32(cd.item())
        check_norm(np.float32(nd.item()), coef, O.joint_norm(parts),
                   max_norm, f"joint {order} t={t}")
        for a, o in zip(arenas, ost):
            O.step_(o, a.wl.gtype, a.wl.mkind, a.wl.vkind, a.wl.lr,
                    a.wl.beta1, a.wl.beta2, a.wl.eps, a.wl.weight_decay, t,
                    s=a.wl.scale, coef=coef)
            assert compare(a, o) == {"w": 0, "m": 0, "v": 0}
    for L in lists:
        L.close()


@pytest.mark.timeout(300)
def test_joint_clip_over_two_full_lists():
    # the full 124M float32 list and the full 124M bfloat16-gradient list
    # (its gradients under a deferred 2^-16) clipped as one model: the joint
    # norm within 1e-6 of the oracle's, and every element of both lists'
    # updates with the joint coefficient, two steps
    arenas = []
    for name in ("gpt2_124m", "gpt2_124m_bf16g"):
        a = WL.Arena(WL.get(name), "cuda")
        a.fill_weights()
        arenas.append(a)
    lists = [make_list(a) for a in arenas]
    ost = [oracle_state(a) for a in arenas]
    nd = torch.zeros(1, device="cuda")
    cd = torch.zeros(1, device="cuda")
    for t in (1, 2):
        parts = []
        for a, L, o in zip(arenas, lists, ost):
            a.fill_grads(t)
            for x, g in zip(o, oracle_grads(a)):
                x.g = g
            if a.wl.scale != 1.0:
                L.scale(a.wl.scale, defer=True)
            parts.append(([x.g for x in o], a.wl.gtype, a.wl.scale))
        clip_norm_joint(lists, 1.0, nd, cd)
        for a, L in zip(arenas, lists):
            L.adamw_step(a.wl.hparams, t, cd)
        torch.cuda.synchronize()
        coef = np.float32(cd.item())
        check_norm(np.float32(nd.item()), coef, O.joint_norm(parts), 1.0,
                   f"joint full t={t}")
        for a, o in zip(arenas, ost):
            wl = a.wl
            in_groups(o, lambda grp, wl=wl: O.step_(
                grp, wl.gtype, wl.mkind, wl.vkind, wl.lr, wl.beta1,
                wl.beta2, wl.eps, wl.weight_decay, t, s=wl.scale, coef=coef))
            assert compare(a, o) == {"w": 0, "m": 0, "v": 0}
    for L in lists:
        L.close()


def test_one_list_joint_is_the_plain_clip_and_repeats_bitwise():
    (a,) = lists_of([SPECS[1]])
    L = make_list(a)
    a.fill_grads(1)
    got = []
    for joint in (False, True, True):
        nd = torch.zeros(1, device="cuda")
        cd = torch.zeros(1, device="cuda")
        if joint:
            clip_norm_joint([L], 0.5, nd, cd)
        else:
            L.clip_norm(0.5, nd, cd)
        torch.cuda.synchronize()
        got.append((nd.view(torch.int32).item(), cd.view(torch.int32).item()))
    assert got[0] == got[1] == got[2]
    # two lists twice: the same bits every time (fixed order of the sums)
    b, c = lists_of([SPECS[0], SPECS[2]])
    Lb, Lc = make_list(b), make_list(c)
    b.fill_grads(1)
    c.fill_grads(1)
    bits = set()
    for _ in range(4):
        nd = torch.zeros(1, device="cuda")
        cd = torch.zeros(1, device="cuda")
        clip_norm_joint([L, Lb, Lc], 0.5, nd, cd)
        torch.cuda.synchronize()
        bits.add(nd.view(torch.int32).item())
    assert len(bits) == 1
    for x in (L, Lb, Lc):
        x.close()


def test_joint_rejects_a_repeated_list_and_pending_factor_under_amp():
    a, b = lists_of([SPECS[0], SPECS[2]])
    La, Lb = make_list(a), make_list(b)
    nd = torch.zeros(1, device="cuda")
    cd = torch.zeros(1, device="cuda")
    with pytest.raises(MtaError) as e:
        clip_norm_joint([La, Lb, La], 1.0, nd, cd)
    assert e.value.code == -1
    amp = AmpState(64.0)
    Lb.scale(0.5, defer=True)
    with pytest.raises(MtaError) as e:
        clip_norm_joint([La, Lb], 1.0, nd, cd, amp=amp)
    assert e.value.code == -6
    La.close()
    Lb.close()


def test_loss_scaled_joint_clip_and_found_inf():
    specs = [([4096 * 2 + 3], WL.F32, 0, 0, 1.0, 64),
             ([7000, 11], WL.F16, 0, 0, 1.0, 65)]
    arenas = lists_of(specs)
    lists = [make_list(a) for a in arenas]
    amp = AmpState(1024.0)
    nd = torch.zeros(1, device="cuda")
    cd = torch.zeros(1, device="cuda")
    for t, bad in ((1, False), (2, True)):
        for a in arenas:
            a.fill_grads(t)
        if bad:                        # an overflow in the float16 list
            arenas[1].view("g", 1)[3] = float("inf")
        parts = [(oracle_grads(a), a.wl.gtype, O.inv_scale(1024.0))
                 for a in arenas]
        clip_norm_joint(lists, 1.0, nd, cd, amp=amp)
        torch.cuda.synchronize()
        st = amp.read()
        assert st["found_inf"] == (1.0 if bad else 0.0)
        if not bad:
            check_norm(np.float32(nd.item()), np.float32(cd.item()),
                       O.joint_norm(parts), 1.0, f"amp joint t={t}")
    for L in lists:
        L.close()


def test_captured_joint_loss_scaled_step_replays_like_eager():
    # the joint loss-scaled clip of a float32 and a float16 list, both
    # lists' updates and the scale update, captured once and replayed;
    # twin lists run the same calls eagerly
    specs = [([4096 * 2 + 3, 100], WL.F32, 0, 0, 1.0, 66),
             ([7000], WL.F16, 1, 1, 1.0, 67)]
    a_cap, a_eag = lists_of(specs), lists_of(specs)
    L_cap = [make_list(a) for a in a_cap]
    L_eag = [make_list(a) for a in a_eag]
    amp_c, amp_e = AmpState(256.0), AmpState(256.0)
    outs = {k: (torch.zeros(1, device="cuda"), torch.zeros(1, device="cuda"))
            for k in ("cap", "eag")}

    def step(lists, arenas, amp, nd, cd):
        clip_norm_joint(lists, 1.0, nd, cd, amp=amp)
        for a, L in zip(arenas, lists):
            L.amp_adamw_step(a.wl.hparams, amp, cd)
        amp.update(2.0, 0.5, 2)

    for a in a_cap + a_eag:
        a.fill_grads(1)
    step(L_cap, a_cap, amp_c, *outs["cap"])     # eager warm-up on both
    step(L_eag, a_eag, amp_e, *outs["eag"])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        step(L_cap, a_cap, amp_c, *outs["cap"])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for t in range(2, 7):
        for a in a_cap + a_eag:
            a.fill_grads(t)
        if t == 4:                       # an overflow step, skipped by both
            for a in (a_cap[1], a_eag[1]):
                a.view("g", 0)[5] = float("inf")
        torch.cuda.synchronize()
        graph.replay()
        step(L_eag, a_eag, amp_e, *outs["eag"])
        torch.cuda.synchronize()
        for x, y in zip(outs["cap"], outs["eag"]):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32)), t
        assert amp_c.read() == amp_e.read(), t
        for a, b in zip(a_cap, a_eag):
            for buf in "wmv":
                assert torch.equal(getattr(a, buf).view(torch.int16),
                                   getattr(b, buf).view(torch.int16)), (t, buf)
    assert amp_c.read()["step"] == 5          # six steps, one skipped
    for L in L_cap + L_eag:
        L.close()
