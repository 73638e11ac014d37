"""GPU parity of the float16 gradient type and of dynamic loss scaling.

float16 gradients: every one of the 65,536 bit patterns goes through the
device's in-place ScaleTensors at several factors and must come back as the
oracle's bits (exact decode, nearest-even encode with float16 subnormals,
overflow to infinity and NaN -> 0xFFFF).

Loss scaling (mta_amp_clip_norm / mta_amp_adamw_step / mta_amp_update): a
device state holds the scale, the found-inf flag, the growth tracker and the
step counter.  Lockstep runs against oracle.amp_step_ and
oracle.AmpState.update check the norm, the flag, the whole state after every
step (scale bit for bit) and w, m, v; injected Inf and NaN gradients must
skip the step without touching any buffer; the step counter drives the bias
corrections at large t.
"""
import numpy as np
import pytest
import torch

import oracle as O
from mixed_precision_optimizer_mta_amd import workloads as WL

pytestmark = pytest.mark.gpu

from parity_util import (check_amp_state, compare, lockstep,  # noqa: E402
                         make_list, oracle_grads, oracle_state)


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import mixed_precision_optimizer_mta_amd as M
    M.lib()
    yield
    torch.cuda.synchronize()


SMALL_SIZES = WL.gpt2_sizes(1000, 64, 128, 2, 256)


def amp_small(gtype=WL.F16, mkind=WL.MOM_F32, vkind=WL.MOM_F32, interval=3,
              growth=2.0, backoff=0.5, scale=65536.0):
    wl = WL.scaled_down(WL.get("gpt2_124m_f16amp"), SMALL_SIZES,
                        name=f"amp_small_g{gtype}m{mkind}v{vkind}")
    wl.gtype, wl.mkind, wl.vkind = gtype, mkind, vkind
    wl.amp_interval, wl.amp_growth, wl.amp_backoff = interval, growth, backoff
    wl.amp_scale = scale
    wl.g_mult = scale
    return wl


def all_f16_patterns_arena():
    wl = WL.Workload("f16_patterns", [1 << 16], WL.F16, 0, 0, steps=1,
                     ident=21)
    arena = WL.Arena(wl, "cuda")
    return wl, arena


@pytest.mark.parametrize("s", [1.0, 0.5, 2.0, 3.0, 0.1, 2.0 ** -24, 1e-3,
                               1e4, 65504.0, 2.0 ** -14 / 3])
def test_f16_every_pattern_through_in_place_scale(s):
    wl, arena = all_f16_patterns_arena()
    pats = torch.arange(-32768, 32768, dtype=torch.int32).to(torch.int16)
    arena.g.view(torch.int16)[:1 << 16].copy_(pats.cuda())
    want = oracle_grads(arena)[0].copy()
    O.scale_(want, WL.F16, s)
    L = make_list(arena)
    L.scale(s, defer=False)
    torch.cuda.synchronize()
    got = oracle_grads(arena)[0]
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (s, [(hex(int(pats[i]) & 0xFFFF), hex(got[i]),
                                hex(want[i])) for i in bad[:8]])
    L.close()


def test_f16_every_pattern_in_the_norm_and_update():
    # all finite float16 patterns in one tensor (the 2048 Inf/NaN patterns
    # left out), with a deferred unscale: norm, clip and AdamW vs the oracle
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = (h & 0x7C00) != 0x7C00
    h = h[finite]
    wl = WL.Workload("f16_finite", [h.size], WL.F16, 0, 0, steps=1,
                     scale=2.0 ** -10, ident=22)
    arena = WL.Arena(wl, "cuda")
    arena.fill_weights()
    arena.g.view(torch.int16)[:h.size].copy_(
        torch.from_numpy(h.view(np.int16)).cuda())
    ostate = oracle_state(arena)
    L = make_list(arena)
    nd = torch.zeros(1, device="cuda")
    cd = torch.zeros(1, device="cuda")
    L.scale(wl.scale, defer=True)
    L.clip_norm(1.0, nd, cd)
    L.adamw_step(wl.hparams, 1, cd)
    torch.cuda.synchronize()
    no = O.norm([ostate[0].g], WL.F16, wl.scale)
    assert abs(nd.item() - no) <= 1e-6 * no
    O.step_(ostate, WL.F16, 0, 0, wl.lr, wl.beta1, wl.beta2, wl.eps,
            wl.weight_decay, 1, s=wl.scale, coef=np.float32(cd.item()))
    assert compare(arena, ostate) == {"w": 0, "m": 0, "v": 0}
    L.close()


@pytest.mark.parametrize("gtype,mkind,vkind", [(WL.F16, 0, 0),
                                               (WL.F16, 1, 1),
                                               (WL.BF16, 1, 0),
                                               (WL.F32, 0, 1)])
def test_amp_lockstep_with_overflow_steps(gtype, mkind, vkind):
    wl = amp_small(gtype, mkind, vkind, interval=3)
    arena = WL.Arena(wl, "cuda")
    o0, o1 = arena.offsets[0], arena.offsets[3]
    inject = {4: [(o0 + 5, float("inf"))],
              7: [(o1 + 1, float("nan"))],
              8: [(o0 + 2, float("-inf")), (o1 + 3, float("inf"))]}
    worst = lockstep(wl, 14, check_guards=True, inject=inject)
    assert worst == {"w": 0, "m": 0, "v": 0}, worst


def test_amp_non_power_of_two_factors_and_a_tiny_scale():
    wl = amp_small(WL.F16, 0, 0, interval=2, growth=1.7, backoff=0.3,
                   scale=3.0)
    arena = WL.Arena(wl, "cuda")
    inject = {3: [(arena.offsets[1], float("inf"))]}
    assert lockstep(wl, 9, inject=inject) == {"w": 0, "m": 0, "v": 0}


def _amp_one_step(wl, step0, scale):
    from mixed_precision_optimizer_mta_amd import AmpState
    arena = WL.Arena(wl, "cuda")
    arena.fill_weights()
    arena.fill_grads(1)
    ostate = oracle_state(arena)
    L = make_list(arena)
    amp_d = AmpState(scale, step=step0)
    amp_o = O.AmpState(scale, step=step0)
    cd = torch.zeros(1, device="cuda")
    L.amp_clip_norm(wl.max_norm, amp_d, None, cd)
    L.amp_adamw_step(wl.hparams, amp_d, cd)
    amp_d.update(2.0, 0.5, 2000)
    torch.cuda.synchronize()
    O.amp_step_(ostate, wl.gtype, wl.mkind, wl.vkind, amp_o, wl.lr, wl.beta1,
                wl.beta2, wl.eps, wl.weight_decay, wl.max_norm,
                coef=np.float32(cd.item()))
    amp_o.update(2.0, 0.5, 2000)
    check_amp_state(amp_d.read(), amp_o, f"step0={step0}")
    worst = compare(arena, ostate, what=f"step0={step0}")
    L.close()
    return worst


@pytest.mark.parametrize("t", [1, 2, 10, 1000, 12345, 10 ** 6, 2 ** 31 + 5])
def test_amp_step_counter_drives_the_bias_corrections(t):
    wl = amp_small(WL.F16, 0, 0)
    wl.beta1, wl.beta2 = 0.9, 0.999
    assert _amp_one_step(wl, t - 1, 1024.0) == {"w": 0, "m": 0, "v": 0}


@pytest.mark.parametrize("betas", [(0.9, 0.95), (0.5, 0.75), (0.0, 0.9999),
                                   (0.99, 0.99999)])
def test_amp_bias_corrections_other_betas(betas):
    wl = amp_small(WL.F16, 1, 0)
    wl.beta1, wl.beta2 = betas
    for t in (1, 3, 77, 4567, 99999):
        assert _amp_one_step(wl, t - 1, 256.0) == {"w": 0, "m": 0, "v": 0}


def test_amp_skip_leaves_every_buffer_untouched():
    from mixed_precision_optimizer_mta_amd import AmpState
    wl = amp_small(WL.F16, 1, 1)
    arena = WL.Arena(wl, "cuda")
    arena.fill_weights()
    arena.fill_grads(1)
    arena.m.fill_(0.25)
    arena.g[arena.offsets[2] + 7] = float("nan")
    before = [x.clone() for x in (arena.w, arena.g, arena.m, arena.v)]
    L = make_list(arena)
    amp = AmpState(4096.0, step=41, growth_tracker=5)
    nd = torch.zeros(1, device="cuda")
    cd = torch.zeros(1, device="cuda")
    L.amp_clip_norm(1.0, amp, nd, cd)
    st = amp.read()
    assert st["found_inf"] == 1.0 and np.isnan(nd.item())
    L.amp_adamw_step(wl.hparams, amp, cd)
    torch.cuda.synchronize()
    for a, b in zip(before, (arena.w, arena.g, arena.m, arena.v)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    amp.update(2.0, 0.5, 2000)
    st = amp.read()
    assert (st["scale"], st["found_inf"], st["growth_tracker"],
            st["step"]) == (2048.0, 0.0, 0, 41)
    L.close()


def test_amp_update_sequence_matches_oracle():
    from mixed_precision_optimizer_mta_amd import AmpState
    rng = np.random.default_rng(5)
    for scale, growth, backoff, interval in ((2.0 ** 126, 2.0, 0.5, 2),
                                             (65536.0, 1.7, 0.3, 3),
                                             (1.0, 3.0, 0.9, 1),
                                             (2.0 ** -130, 2.0, 0.5, 1)):
        dev = AmpState(scale, step=7)
        ora = O.AmpState(scale, step=7)
        for k in range(60):
            found = float(rng.random() < 0.3)
            st = dev.read()
            dev.write(st["scale"], st["step"], st["growth_tracker"], found)
            ora.found_inf = np.float32(found)
            dev.update(growth, backoff, interval)
            ora.update(growth, backoff, interval)
            check_amp_state(dev.read(), ora, f"{scale} k={k}")


def test_amp_rejects_a_pending_deferred_factor():
    from mixed_precision_optimizer_mta_amd import AmpState, MtaError
    wl = amp_small()
    arena = WL.Arena(wl, "cuda")
    L = make_list(arena)
    amp = AmpState(1024.0)
    cd = torch.zeros(1, device="cuda")
    L.scale(0.5, defer=True)
    with pytest.raises(MtaError) as e:
        L.amp_clip_norm(1.0, amp, None, cd)
    assert e.value.code == -6
    with pytest.raises(MtaError) as e:
        L.amp_adamw_step(wl.hparams, amp, cd)
    assert e.value.code == -6
    L.adamw_step(wl.hparams, 1, cd)         # consumes the factor
    L.amp_clip_norm(1.0, amp, None, cd)     # allowed again
    torch.cuda.synchronize()
    L.close()


@pytest.mark.timeout(600)
def test_full_gpt2_124m_f16amp_every_element():
    # 20 loss-scaled steps, two of them skipped (an Inf at step 5, a NaN at
    # step 12): the norm, the found-inf flag and the loss-scale state are
    # checked at every step, and every element of w, m, v after each step
    wl = WL.get("gpt2_124m_f16amp")
    arena = WL.Arena(wl, "cuda")
    inject = {5: [(arena.offsets[0] + 3, float("inf"))],
              12: [(arena.offsets[57] + 1, float("nan"))]}
    del arena
    worst = lockstep(wl, wl.steps, inject=inject)
    assert worst == {"w": 0, "m": 0, "v": 0}, worst


def test_amp_constants_follow_the_hyperparameters_at_one_step_count():
    # the update keeps the last step's t-dependent constants in a per-list
    # cache keyed by t and by the generation of (lr, beta1, beta2): two
    # loss-scaled steps at the same t (no mta_amp_update between them) with
    # different lr, then with different betas, each match the oracle's
    # amp_step_ with its own hyperparameters; a list of 600 tiles, so many
    # workgroups read the cache within each launch
    from mixed_precision_optimizer_mta_amd import AmpState
    wl = WL.Workload("amp_cache", [4096 * 600 + 3, 77], WL.F16,
                     WL.MOM_BF16X2, WL.MOM_F32, steps=1, g_mult=1024.0,
                     amp=True, amp_scale=1024.0, ident=24)
    arena = WL.Arena(wl, "cuda")
    arena.fill_weights()
    arena.fill_grads(1)
    ost = oracle_state(arena)
    L = make_list(arena)
    amp_d, amp_o = AmpState(1024.0), O.AmpState(1024.0)
    cd = torch.zeros(1, device="cuda")
    for hp in (dict(lr=3e-4, beta1=0.9, beta2=0.999),
               dict(lr=1e-3, beta1=0.9, beta2=0.999),
               dict(lr=1e-3, beta1=0.8, beta2=0.99),
               dict(lr=1e-3, beta1=0.8, beta2=0.99)):
        h = dict(hp, eps=1e-8, weight_decay=0.1)
        L.amp_clip_norm(1.0, amp_d, None, cd)
        L.amp_adamw_step(h, amp_d, cd)
        torch.cuda.synchronize()
        _, _, found = O.amp_step_(ost, wl.gtype, wl.mkind, wl.vkind, amp_o,
                                  h["lr"], h["beta1"], h["beta2"], h["eps"],
                                  h["weight_decay"], 1.0,
                                  coef=np.float32(cd.item()))
        assert not found
        assert compare(arena, ost, what=str(hp)) == {"w": 0, "m": 0, "v": 0}
    # the step counter was never advanced: every step above ran at t = 1
    check_amp_state(amp_d.read(), amp_o, "no update")
    L.close()
