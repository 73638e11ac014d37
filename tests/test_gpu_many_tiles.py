"""GPU parity on lists of many tiles, every element, for every (g, m, v)
kind of the update and every rule.

The full-size workloads use one (g, m, v) kind each; these lists cover
all twelve kinds -- float32, bfloat16 or float16 gradients, each moment
float32 or packed bfloat16 -- at a size where every workgroup of the update
handles tiles from several tensors (over 800 tiles of 4096 elements: more
than three per compute unit of an MI355X), with ragged tails, a one-tile
tensor and a tensor shorter than a vector, and compare w, m, v (and g when
a rule zeroes it) against the oracle bit for bit after each of two steps.
Lockstep protocol: the device norm is checked against the oracle's and its
coefficient fed to the oracle's step ("Mica 7.7", section "The whole model
in one call": the multi-tensor step leaves each group as the single-group
step would; "BendTorch main.bend", section "Optimizers": adam_decay,
adam_m, adam_v, adam_w, adam_grad, sgd_l, mom_l, adamh_l, adamhv_l).
"""
import pytest
import torch

from mixed_precision_optimizer_mta_amd import workloads as WL

pytestmark = pytest.mark.gpu

from parity_util import lockstep, make_list, opt_for, rule_lockstep  # noqa: E402,E501


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import mixed_precision_optimizer_mta_amd as M
    M.lib()
    yield
    torch.cuda.synchronize()


# 501 + 251 + 1 + 51 + 1 + 30 = 835 tiles, 3,442,573 elements; the
# gradients' joint norm (about 1.9) is above the clip threshold, so the
# coefficient is below 1
MANY = [4096 * 500 + 1237, 4096 * 250 + 3, 77, 4096 * 50 + 4095, 9,
        4096 * 30]
ALL_KINDS = [(g, m, v) for g in (WL.F32, WL.BF16, WL.F16)
             for m in (0, 1) for v in (0, 1)]


def many(gtype, mkind, vkind, ident):
    # 16-bit gradients hold 1024 * g and are unscaled by 2^-10 (deferred)
    scaled = gtype != WL.F32
    return WL.Workload("many_tiles", MANY, gtype, mkind, vkind, steps=2,
                       g_mult=1024.0 if scaled else 1.0,
                       scale=2.0 ** -10 if scaled else 1.0, ident=ident)


def _check_shape(wl):
    arena = WL.Arena(wl, "cuda")
    L = make_list(arena)
    info = L.info()
    L.close()
    assert info["tiles"] == 835
    assert info["tiles"] >= 3 * 256


@pytest.mark.parametrize("gtype,mkind,vkind", ALL_KINDS)
def test_adamw_step_every_kind_many_tiles(gtype, mkind, vkind):
    wl = many(gtype, mkind, vkind, 51)
    _check_shape(wl)
    worst = lockstep(wl, 2, check_guards=True)
    assert worst == {"w": 0, "m": 0, "v": 0}, worst


# AdamW without zeroing is the mta_adamw_step test above (mta_step runs
# the same kernel)
ADAM_RULES = [("adamw", True), ("adam", False), ("adam", True)]


@pytest.mark.parametrize("kind,zero", ADAM_RULES)
@pytest.mark.parametrize("gtype,mkind,vkind", ALL_KINDS)
def test_adam_rules_every_kind_many_tiles(gtype, mkind, vkind, kind, zero):
    wl = many(gtype, mkind, vkind, 52)
    rule_lockstep(wl, opt_for(kind, zero), 2, check_guards=True)


@pytest.mark.parametrize("zero", [False, True])
@pytest.mark.parametrize("kind", ["sgd", "momentum"])
@pytest.mark.parametrize("gtype", [WL.F32, WL.BF16, WL.F16])
def test_sgd_rules_every_gradient_type_many_tiles(gtype, kind, zero):
    wl = many(gtype, 0, 0, 53)
    rule_lockstep(wl, opt_for(kind, zero), 2, check_guards=True)
