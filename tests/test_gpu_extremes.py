"""Extreme values through every update rule, bit for bit against the oracle.

Weights, gradients and moments are seeded with subnormals, values near the
float32 limits, signed zeros, NaN and infinities beside ordinary numbers, and
the hyperparameters include degenerate ones (lr = 0, eps = 0, beta = 0, tiny
eps, large lr) and unscale factors that make gradients subnormal or
overflow.  The kernels are built with denormals kept and correctly rounded
'/' and sqrt, so every case must match the oracle exactly.
"""
import numpy as np
import pytest
import torch

import oracle as O
from mixed_precision_optimizer_mta_amd import workloads as WL

pytestmark = pytest.mark.gpu

from parity_util import (bf16_ulp, check_norm, dev_bf16_bits,  # noqa: E402
                         dev_f32, f32_ulp, grad_np, mom_np, oracle_grads)

SPECIAL = np.array([0.0, -0.0, 1e-45, -1e-45, 1e-40, -3e-39, 1.1754942e-38,
                    1e-30, 3e38, -3e38, 1e38, np.inf, -np.inf, np.nan, 1.0,
                    -1.0, 0.5, 1e-7, 65504.0, 1e5], dtype=np.float32)
# finite and small: a clipped step's joint norm stays finite, so the
# coefficient does not turn every element into NaN or 0
FINITE_SMALL = np.array([0.0, -0.0, 1e-45, -1e-45, 1e-40, -3e-39,
                         1.1754942e-38, 1e-30, 1.0, -1.0, 0.5, 1e-7],
                        dtype=np.float32)


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import mixed_precision_optimizer_mta_amd as M
    M.lib()
    yield
    torch.cuda.synchronize()


def _spiked(rng, n, scale, values=SPECIAL):
    x = (rng.standard_normal(n) * scale).astype(np.float32)
    k = rng.choice(n, size=n // 3, replace=False)
    x[k] = rng.choice(values, size=k.size)
    return x


def _fill(arena, seed, state_specials, clip):
    wl = arena.wl
    rng = np.random.default_rng([20261202, 404, seed])
    n = arena.total
    arena.w.copy_(torch.from_numpy(_spiked(rng, n, 0.02)))
    g = _spiked(rng, n, 1e-2, FINITE_SMALL if clip else SPECIAL)
    arena.g.copy_(torch.from_numpy(g).to(arena.g.dtype))
    for b in "mv":
        if state_specials:
            x = _spiked(rng, n, 1e-3)
            if b == "v":
                x = np.abs(x)
        else:
            x = np.zeros(n, np.float32)
        t = getattr(arena, b)
        t.copy_(torch.from_numpy(x).to(t.dtype))


CASES = [
    # kind, gtype, mkind, vkind, hyper overrides, scale, max_norm (None: no
    # clip, every special of g reaches its own element only)
    ("adamw", 0, 0, 0, {}, 1.0, None),
    ("adamw", 0, 0, 0, {}, 1.0, 1.0),
    ("adamw", 1, 1, 1, {}, 2.0 ** -126, None),
    ("adamw", 2, 1, 0, {}, 2.0 ** 100, None),
    ("adamw", 1, 1, 1, {}, 2.0 ** -120, 1e-30),
    ("adamw", 0, 0, 0, {"eps": 0.0}, 1.0, None),
    ("adamw", 0, 0, 1, {"eps": 1e-30, "lr": 1.0}, 1.0, None),
    ("adamw", 0, 0, 0, {"lr": 0.0}, 1.0, None),
    ("adamw", 0, 1, 1, {"beta1": 0.0, "beta2": 0.0}, 1.0, None),
    ("adam", 0, 0, 0, {"weight_decay": 1e30}, 1.0, None),
    ("adam", 1, 0, 1, {}, 0.5, 1e-20),
    ("sgd", 0, 0, 0, {"lr": 1e30}, 1.0, None),
    ("sgd", 2, 0, 0, {}, 2.0 ** -24, None),
    ("sgd", 0, 0, 0, {}, 1.0, 1e-3),
    ("momentum", 0, 0, 0, {"momentum": 0.0}, 1.0, None),
    ("momentum", 1, 0, 0, {"momentum": 1e30}, 1.0, None),
    ("momentum", 0, 0, 0, {}, 1.0, 0.5),
]


@pytest.mark.parametrize("state_specials", [False, True])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_extreme_values_match_the_oracle(case, state_specials):
    from mixed_precision_optimizer_mta_amd import MtaList
    kind, gtype, mkind, vkind, hyper, scale, max_norm = CASES[case]
    adam = kind in ("adamw", "adam")
    opt = dict(kind=kind, lr=1e-3 if adam else 0.05, beta1=0.9, beta2=0.999,
               eps=1e-8, weight_decay=0.1 if adam else 0.0, momentum=0.9,
               zero_grad=False)
    opt.update(hyper)
    clip = max_norm is not None
    wl = WL.Workload("extremes", [5000, 4096, 7, 4096 * 2 + 1], gtype, mkind,
                     vkind, steps=2, scale=scale,
                     max_norm=max_norm if clip else 1.0, ident=80 + case)
    arena = WL.Arena(wl, "cuda")
    _fill(arena, case, state_specials, clip)
    has_m, has_v = kind != "sgd", adam
    ents = [(w, g, m if has_m else None, v if has_v else None, n)
            for (w, g, m, v, n) in arena.entries()]
    L = MtaList([], entries=ents, gtype=gtype, mkind=mkind, vkind=vkind)
    ost = []
    for i in range(wl.count):
        views = [arena.view(b, i) for b in "wgmv"]
        ost.append(O.Tensor(dev_f32(views[0]), grad_np(views[1], gtype),
                            mom_np(views[2], mkind) if has_m else None,
                            mom_np(views[3], vkind) if has_v else None))
    nd = torch.zeros(1, device="cuda")
    cd = torch.zeros(1, device="cuda")
    for t in (1, 2):
        if scale != 1.0:
            L.scale(scale, defer=True)
        if clip:
            L.clip_norm(max_norm, nd, cd)
            L.step(opt, t, cd)
        else:
            L.step(opt, t, None)
        torch.cuda.synchronize()
        coef = np.float32(cd.item()) if clip else np.float32(1.0)
        if clip:
            nrm = O.norm([o.g for o in ost], gtype, scale)
            assert np.isfinite(nrm), case
            check_norm(np.float32(nd.item()), coef, nrm, max_norm,
                       f"case {case}")
            assert coef < 1.0, (case, coef)      # the clip is active
        O.opt_step_(ost, opt, gtype, mkind, vkind, t, s=scale, coef=coef)
        for i, o in enumerate(ost):
            n = wl.sizes[i]
            w, m, v = (arena.view(b, i) for b in "wmv")
            d = f32_ulp(dev_f32(w), o.w)
            assert d.max() == 0, (case, t, i, "w", int(np.argmax(d)))
            for has, x, k, ob, name in ((has_m, m, mkind, o.m, "m"),
                                        (has_v, v, vkind, o.v, "v")):
                if not has:
                    continue
                if k == WL.MOM_BF16X2:
                    d = bf16_ulp(dev_bf16_bits(x), O.unpack_words(ob, n))
                else:
                    d = f32_ulp(dev_f32(x), ob)
                assert d.max() == 0, (case, t, i, name, int(np.argmax(d)))
    # the check must not be vacuous: unless a hyperparameter is meant to
    # overflow, most weights stay finite
    if not any(abs(x) >= 1e29 for x in hyper.values()):
        w_all = np.concatenate([o.w for o in ost])
        assert np.isfinite(w_all).mean() > 0.3, (
            case, np.isfinite(w_all).mean())
    L.close()
