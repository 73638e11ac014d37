"""GPU parity of the in-place clip: ScaleTensors by a factor held in device
memory (mta_scale_device), gradient-only lists (w, m, v NULL), and
GradClipper, PyTorch's clip_grad_norm_ on the device ("Mica 7.7: a training
step on the card, in every float type", section "Values that stay on the
card": the norm is measured, the factor decided and the gradients scaled on
the card).  Every scaled gradient is compared bit for bit with the oracle's
ScaleTensors (oracle.scale_) by the same factor; the norm with the oracle's
(1e-6 relative) and the coefficient with the clip rule applied to the
device norm (exact), as in the lockstep protocol.
"""
import numpy as np
import pytest
import torch

import oracle as O
from mixed_precision_optimizer_mta_amd import workloads as WL

pytestmark = pytest.mark.gpu

from parity_util import check_norm, grad_np, make_list, oracle_grads  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import mixed_precision_optimizer_mta_amd as M
    M.lib()
    yield
    torch.cuda.synchronize()


EDGE = [0, 1, 2, 3, 7, 8, 9, 17, 4095, 4096, 4097, 8193, 3 * 4096 + 5]


def _bits(a, gtype):
    return a.view(np.uint16 if gtype else np.uint32)


@pytest.mark.parametrize("gtype", [0, 1, 2])
def test_scale_by_a_device_factor(gtype):
    wl = WL.Workload("scale_dev", EDGE, gtype, 0, 0, steps=1, g_sigma=30.0,
                     ident=61)
    arena = WL.Arena(wl, "cuda")
    arena.fill_grads(1)
    gs = oracle_grads(arena)
    L = make_list(arena)
    f = torch.empty(1, device="cuda")
    for s in (0.37, 1.0, 2.0 ** -10, 3.0, 0.0, float("nan")):
        f.fill_(s)
        L.scale_device(f)
        torch.cuda.synchronize()
        for g in gs:
            O.scale_(g, gtype, np.float32(s))
        for i, (a, b) in enumerate(zip(oracle_grads(arena), gs)):
            assert np.array_equal(_bits(a, gtype), _bits(b, gtype)), (s, i)
    L.close()


def test_device_factor_leaves_a_deferred_factor_pending():
    # the in-place scale by a device factor does not consume a deferred
    # host factor: the next norm still reads f32(g' * s)
    wl = WL.Workload("scale_dev_defer", [4097, 9], 0, 0, 0, steps=1,
                     ident=62)
    arena = WL.Arena(wl, "cuda")
    arena.fill_grads(1)
    gs = oracle_grads(arena)
    L = make_list(arena)
    L.scale(0.5, defer=True)
    f = torch.full((1,), 0.25, device="cuda")
    L.scale_device(f)
    nd, cd = torch.zeros(1, device="cuda"), torch.zeros(1, device="cuda")
    L.clip_norm(1.0, nd, cd)
    torch.cuda.synchronize()
    for g in gs:
        O.scale_(g, 0, np.float32(0.25))
    check_norm(np.float32(nd.item()), np.float32(cd.item()),
               O.norm(gs, 0, 0.5), 1.0, "deferred after device scale")
    L.close()


@pytest.mark.parametrize("gtype", [0, 1, 2])
def test_gradient_only_list(gtype):
    # g alone: the same norm as a full list over the same gradients, the
    # in-place scales, and every update or weight copy refused before any
    # launch with nothing written
    from mixed_precision_optimizer_mta_amd import MtaError, MtaList
    wl = WL.Workload("gonly", EDGE, gtype, 0, 0, steps=1, g_sigma=0.5,
                     ident=63)
    arena = WL.Arena(wl, "cuda")
    arena.fill_weights()
    arena.fill_grads(1)
    full = make_list(arena)
    ents = [(None, g, None, None, n) for (_, g, _, _, n) in arena.entries()]
    G = MtaList([], entries=ents, gtype=gtype, mkind=0, vkind=0)
    info = G.info()
    assert info["state_buffers"] == 0 and info["count"] == wl.count
    n1, c1 = torch.zeros(1, device="cuda"), torch.zeros(1, device="cuda")
    n2, c2 = torch.zeros(1, device="cuda"), torch.zeros(1, device="cuda")
    full.clip_norm(0.1, n1, c1)
    G.clip_norm(0.1, n2, c2)
    torch.cuda.synchronize()
    assert n1.item() == n2.item() and c1.item() == c2.item()
    w_before = arena.w.clone()
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
    for call in (lambda: G.adamw_step(hp, 1, c2),
                 lambda: G.step(dict(kind="sgd", lr=0.1, beta1=0.9,
                                     beta2=0.999, eps=1e-8, weight_decay=0.0,
                                     momentum=0.0, zero_grad=False), 1),
                 lambda: G.set_weight_copies(
                     [torch.zeros(n, dtype=torch.bfloat16, device="cuda")
                      for n in wl.sizes])):
        with pytest.raises(MtaError) as e:
            call()
        assert e.value.code == -6, str(e.value)          # MTA_ESTATE
    torch.cuda.synchronize()
    assert torch.equal(arena.w, w_before)
    gs = oracle_grads(arena)
    G.scale(0.5, defer=False)
    torch.cuda.synchronize()
    for g in gs:
        O.scale_(g, gtype, np.float32(0.5))
    for a, b in zip(oracle_grads(arena), gs):
        assert np.array_equal(_bits(a, gtype), _bits(b, gtype))
    G.close()
    full.close()


def _params(seed, dtypes):
    torch.manual_seed(seed)
    sizes = [1, 7, 4096, 4097, 3 * 4096 + 5, 0, 300 * 257]
    ps = []
    for i, n in enumerate(sizes):
        dt = dtypes[i % len(dtypes)]
        p = torch.nn.Parameter(torch.randn(n, device="cuda").to(dt))
        p.grad = (torch.randn(n, device="cuda") * 0.3).to(dt)
        ps.append(p)
    ps.append(torch.nn.Parameter(torch.randn(5, device="cuda")))  # no grad
    return ps


@pytest.mark.parametrize("dtypes", [
    (torch.float32,), (torch.bfloat16,),
    (torch.float32, torch.bfloat16, torch.float16)])
@pytest.mark.parametrize("max_norm", [0.5, 1e30])
def test_grad_clipper_matches_the_oracle(dtypes, max_norm):
    from mixed_precision_optimizer_mta_amd import GradClipper
    ps = _params(7, dtypes)
    code = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}
    clip = GradClipper(ps)
    for rnd in range(3):
        if rnd == 2:                      # a gradient moves: tables rebuilt
            ps[2].grad = ps[2].grad.clone()
        with_grad = [p for p in ps if p.grad is not None]
        gs = [grad_np(p.grad, code[p.grad.dtype]) for p in with_grad]
        # the joint norm over every dtype: float64 sums of squares, added
        parts = {}
        for p, g in zip(with_grad, gs):
            parts.setdefault(code[p.grad.dtype], []).append(g)
        total = O.joint_sumsq([(v, k, 1.0) for k, v in parts.items()])
        nrm = clip(max_norm)
        torch.cuda.synchronize()
        ng, coef = np.float32(nrm.item()), np.float32(clip.coef.item())
        check_norm(ng, coef, float(np.sqrt(total)), max_norm,
                   f"clipper {dtypes} round {rnd}")
        for p, g in zip(with_grad, gs):
            O.scale_(g, code[p.grad.dtype], coef)
            got = grad_np(p.grad, code[p.grad.dtype])
            assert np.array_equal(_bits(got, code[p.grad.dtype]),
                                  _bits(g, code[p.grad.dtype])), rnd
    assert ps[-1].grad is None
    clip.close()


def test_grad_clipper_agrees_with_torch():
    # PyTorch's own clip_grad_norm_ sums in another order: the norms agree
    # within float32 rounding and the clipped gradients within a few ulp
    from mixed_precision_optimizer_mta_amd import GradClipper
    a = _params(11, (torch.float32,))
    b = [torch.nn.Parameter(p.detach().clone()) for p in a]
    for pa, pb in zip(a, b):
        pb.grad = None if pa.grad is None else pa.grad.clone()
    nrm = GradClipper(a)(0.5)
    ref = torch.nn.utils.clip_grad_norm_(b, 0.5)
    torch.cuda.synchronize()
    assert abs(nrm.item() - ref.item()) <= 1e-6 * ref.item()
    for pa, pb in zip(a, b):
        if pa.grad is not None and pa.grad.numel():
            torch.testing.assert_close(pa.grad, pb.grad, rtol=1e-6, atol=0)
