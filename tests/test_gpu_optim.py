"""MtaOptimizer, the torch.optim-style front end: a real torch model's
parameters and autograd gradients, one joint clip over every parameter
group, one launch per parameter set (groups that differ only by a zero
weight decay share one).  Checked bit for bit against the oracle
(lockstep on the device coefficient) and within rounding against
torch.optim.AdamW + clip_grad_norm_; state_dict round trips continue
exactly; reallocated gradients rebuild the tables."""
import copy

import numpy as np
import pytest
import torch

import oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import mixed_precision_optimizer_mta_amd as M
    M.lib()
    yield
    torch.cuda.synchronize()


def _model(seed=0):
    torch.manual_seed(seed)
    return torch.nn.Sequential(
        torch.nn.Linear(300, 513), torch.nn.GELU(),
        torch.nn.Linear(513, 257), torch.nn.GELU(),
        torch.nn.Linear(257, 10)).cuda()


def _grads(model, step):
    torch.manual_seed(1000 + step)
    x = torch.randn(64, 300, device="cuda")
    y = torch.randint(0, 10, (64,), device="cuda")
    loss = torch.nn.functional.cross_entropy(model(x), y)
    model.zero_grad(set_to_none=False)
    loss.backward()


def _host(t):
    return t.detach().cpu().numpy().copy()


@pytest.mark.parametrize("kind", ["adamw", "adam", "sgd", "momentum"])
def test_matches_the_oracle_bitwise(kind):
    from mixed_precision_optimizer_mta_amd import MtaOptimizer
    model = _model()
    params = list(model.parameters())
    adam = kind in ("adamw", "adam")
    groups = [{"params": params[:2], "lr": 1e-3 if adam else 0.05},
              {"params": params[2:], "lr": 3e-4 if adam else 0.02,
               "weight_decay": 0.0}]
    wd = 0.05 if adam else 0.0
    opt = MtaOptimizer(groups, kind=kind, betas=(0.9, 0.99), eps=1e-8,
                       weight_decay=wd, momentum=0.9, max_norm=0.5)
    ost = [[O.Tensor(_host(p), None, np.zeros(p.numel(), np.float32),
                     np.zeros(p.numel(), np.float32)) for p in g["params"]]
           for g in groups]
    for t in range(1, 5):
        _grads(model, t)
        for g, og in zip(groups, ost):
            for p, o in zip(g["params"], og):
                o.g = _host(p.grad).ravel()
                o.w = o.w.ravel()
        opt.step()
        torch.cuda.synchronize()
        coef = np.float32(opt.last_coef.item())
        allg = [o.g for og in ost for o in og]
        nrm = O.norm(allg, O.F32)
        assert abs(float(opt.last_norm.item()) - nrm) <= 1e-6 * nrm
        assert coef == O.clip_coef(0.5, np.float32(opt.last_norm.item()))
        for g, og in zip(groups, ost):
            o_opt = dict(kind=kind, lr=g["lr"], beta1=0.9, beta2=0.99,
                         eps=1e-8, weight_decay=g.get("weight_decay", wd),
                         momentum=0.9)
            O.opt_step_(og, o_opt, O.F32, 0, 0, t, coef=coef)
            for p, o in zip(g["params"], og):
                assert np.array_equal(_host(p).ravel().view(np.uint32),
                                      o.w.view(np.uint32)), (kind, t)


def test_close_to_torch_adamw_with_clip():
    from mixed_precision_optimizer_mta_amd import MtaOptimizer
    a = _model(3)
    b = copy.deepcopy(a)
    opt_a = MtaOptimizer(a.parameters(), kind="adamw", lr=1e-3,
                         weight_decay=0.1, max_norm=1.0)
    opt_b = torch.optim.AdamW(b.parameters(), lr=1e-3, weight_decay=0.1,
                              foreach=False)
    for t in range(1, 6):
        _grads(a, t)
        _grads(b, t)
        opt_a.step()
        torch.nn.utils.clip_grad_norm_(b.parameters(), 1.0, foreach=False)
        opt_b.step()
    for pa, pb in zip(a.parameters(), b.parameters()):
        assert torch.allclose(pa, pb, rtol=1e-5, atol=1e-7), \
            (pa - pb).abs().max().item()


def test_state_dict_round_trip_continues_exactly():
    from mixed_precision_optimizer_mta_amd import MtaOptimizer
    for packed in (False, True):
        ref = _model(5)
        opt_ref = MtaOptimizer(ref.parameters(), kind="adamw", lr=1e-3,
                               weight_decay=0.1, max_norm=1.0,
                               packed_moments=packed)
        for t in range(1, 7):
            _grads(ref, t)
            opt_ref.step()
        run = _model(5)
        opt = MtaOptimizer(run.parameters(), kind="adamw", lr=1e-3,
                           weight_decay=0.1, max_norm=1.0,
                           packed_moments=packed)
        for t in range(1, 4):
            _grads(run, t)
            opt.step()
        saved = copy.deepcopy(opt.state_dict())
        run2 = copy.deepcopy(run)
        opt2 = MtaOptimizer(run2.parameters(), kind="adamw", lr=1e-3,
                            weight_decay=0.1, max_norm=1.0,
                            packed_moments=packed)
        opt2.load_state_dict(saved)
        for t in range(4, 7):
            _grads(run2, t)
            opt2.step()
        torch.cuda.synchronize()
        for pa, pb in zip(ref.parameters(), run2.parameters()):
            assert torch.equal(pa, pb), packed


def test_reallocated_gradients_and_fused_zeroing():
    from mixed_precision_optimizer_mta_amd import MtaOptimizer
    a = _model(7)
    b = copy.deepcopy(a)
    opt_a = MtaOptimizer(a.parameters(), kind="momentum", lr=0.05,
                         momentum=0.9, max_norm=1.0)
    opt_b = MtaOptimizer(b.parameters(), kind="momentum", lr=0.05,
                         momentum=0.9, max_norm=1.0, zero_grad=True)
    for t in range(1, 5):
        for p in a.parameters():
            p.grad = None            # PyTorch allocates fresh gradients
        _grads(a, t)
        _grads(b, t)
        opt_a.step()
        opt_b.step()
        torch.cuda.synchronize()
        for p in b.parameters():     # zeroed inside the update launch
            assert not bool(p.grad.any())
    for pa, pb in zip(a.parameters(), b.parameters()):
        assert torch.equal(pa, pb)


def test_loss_scaled_front_end_matches_the_oracle_and_skips_overflow():
    from mixed_precision_optimizer_mta_amd import MtaOptimizer
    model = _model(11)
    params = list(model.parameters())
    opt = MtaOptimizer(params, kind="adamw", lr=1e-3, weight_decay=0.1,
                       max_norm=1.0, loss_scale=256.0, growth_interval=2)
    assert opt.loss_scale.item() == 256.0
    amp_o = O.AmpState(256.0)
    ost = [O.Tensor(_host(p).ravel(), None, np.zeros(p.numel(), np.float32),
                    np.zeros(p.numel(), np.float32)) for p in params]
    for t in range(1, 7):
        torch.manual_seed(2000 + t)
        x = torch.randn(32, 300, device="cuda")
        y = torch.randint(0, 10, (32,), device="cuda")
        model.zero_grad(set_to_none=False)
        loss = torch.nn.functional.cross_entropy(model(x), y)
        (loss * opt.loss_scale).backward()     # no host read of the scale
        if t == 4:
            params[0].grad[0, 0] = float("inf")
        for p, o in zip(params, ost):
            o.g = _host(p.grad).ravel()
        opt.step()
        torch.cuda.synchronize()
        coef = np.float32(opt.last_coef.item())
        _, _, found = O.amp_opt_step_(
            ost, dict(kind="adamw", lr=1e-3, beta1=0.9, beta2=0.999,
                      eps=1e-8, weight_decay=0.1, momentum=0.0),
            O.F32, 0, 0, amp_o, 1.0, coef=coef)
        assert found == (t == 4)
        amp_o.update(2.0, 0.5, 2)
        st = opt.amp.read()
        assert (np.float32(st["scale"]), st["step"], st["growth_tracker"]) \
            == (amp_o.scale, amp_o.step, amp_o.tracker), (t, st)
        for p, o in zip(params, ost):
            assert np.array_equal(_host(p).ravel().view(np.uint32),
                                  o.w.view(np.uint32)), t
    assert opt.amp.read()["step"] == 5


def _split_groups(model):
    """The usual two groups: matrices decay, biases do not."""
    ps = list(model.parameters())
    return [{"params": [p for p in ps if p.dim() == 2]},
            {"params": [p for p in ps if p.dim() == 1], "weight_decay": 0.0}]


@pytest.mark.parametrize("split", [False, True])
def test_capturable_step_replays_like_eager_steps(split):
    # the optimizer step captured once in a HIP graph; gradients are made
    # eagerly into the same storage before every replay; split: a decay and
    # a no-decay group in one launch (the flags live in the captured tables)
    from mixed_precision_optimizer_mta_amd import MtaOptimizer
    a = _model(13)
    b = copy.deepcopy(a)
    kw = dict(kind="adamw", lr=1e-3, weight_decay=0.1, max_norm=1.0,
              capturable=True, zero_grad=True)

    def params(m):
        return _split_groups(m) if split else m.parameters()

    opt_a, opt_b = MtaOptimizer(params(a), **kw), \
        MtaOptimizer(params(b), **kw)
    _grads(a, 1)
    _grads(b, 1)
    opt_a.step()                   # eager: builds the tables
    opt_b.step()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        opt_a.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for t in range(2, 8):
        _grads(a, t)
        _grads(b, t)
        torch.cuda.synchronize()
        graph.replay()
        opt_b.step()
        torch.cuda.synchronize()
        for pa, pb in zip(a.parameters(), b.parameters()):
            assert torch.equal(pa, pb), t
            assert not bool(pa.grad.any())
        assert opt_a.amp.read() == opt_b.amp.read()
    assert opt_a.amp.read()["step"] == 7
    assert opt_a.loss_scale.item() == 1.0
    assert len(opt_a._plan["updates"]) == 1


def test_capturable_matches_the_plain_step_on_finite_gradients():
    from mixed_precision_optimizer_mta_amd import MtaOptimizer
    a = _model(17)
    b = copy.deepcopy(a)
    opt_a = MtaOptimizer(a.parameters(), kind="adam", lr=1e-3,
                         weight_decay=0.05, max_norm=0.7, capturable=True)
    opt_b = MtaOptimizer(b.parameters(), kind="adam", lr=1e-3,
                         weight_decay=0.05, max_norm=0.7)
    for t in range(1, 6):
        _grads(a, t)
        _grads(b, t)
        opt_a.step()
        opt_b.step()
    torch.cuda.synchronize()
    # the device step constants use the correctly rounded power, the host
    # ones libm's pow; they agree at these t, so the runs are identical
    for pa, pb in zip(a.parameters(), b.parameters()):
        assert torch.equal(pa, pb)


def _bits16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(
        np.uint16).ravel().copy()


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16],
                         ids=["bf16", "f16"])
def test_master_weights_match_the_oracle_bitwise(dt):
    # a 16-bit model: float32 masters in the optimizer, 16-bit gradients,
    # and the new masters' 16-bit rounding written into the parameters by
    # the update launch; float16 runs loss-scaled with an overflow at t = 4
    from mixed_precision_optimizer_mta_amd import MtaOptimizer
    model = _model(13).to(dt)
    params = list(model.parameters())
    gt = O.BF16 if dt == torch.bfloat16 else O.F16
    scaled = dt == torch.float16
    opt = MtaOptimizer(params, kind="adamw", lr=1e-3, weight_decay=0.1,
                       max_norm=1.0, master_weights=True,
                       loss_scale=1024.0 if scaled else None,
                       growth_interval=2)
    rule = dict(kind="adamw", lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                weight_decay=0.1, momentum=0.0)
    ost = [O.Tensor(_host(p.float()).ravel(), None,
                    np.zeros(p.numel(), np.float32),
                    np.zeros(p.numel(), np.float32),
                    np.zeros(p.numel(), np.uint16), gt) for p in params]
    amp_o = O.AmpState(1024.0) if scaled else None
    for t in range(1, 7):
        torch.manual_seed(3000 + t)
        x = torch.randn(32, 300, device="cuda", dtype=dt)
        y = torch.randint(0, 10, (32,), device="cuda")
        model.zero_grad(set_to_none=False)
        loss = torch.nn.functional.cross_entropy(model(x).float(), y)
        (loss * opt.loss_scale if scaled else loss).backward()
        if scaled and t == 4:
            params[2].grad[1, 1] = float("inf")
        for p, o in zip(params, ost):
            assert p.grad.dtype == dt
            o.g = _bits16(p.grad)
        before = [_bits16(p) for p in params]
        opt.step()
        torch.cuda.synchronize()
        coef = np.float32(opt.last_coef.item())
        if scaled:
            _, _, found = O.amp_opt_step_(ost, rule, gt, 0, 0, amp_o, 1.0,
                                          coef=coef)
            assert found == (t == 4)
            amp_o.update(2.0, 0.5, 2)
            assert opt.amp.read()["step"] == amp_o.step
        else:
            nrm = O.norm([o.g for o in ost], gt)
            assert abs(float(opt.last_norm.item()) - nrm) <= 1e-6 * nrm
            O.opt_step_(ost, rule, gt, 0, 0, t, coef=coef)
        for p, o, b in zip(params, ost, before):
            w = opt.state[p]["master_weight"]
            assert w.dtype == torch.float32
            assert np.array_equal(_host(w).ravel().view(np.uint32),
                                  o.w.view(np.uint32)), (t, "master")
            assert np.array_equal(_bits16(p), o.w16), (t, "parameter")
            if scaled and t == 4:
                assert np.array_equal(_bits16(p), b)   # skipped step


def test_master_weights_state_dict_keeps_float32_state():
    from mixed_precision_optimizer_mta_amd import MtaOptimizer

    def make():
        m = _model(17).to(torch.bfloat16)
        return m, MtaOptimizer(m.parameters(), kind="adamw", lr=1e-3,
                               weight_decay=0.1, max_norm=1.0,
                               master_weights=True)

    def grads(m, t):
        torch.manual_seed(4000 + t)
        x = torch.randn(16, 300, device="cuda", dtype=torch.bfloat16)
        y = torch.randint(0, 10, (16,), device="cuda")
        m.zero_grad(set_to_none=False)
        torch.nn.functional.cross_entropy(m(x).float(), y).backward()

    ref, opt_ref = make()
    for t in range(1, 7):
        grads(ref, t)
        opt_ref.step()
    run, opt = make()
    for t in range(1, 4):
        grads(run, t)
        opt.step()
    saved = copy.deepcopy(opt.state_dict())
    run2 = copy.deepcopy(run)
    opt2 = MtaOptimizer(run2.parameters(), kind="adamw", lr=1e-3,
                        weight_decay=0.1, max_norm=1.0, master_weights=True)
    opt2.load_state_dict(saved)
    for p in run2.parameters():
        for name in ("master_weight", "exp_avg", "exp_avg_sq"):
            assert opt2.state[p][name].dtype == torch.float32, name
    for t in range(4, 7):
        grads(run2, t)
        opt2.step()
    torch.cuda.synchronize()
    for pa, pb in zip(ref.parameters(), run2.parameters()):
        assert torch.equal(pa.view(torch.int16), pb.view(torch.int16))
        assert torch.equal(opt_ref.state[pa]["master_weight"],
                           opt2.state[pb]["master_weight"])


def test_master_weights_loss_scaled_step_replays_in_a_graph():
    # a float16 model, float32 masters, device loss scaling: the whole
    # optimizer step captured once and replayed matches eager steps bit for
    # bit (masters, parameters and the scale state)
    from mixed_precision_optimizer_mta_amd import MtaOptimizer
    a = _model(19).to(torch.float16)
    b = copy.deepcopy(a)
    kw = dict(kind="adamw", lr=1e-3, weight_decay=0.1, max_norm=1.0,
              master_weights=True, loss_scale=512.0, growth_interval=3,
              zero_grad=True)
    opt_a, opt_b = MtaOptimizer(a.parameters(), **kw), \
        MtaOptimizer(b.parameters(), **kw)

    def grads(m, opt, t):
        torch.manual_seed(5000 + t)
        x = torch.randn(16, 300, device="cuda", dtype=torch.float16)
        y = torch.randint(0, 10, (16,), device="cuda")
        loss = torch.nn.functional.cross_entropy(m(x).float(), y)
        (loss * opt.loss_scale).backward()

    for m, o in ((a, opt_a), (b, opt_b)):
        grads(m, o, 1)
        o.step()                   # eager: builds the tables and masters
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        opt_a.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for t in range(2, 9):
        grads(a, opt_a, t)
        grads(b, opt_b, t)
        torch.cuda.synchronize()
        graph.replay()
        opt_b.step()
        torch.cuda.synchronize()
        for pa, pb in zip(a.parameters(), b.parameters()):
            assert torch.equal(pa.view(torch.int16), pb.view(torch.int16)), t
            assert torch.equal(opt_a.state[pa]["master_weight"],
                               opt_b.state[pb]["master_weight"]), t
            assert not bool(pa.grad.any())
        assert opt_a.amp.read() == opt_b.amp.read()
    assert opt_a.amp.read()["step"] >= 6


class _Mixed(torch.nn.Module):
    """A bfloat16 model with one layer kept in float32 (a parameter whose
    uses need full precision)."""

    def __init__(self, seed):
        super().__init__()
        torch.manual_seed(seed)
        self.a = torch.nn.Linear(300, 257).to(torch.bfloat16)
        self.b = torch.nn.Linear(257, 10)          # float32

    def forward(self, x):
        h = torch.nn.functional.gelu(self.a(x))
        return self.b(h.float())


@pytest.mark.parametrize("kind", ["adamw", "adam", "sgd", "momentum"])
def test_master_weights_with_a_float32_layer_match_the_oracle(kind):
    # bfloat16 parameters: float32 masters and copies written back; the
    # float32 layer is its own weight; one joint clip over both gradient
    # types; every rule (momentum keeps a float32 buffer)
    from mixed_precision_optimizer_mta_amd import MtaOptimizer
    model = _Mixed(23).cuda()
    params = list(model.parameters())
    adam = kind in ("adamw", "adam")
    lr = 1e-3 if adam else 0.05
    opt = MtaOptimizer(params, kind=kind, lr=lr, betas=(0.9, 0.99),
                       weight_decay=0.05 if adam else 0.0, momentum=0.9,
                       max_norm=0.5, master_weights=True)
    rule = dict(kind=kind, lr=lr, beta1=0.9, beta2=0.99, eps=1e-8,
                weight_decay=0.05 if adam else 0.0, momentum=0.9)
    half = [p for p in params if p.dtype == torch.bfloat16]
    full = [p for p in params if p.dtype == torch.float32]
    assert half and full

    def state(p):
        n = p.numel()
        m = np.zeros(n, np.float32) if kind != "sgd" else None
        v = np.zeros(n, np.float32) if adam else None
        if p.dtype == torch.float32:
            return O.Tensor(_host(p).ravel(), None, m, v)
        return O.Tensor(_host(p.float()).ravel(), None, m, v,
                        np.zeros(n, np.uint16), O.BF16)

    o_half = [state(p) for p in half]
    o_full = [state(p) for p in full]
    for t in range(1, 5):
        torch.manual_seed(6000 + t)
        x = torch.randn(32, 300, device="cuda", dtype=torch.bfloat16)
        y = torch.randint(0, 10, (32,), device="cuda")
        model.zero_grad(set_to_none=False)
        torch.nn.functional.cross_entropy(model(x), y).backward()
        for p, o in zip(half, o_half):
            o.g = _bits16(p.grad)
        for p, o in zip(full, o_full):
            o.g = _host(p.grad).ravel()
        opt.step()
        torch.cuda.synchronize()
        parts = [([o.g for o in o_full], O.F32, 1.0),
                 ([o.g for o in o_half], O.BF16, 1.0)]
        nrm = O.joint_norm(parts)
        assert abs(float(opt.last_norm.item()) - nrm) <= 1e-6 * nrm
        coef = np.float32(opt.last_coef.item())
        assert coef == O.clip_coef(0.5, np.float32(opt.last_norm.item()))
        O.opt_step_(o_full, rule, O.F32, 0, 0, t, coef=coef)
        O.opt_step_(o_half, rule, O.BF16, 0, 0, t, coef=coef)
        for p, o in zip(full, o_full):
            assert np.array_equal(_host(p).ravel().view(np.uint32),
                                  o.w.view(np.uint32)), (kind, t)
        for p, o in zip(half, o_half):
            w = opt.state[p]["master_weight"]
            assert np.array_equal(_host(w).ravel().view(np.uint32),
                                  o.w.view(np.uint32)), (kind, t)
            assert np.array_equal(_bits16(p), o.w16), (kind, t)
        if kind == "momentum":
            for p in params:
                assert opt.state[p]["momentum_buffer"].dtype == torch.float32


def test_plan_follows_schedules_empty_params_and_missing_grads():
    # a learning-rate schedule changes lr every step (no rebuild needed), a
    # zero-element parameter and a group without gradients ride along, and
    # a gradient that moves forces a rebuild; bitwise against the oracle
    from mixed_precision_optimizer_mta_amd import MtaOptimizer
    model = _model(29)
    params = list(model.parameters())
    empty = torch.nn.Parameter(torch.zeros(0, device="cuda"))
    idle = torch.nn.Parameter(torch.ones(5, device="cuda"))   # never a grad
    opt = MtaOptimizer([{"params": params + [empty]}, {"params": [idle]}],
                       kind="adamw", lr=1e-3, betas=(0.9, 0.99),
                       weight_decay=0.1, max_norm=0.7)
    sched = torch.optim.lr_scheduler.LambdaLR(opt, lambda s: 1.0 / (1 + s))
    ost = [O.Tensor(_host(p).ravel(), None, np.zeros(p.numel(), np.float32),
                    np.zeros(p.numel(), np.float32)) for p in params]
    for t in range(1, 6):
        _grads(model, t)
        empty.grad = torch.zeros(0, device="cuda")
        if t == 4:                       # a gradient moves: rebuild
            params[0].grad = params[0].grad.clone()
        lr = opt.param_groups[0]["lr"]
        for p, o in zip(params, ost):
            o.g = _host(p.grad).ravel()
        opt.step()
        sched.step()
        torch.cuda.synchronize()
        coef = np.float32(opt.last_coef.item())
        O.opt_step_(ost, dict(kind="adamw", lr=lr, beta1=0.9, beta2=0.99,
                              eps=1e-8, weight_decay=0.1, momentum=0.0),
                    O.F32, 0, 0, t, coef=coef)
        for p, o in zip(params, ost):
            assert np.array_equal(_host(p).ravel().view(np.uint32),
                                  o.w.view(np.uint32)), t
    assert torch.equal(idle.detach(), torch.ones(5, device="cuda"))
    sd = opt.state_dict()
    assert all(sd["state"][i]["step"] == 5 for i in range(len(params)))


def test_decay_and_no_decay_groups_share_one_launch():
    # the usual split (matrices decay, biases do not) is one list with the
    # biases flagged; a second nonzero decay or a different lr separates
    # the groups again, and equal values join them; every step bitwise
    # against the oracle run group by group with each group's own decay
    from mixed_precision_optimizer_mta_amd import MtaOptimizer
    model = _model(37)
    params = list(model.parameters())
    mats = [p for p in params if p.dim() == 2]
    vecs = [p for p in params if p.dim() == 1]
    groups = [{"params": mats, "weight_decay": 0.1},
              {"params": vecs, "weight_decay": 0.0}]
    opt = MtaOptimizer(groups, kind="adamw", lr=1e-3, betas=(0.9, 0.99),
                       max_norm=0.7)
    ost = [[O.Tensor(_host(p).ravel(), None, np.zeros(p.numel(), np.float32),
                     np.zeros(p.numel(), np.float32)) for p in g["params"]]
           for g in groups]
    launches = []
    for t in range(1, 8):
        if t == 3:                                  # two nonzero decays
            opt.param_groups[1]["weight_decay"] = 0.05
        if t == 4:                                  # equal again: one set
            opt.param_groups[1]["weight_decay"] = 0.1
        if t == 5:                                  # back to the split
            opt.param_groups[1]["weight_decay"] = 0.0
        if t == 6:                                  # different lr
            opt.param_groups[1]["lr"] = 5e-4
        if t == 7:
            opt.param_groups[1]["lr"] = 1e-3
        _grads(model, t)
        for g, og in zip(groups, ost):
            for p, o in zip(g["params"], og):
                o.g = _host(p.grad).ravel()
        opt.step()
        launches.append(len(opt._plan["updates"]))
        torch.cuda.synchronize()
        coef = np.float32(opt.last_coef.item())
        for g, og in zip(opt.param_groups, ost):
            O.opt_step_(og, dict(kind="adamw", lr=g["lr"], beta1=0.9,
                                 beta2=0.99, eps=1e-8,
                                 weight_decay=g["weight_decay"],
                                 momentum=0.0), O.F32, 0, 0, t, coef=coef)
            for p, o in zip(g["params"], og):
                assert np.array_equal(_host(p).ravel().view(np.uint32),
                                      o.w.view(np.uint32)), t
    assert launches == [1, 1, 2, 1, 1, 2, 1]
    sd = opt.state_dict()
    assert all(s["step"] == 7 for s in sd["state"].values())


def _scaled_grads(model, opt, t, inf_at=None):
    torch.manual_seed(3000 + t)
    x = torch.randn(32, 300, device="cuda")
    y = torch.randint(0, 10, (32,), device="cuda")
    model.zero_grad(set_to_none=False)
    loss = torch.nn.functional.cross_entropy(model(x), y)
    (loss * opt.loss_scale).backward()
    if t == inf_at:
        next(model.parameters()).grad[0, 0] = float("inf")


def test_loss_scaled_state_dict_resumes_exactly():
    # a loss-scaled run checkpointed after an overflow step: the scale, the
    # growth tracker and the device step counter come back with the
    # moments, so the resumed run continues bit for bit (an optimizer made
    # with another initial scale takes the saved one); a plain optimizer
    # loading the same checkpoint takes the step count per parameter, and a
    # loss-scaled one loading a plain checkpoint takes its count
    from mixed_precision_optimizer_mta_amd import MtaOptimizer
    kw = dict(kind="adamw", lr=1e-3, weight_decay=0.1, max_norm=1.0,
              growth_interval=2)
    model_a = _model(13)
    opt_a = MtaOptimizer(model_a.parameters(), loss_scale=256.0, **kw)
    for t in range(1, 5):
        _scaled_grads(model_a, opt_a, t, inf_at=2)
        opt_a.step()
    sd = copy.deepcopy(opt_a.state_dict())
    amp_a = opt_a.amp.read()
    assert sd["mta_amp"] == amp_a and amp_a["step"] == 3
    assert all(s["step"] == 3 for s in sd["state"].values())
    model_b = _model(99)
    with torch.no_grad():
        for pb, pa in zip(model_b.parameters(), model_a.parameters()):
            pb.copy_(pa)
    opt_b = MtaOptimizer(model_b.parameters(), loss_scale=65536.0, **kw)
    opt_b.load_state_dict(sd)
    assert opt_b.amp.read() == amp_a
    for t in range(5, 9):
        for m, o in ((model_a, opt_a), (model_b, opt_b)):
            _scaled_grads(m, o, t, inf_at=7)
            o.step()
        torch.cuda.synchronize()
        assert opt_a.amp.read() == opt_b.amp.read(), t
        for pa, pb in zip(model_a.parameters(), model_b.parameters()):
            assert torch.equal(pa.detach().view(torch.int32),
                               pb.detach().view(torch.int32)), t
    plain = MtaOptimizer(_model(5).parameters(), **{k: v for k, v in
                                                     kw.items()
                                                     if k != "growth_interval"})
    plain.load_state_dict(sd)
    assert all(s["step"] == 3 for s in plain.state_dict()["state"].values())
    model_c = _model(17)
    opt_c = MtaOptimizer(model_c.parameters(), kind="adamw", lr=1e-3,
                         weight_decay=0.1, max_norm=1.0)
    for t in range(1, 3):
        _grads(model_c, t)
        opt_c.step()
    scaled = MtaOptimizer(_model(17).parameters(), loss_scale=512.0, **kw)
    scaled.load_state_dict(opt_c.state_dict())
    st = scaled.amp.read()
    assert (st["step"], st["scale"], st["found_inf"]) == (2, 512.0, 0.0)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_master_weights_with_a_no_decay_group_share_one_launch(dt):
    # a 16-bit model in the usual two groups: one list whose tensors carry
    # both their 16-bit parameter (the weight copy) and, for the biases, the
    # no-decay flag; masters and parameters bitwise against the oracle run
    # group by group (float16 loss-scaled, as a float16 run is)
    from mixed_precision_optimizer_mta_amd import MtaOptimizer
    model = _model(41).to(dt)
    params = list(model.parameters())
    mats = [p for p in params if p.dim() == 2]
    vecs = [p for p in params if p.dim() == 1]
    groups = [{"params": mats, "weight_decay": 0.1},
              {"params": vecs, "weight_decay": 0.0}]
    gt = O.BF16 if dt == torch.bfloat16 else O.F16
    scaled = dt == torch.float16
    opt = MtaOptimizer(groups, kind="adamw", lr=1e-3, max_norm=1.0,
                       master_weights=True,
                       loss_scale=1024.0 if scaled else None)
    ost = [[O.Tensor(_host(p.float()).ravel(), None,
                     np.zeros(p.numel(), np.float32),
                     np.zeros(p.numel(), np.float32),
                     np.zeros(p.numel(), np.uint16), gt)
            for p in g["params"]] for g in groups]
    amp_o = O.AmpState(1024.0) if scaled else None
    for t in range(1, 4):
        torch.manual_seed(5000 + t)
        x = torch.randn(32, 300, device="cuda", dtype=dt)
        y = torch.randint(0, 10, (32,), device="cuda")
        model.zero_grad(set_to_none=False)
        loss = torch.nn.functional.cross_entropy(model(x).float(), y)
        (loss * opt.loss_scale if scaled else loss).backward()
        for g, og in zip(groups, ost):
            for p, o in zip(g["params"], og):
                o.g = _bits16(p.grad)
        opt.step()
        torch.cuda.synchronize()
        assert len(opt._plan["updates"]) == 1
        coef = np.float32(opt.last_coef.item())
        for g, og in zip(groups, ost):
            rule = dict(kind="adamw", lr=1e-3, beta1=0.9, beta2=0.999,
                        eps=1e-8, weight_decay=g["weight_decay"],
                        momentum=0.0)
            if scaled:
                one = O.AmpState(amp_o.scale, amp_o.step, amp_o.tracker)
                _, _, found = O.amp_opt_step_(og, rule, gt, 0, 0, one, 1.0,
                                              coef=coef)
                assert not found
            else:
                O.opt_step_(og, rule, gt, 0, 0, t, coef=coef)
        if scaled:
            amp_o.update(2.0, 0.5, 2000)
        for g, og in zip(groups, ost):
            for p, o in zip(g["params"], og):
                w = opt.state[p]["master_weight"]
                assert np.array_equal(_host(w).ravel().view(np.uint32),
                                      o.w.view(np.uint32)), (t, "master")
                assert np.array_equal(_bits16(p), o.w16), (t, "parameter")


def test_works_under_torch_grad_scaler():
    # PyTorch's own loss-scaling loop drives MtaOptimizer like any
    # optimizer: GradScaler unscales the gradients in place, skips the step
    # on an overflow and adjusts its scale; the parameters follow
    # torch.optim.AdamW under the same scaler within rounding (PyTorch's
    # lerp uses an fma), and the overflow step leaves them untouched
    from mixed_precision_optimizer_mta_amd import MtaOptimizer
    a = _model(23)
    b = copy.deepcopy(a)
    opt_a = MtaOptimizer(a.parameters(), kind="adamw", lr=1e-3,
                         weight_decay=0.1)
    opt_b = torch.optim.AdamW(b.parameters(), lr=1e-3, weight_decay=0.1,
                              foreach=False)
    sc_a = torch.amp.GradScaler("cuda", init_scale=1024.0, growth_interval=2)
    sc_b = torch.amp.GradScaler("cuda", init_scale=1024.0, growth_interval=2)
    for t in range(1, 7):
        before = [p.detach().clone() for p in a.parameters()]
        for m, opt, sc in ((a, opt_a, sc_a), (b, opt_b, sc_b)):
            torch.manual_seed(4000 + t)
            x = torch.randn(32, 300, device="cuda")
            y = torch.randint(0, 10, (32,), device="cuda")
            m.zero_grad(set_to_none=False)
            loss = torch.nn.functional.cross_entropy(m(x), y)
            sc.scale(loss).backward()
            if t == 3:
                next(m.parameters()).grad[0, 0] = float("inf")
            sc.step(opt)
            sc.update()
        torch.cuda.synchronize()
        assert sc_a.get_scale() == sc_b.get_scale(), t
        for pa, pb, p0 in zip(a.parameters(), b.parameters(), before):
            if t == 3:
                assert torch.equal(pa.detach(), p0), "overflow step taken"
            torch.testing.assert_close(pa, pb, rtol=1e-5, atol=1e-7)


def test_default_zero_grad_loop_keeps_one_plan():
    # the plain PyTorch loop: backward, step, zero_grad() with the default
    # arguments.  The optimizer's zero_grad zeroes in place by default, so
    # the gradients keep their addresses and every step after the first
    # reuses the device tables; set_to_none=True reallocates them and costs
    # a rebuild at the next step
    from mixed_precision_optimizer_mta_amd import MtaOptimizer
    model = _model()
    opt = MtaOptimizer(model.parameters(), kind="adamw", lr=1e-3,
                       weight_decay=0.01, max_norm=1.0)
    x = torch.randn(64, 300, device="cuda")
    y = torch.randint(0, 10, (64,), device="cuda")
    for _ in range(6):
        torch.nn.functional.cross_entropy(model(x), y).backward()
        opt.step()
        opt.zero_grad()
    torch.cuda.synchronize()
    built = opt.tables_built            # the update list and the norm list
    assert built == 2, built
    assert all(p.grad is not None and not p.grad.any()
               for p in model.parameters())
    opt.zero_grad(set_to_none=True)
    torch.nn.functional.cross_entropy(model(x), y).backward()
    opt.step()
    torch.cuda.synchronize()
    assert opt.tables_built == built + 2
