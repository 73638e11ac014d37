"""MtaOptimizer argument checks that need no GPU."""
import pytest
import torch

from mixed_precision_optimizer_mta_amd import MtaOptimizer


def _params():
    return [torch.nn.Parameter(torch.zeros(10))]


def test_rejects_unknown_kind_and_packed_sgd():
    with pytest.raises(ValueError):
        MtaOptimizer(_params(), kind="lamb")
    with pytest.raises(ValueError):
        MtaOptimizer(_params(), kind="sgd", packed_moments=True)


def test_step_refuses_cpu_parameters_before_any_library_call():
    ps = _params()
    ps[0].grad = torch.zeros(10)
    opt = MtaOptimizer(ps, kind="adamw", max_norm=1.0)
    with pytest.raises(TypeError):
        opt.step()


def test_step_without_gradients_is_a_no_op():
    ps = _params()
    opt = MtaOptimizer(ps, kind="sgd", lr=0.1)
    assert opt.step() is None
    assert torch.equal(ps[0].detach(), torch.zeros(10))


def test_master_weights_refuse_cpu_and_plain_mode_refuses_16_bit():
    ps = _params()
    ps[0].grad = torch.zeros(10)
    with pytest.raises(TypeError):       # parameters off the GPU
        MtaOptimizer(ps, master_weights=True).step()
    h = [torch.nn.Parameter(torch.zeros(10, dtype=torch.bfloat16))]
    h[0].grad = torch.zeros(10, dtype=torch.bfloat16)
    with pytest.raises(TypeError):       # 16-bit without master weights
        MtaOptimizer(h).step()


def test_parameter_sets_follow_the_hyperparameters():
    # groups with equal lr, betas, eps and momentum share a launch when at
    # most one nonzero weight decay appears among them; the zero-decay
    # groups' tensors are the flagged ones
    def groups(*specs):
        return [dict(params=_params(), **s) for s in specs]

    def sets(opt):
        return opt._merge_sig()

    opt = MtaOptimizer(groups({"weight_decay": 0.1}, {"weight_decay": 0.0}),
                       kind="adamw", lr=1e-3)
    assert sets(opt) == ((0, False), (0, True))
    # another nonzero decay: each group alone
    opt.param_groups[1]["weight_decay"] = 0.05
    assert sets(opt) == ((0, False), (1, False))
    # equal decays share again; so do groups whose decays are all 0
    opt.param_groups[1]["weight_decay"] = 0.1
    assert sets(opt) == ((0, False), (0, False))
    # a different lr (or betas, eps, momentum) separates
    opt.param_groups[1]["lr"] = 2e-3
    assert sets(opt) == ((0, False), (1, False))
    opt = MtaOptimizer(groups({"weight_decay": 0.0}, {"weight_decay": 0.1},
                              {"weight_decay": 0.0, "betas": (0.8, 0.9)},
                              {"weight_decay": 0.0}),
                       kind="adamw", lr=1e-3)
    assert sets(opt) == ((0, True), (0, False), (2, True), (0, True))
    # two nonzero decays in one bucket: none of that bucket's groups merge
    opt.param_groups[3]["weight_decay"] = 0.2
    assert sets(opt) == ((0, True), (1, False), (2, True), (3, False))
