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
