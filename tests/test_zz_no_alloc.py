"""mta_clip_norm_noalloc, the norm for callers that cannot allocate device
memory, against mta_clip_norm on the same gradients: the same norm and
coefficient bits (same kernel, same launch shape), the norm within 1e-6 of
the oracle's, on two calls in a row, the second with a smaller input; and
a list too large for its scratch refused before any device work."""
import numpy as np
import pytest
import torch

import oracle as O
from mixed_precision_optimizer_mta_amd import _binding as B
from mixed_precision_optimizer_mta_amd import workloads as WL

pytestmark = pytest.mark.gpu

from parity_util import check_norm, make_list, oracle_grads  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    B.lib()
    yield
    torch.cuda.synchronize()


def _bits(t):
    return int(t.view(torch.int32).item())


def _f32(bits):
    return np.array([bits], np.int32).view(np.float32)[0]


def _via_list(wl, arena, scale, max_norm):
    L = make_list(arena)
    nd = torch.full((1,), -1.0, device="cuda")
    cd = torch.full((1,), -1.0, device="cuda")
    if scale != 1.0:
        L.scale(scale, defer=True)
    L.clip_norm(max_norm, nd, cd)
    torch.cuda.synchronize()
    L.close()
    return _bits(nd), _bits(cd), nd.item()


def _noalloc(wl, arena, scale, max_norm):
    # gradients only: w, m, v are not needed
    ents = [(None, g, None, None, n) for (_, g, _, _, n) in arena.entries()]
    nd = torch.full((1,), -1.0, device="cuda")
    cd = torch.full((1,), -1.0, device="cuda")
    B.mta_clip_norm_noalloc(ents, wl.gtype, scale, max_norm, nd.data_ptr(),
                            cd.data_ptr(),
                            torch.cuda.current_stream().cuda_stream)
    return _bits(nd), _bits(cd), nd.item()


def _case(sizes, gtype, scale, ident):
    wl = WL.Workload("noalloc", sizes, gtype, 0, 0, steps=1,
                     g_mult=1.0 / scale, ident=ident)
    arena = WL.Arena(wl, "cuda")
    arena.fill_grads(1)
    return wl, arena


@pytest.mark.parametrize("gtype", [WL.F32, WL.BF16, WL.F16])
def test_noalloc_norm_equals_the_list_norm_twice_second_smaller(gtype):
    scale = 2.0 ** -8 if gtype != WL.F32 else 1.0
    first = [4096 * 900 + 7, 3, 4096 * 40, 1]       # 943 tiles, grid-sized
    second = [4096 * 5 + 1, 77]                     # far fewer tiles
    for k, sizes in enumerate((first, second)):
        wl, arena = _case(sizes, gtype, scale, 91 + k)
        got = _noalloc(wl, arena, scale, 1.0)
        want = _via_list(wl, arena, scale, 1.0)
        assert got[:2] == want[:2], (k, got, want)
        no = O.norm(oracle_grads(arena), gtype, scale)
        check_norm(np.float32(got[2]), _f32(got[1]), no, 1.0,
                   f"noalloc call {k}")


def test_noalloc_empty_and_zero_gradients():
    # zero gradients: norm 0, coefficient 1 (as mta_clip_norm gives)
    wl, arena = _case([0, 5, 0], WL.F32, 1.0, 95)
    arena.g.zero_()
    got = _noalloc(wl, arena, 1.0, 1.0)
    assert got[:2] == _via_list(wl, arena, 1.0, 1.0)[:2]
    assert got[2] == 0.0 and _f32(got[1]) == 1.0
    # no tensors at all
    nd = torch.full((1,), -1.0, device="cuda")
    cd = torch.full((1,), -1.0, device="cuda")
    B.mta_clip_norm_noalloc([], WL.F32, 1.0, 1.0, nd.data_ptr(),
                            cd.data_ptr())
    assert nd.item() == 0.0 and cd.item() == 1.0


def test_noalloc_refuses_a_list_larger_than_its_scratch():
    # 2^33 elements in one tensor need 2^21 tiles: more than the 32 MiB
    # scratch's table holds.  The pointers are never dereferenced: the
    # size check comes before any device work
    n = 1 << 33
    ents = [(None, 1 << 40, None, None, n)]
    cd = torch.zeros(1, device="cuda")
    with pytest.raises(B.MtaError) as e:
        B.mta_clip_norm_noalloc(ents, WL.BF16, 1.0, 1.0, None, cd.data_ptr())
    assert e.value.code == -1
    assert "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert cd.item() == 0.0                          # nothing ran
