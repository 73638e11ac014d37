"""A loss-scaled step keeps every value it needs on the device (scale,
found-inf flag, step counter, norm, clip coefficient), so the whole step --
mta_amp_clip_norm, mta_amp_step / mta_amp_adamw_step, mta_amp_update -- can
be captured once in a HIP graph and replayed every iteration.  Each replay
here is checked bit for bit against the same calls made eagerly on a twin
set of buffers, with eager work and synchronizations between the replays
and overflow steps among them.  None of the calls records a memset: the
norm kernel re-arms its own ticket.
"""
import numpy as np
import pytest
import torch

from mixed_precision_optimizer_mta_amd import workloads as WL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import mixed_precision_optimizer_mta_amd as M
    M.lib()
    yield
    torch.cuda.synchronize()


def _twin(wl, kind):
    from mixed_precision_optimizer_mta_amd import AmpState, MtaList
    arena = WL.Arena(wl, "cuda")
    arena.fill_weights()
    has_m, has_v = kind != "sgd", kind in ("adamw", "adam")
    ents = [(w, g, m if has_m else None, v if has_v else None, n)
            for (w, g, m, v, n) in arena.entries()]
    L = MtaList([], entries=ents, gtype=wl.gtype, mkind=wl.mkind,
                vkind=wl.vkind)
    return arena, L, AmpState(wl.amp_scale), torch.zeros(1, device="cuda"), \
        torch.zeros(1, device="cuda")


@pytest.mark.parametrize("kind", ["adamw", "adam", "sgd", "momentum"])
def test_captured_loss_scaled_step_replays_like_eager_calls(kind):
    wl = WL.Workload("graph", [4096 * 5 + 3, 1000, 1, 4096], WL.F16,
                     WL.MOM_F32, WL.MOM_F32, steps=8, g_mult=512.0,
                     amp=True, amp_scale=512.0, amp_interval=2, ident=41)
    adam = kind in ("adamw", "adam")
    opt = dict(kind=kind, lr=1e-3 if adam else 0.05, beta1=0.9,
               beta2=0.999, eps=1e-8, weight_decay=0.1 if adam else 0.0,
               momentum=0.9, zero_grad=(kind == "momentum"))
    A = _twin(wl, kind)   # captured
    E = _twin(wl, kind)   # eager

    def one_step(parts):
        arena, L, amp, nd, cd = parts
        L.amp_clip_norm(wl.max_norm, amp, nd, cd)
        if kind == "adamw" and not opt["zero_grad"]:
            L.amp_adamw_step(wl.hparams, amp, cd)
        else:
            L.amp_step(opt, amp, cd)
        amp.update(wl.amp_growth, wl.amp_backoff, wl.amp_interval)

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            one_step(A)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # capturing ran nothing: the state is still the initial one
    assert A[2].read()["step"] == 0

    for t in range(1, 9):
        for arena in (A[0], E[0]):
            arena.fill_grads(t)
            if t in (3, 6):
                arena.g[arena.offsets[1] + 17] = float("inf")
        torch.cuda.synchronize()
        graph.replay()
        one_step(E)
        torch.cuda.synchronize()
        sa, se = A[2].read(), E[2].read()
        assert sa == se, (t, sa, se)
        for b in "wgmv":
            x, y = getattr(A[0], b), getattr(E[0], b)
            ity = torch.int32 if x.dtype == torch.float32 else torch.int16
            assert torch.equal(x.view(ity), y.view(ity)), (kind, t, b)
        for i in (3, 4):
            assert torch.equal(A[i], E[i]), (kind, t, i)
    st = A[2].read()
    assert st["step"] == 6 and st["scale"] != 512.0   # 2 skipped, grown
    for parts in (A, E):
        parts[1].close()


def test_replays_on_a_list_whose_tiles_span_the_grid_many_times():
    # a list with more tiles than the grid has workgroups: every replay
    # walks the tile table with a grid stride and re-arms the norm ticket
    wl = WL.Workload("graph_big", [4096 * 700 + 11, 333], WL.BF16,
                     WL.MOM_BF16X2, WL.MOM_F32, steps=5, g_mult=256.0,
                     amp=True, amp_scale=256.0, ident=42)
    A = _twin(wl, "adamw")
    E = _twin(wl, "adamw")

    def one_step(parts):
        arena, L, amp, nd, cd = parts
        L.amp_clip_norm(wl.max_norm, amp, nd, cd)
        L.amp_adamw_step(wl.hparams, amp, cd)
        amp.update()

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            one_step(A)
    torch.cuda.current_stream().wait_stream(side)
    for t in range(1, 6):
        for arena in (A[0], E[0]):
            arena.fill_grads(t)
        torch.cuda.synchronize()
        graph.replay()
        one_step(E)
        torch.cuda.synchronize()
        assert A[2].read() == E[2].read()
        assert torch.equal(A[3], E[3]) and torch.equal(A[4], E[4])
        for b in "wmv":
            x, y = getattr(A[0], b), getattr(E[0], b)
            ity = torch.int32 if x.dtype == torch.float32 else torch.int16
            assert torch.equal(x.view(ity), y.view(ity)), (t, b)
    assert np.isfinite(A[3].item())
    for parts in (A, E):
        parts[1].close()
