"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Every test here runs the hot path on the device -- mta_scale (deferred or
in place), mta_clip_norm, mta_adamw_step -- and compares with the oracle
element by element (lockstep protocol, see parity_util).  Every list, the
full-size workloads included, is compared on every element.
"""

import numpy as np
import pytest
import torch

import oracle as O
from mixed_precision_optimizer_mta_amd import workloads as WL

pytestmark = pytest.mark.gpu

from parity_util import (check_norm, compare, expected_tiles,  # noqa: E402
                         lockstep, make_list, oracle_grads, oracle_state)


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import mixed_precision_optimizer_mta_amd as M
    M.lib()          # libmta.so must load; there is no other path
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------- small lists

SMALL = {
    "gpt2_124m": WL.gpt2_sizes(1000, 64, 128, 2, 256),
    "gpt2_124m_bf16g": WL.gpt2_sizes(1000, 64, 128, 2, 256),
    "gpt2_124m_f16amp": WL.gpt2_sizes(1000, 64, 128, 2, 256),
    "gpt2_xl": WL.gpt2_sizes(1000, 96, 64, 3, 384),
}


def small(name):
    wl = WL.get(name)
    if name == "tiny":
        return wl
    if name == "ragged":
        rng = np.random.default_rng(77)
        u = rng.random(300)
        sizes = [int(max(1, np.floor(2.0 ** (14 * x)))) for x in u]
        sizes += [1000 * 64] * 2
        zero = [int(i) for i in rng.permutation(300)[:3]]
        return WL.scaled_down(wl, sizes, zero_grad=zero)
    return WL.scaled_down(wl, SMALL[name])


@pytest.mark.parametrize("name", WL.NAMES)
def test_small_lists_lockstep(name):
    wl = small(name)
    steps = wl.steps if name != "gpt2_124m" else 5
    worst = lockstep(wl, steps, check_guards=True)
    # the arithmetic is the same sequence of correctly rounded operations on
    # both sides: expect identical bits, not just the tolerance
    assert worst == {"w": 0, "m": 0, "v": 0}, worst


ALL_KINDS = [(g, m, v) for g in (0, 1, 2) for m in (0, 1) for v in (0, 1)]


@pytest.mark.parametrize("gtype,mkind,vkind", ALL_KINDS)
def test_edge_sizes_every_kind(gtype, mkind, vkind):
    sizes = [0, 1, 2, 3, 7, 8, 9, 15, 17, 4095, 4096, 4097, 8191, 8193,
             3 * 4096 + 5]
    wl = WL.Workload("edges", sizes, gtype, mkind, vkind, steps=3,
                     g_sigma=0.3, ident=11)
    worst = lockstep(wl, 3, check_guards=True)
    assert worst == {"w": 0, "m": 0, "v": 0}, worst


UNALIGNED_KINDS = [(0, 0, 0), (1, 1, 0), (1, 1, 1), (2, 0, 1)]


@pytest.mark.parametrize("gtype,mkind,vkind", UNALIGNED_KINDS)
def test_unaligned_tensors_peel_a_head_then_vectorize(gtype, mkind, vkind):
    # element offsets of 1 (mod 8) put every buffer 4 or 2 bytes off 16-byte
    # alignment, all by the same element count: a head of up to 63 elements
    # brings every buffer to a cache-line boundary, and the rest of the
    # tensor runs on the vector path
    sizes = [5000, 4096, 33, 9000, 7, 3]
    offsets, pos = [], 0
    for n in sizes:
        offsets.append(pos + 1)             # 1 (mod 8): 4 or 2 bytes off
        pos += -(-(n + 1) // 8) * 8 + 8
    wl = WL.Workload("unaligned", sizes, gtype, mkind, vkind, steps=2,
                     ident=12)
    arena = WL.Arena(wl, "cuda", offsets)
    L = make_list(arena)
    info = L.info()
    assert (info["tiles"], info["vector_tensors"]) == \
        expected_tiles(arena.entries(), gtype, mkind, vkind)
    assert info["vector_tensors"] == 4      # 7 and 3: all head
    assert info["tiles"] == 3 + 2 + 2 + 4 + 1 + 1
    L.close()
    worst = lockstep(wl, 2, offsets=offsets, check_guards=True)
    assert worst == {"w": 0, "m": 0, "v": 0}, worst


@pytest.mark.parametrize("gtype,mkind,vkind", UNALIGNED_KINDS)
def test_disagreeing_misalignments_take_the_element_path(gtype, mkind, vkind):
    # g one element further than w, m, v: no head length aligns both
    sizes = [5000, 4096, 33, 9000]
    wl = WL.Workload("unaligned2", sizes, gtype, mkind, vkind, steps=2,
                     ident=14)
    arena = WL.Arena(wl, "cuda", g_shift=1)
    L = make_list(arena)
    info = L.info()
    assert info["vector_tensors"] == 0
    assert info["tiles"] == 2 + 1 + 1 + 3
    L.close()
    worst = lockstep(wl, 2, check_guards=True, g_shift=1)
    assert worst == {"w": 0, "m": 0, "v": 0}, worst


@pytest.mark.parametrize("gtype,mkind,vkind", [(0, 0, 0), (1, 1, 0),
                                               (2, 1, 1)])
def test_flat_buffer_layout(gtype, mkind, vkind):
    # tensors back to back in one buffer per kind, as a flat parameter
    # buffer holds them: every start offset mod 8 occurs
    rng = np.random.default_rng(15)
    sizes = [int(x) for x in rng.integers(1, 12000, size=40)]
    offsets = np.concatenate([[0], np.cumsum(sizes)[:-1]]).tolist()
    wl = WL.Workload("flat", sizes, gtype, mkind, vkind, steps=2,
                     g_sigma=0.05, ident=16)
    arena = WL.Arena(wl, "cuda", offsets)
    L = make_list(arena)
    info = L.info()
    assert (info["tiles"], info["vector_tensors"]) == \
        expected_tiles(arena.entries(), gtype, mkind, vkind)
    assert info["vector_tensors"] >= sum(1 for n in sizes if n >= 64)
    L.close()
    worst = lockstep(wl, 2, offsets=offsets, check_guards=True)
    assert worst == {"w": 0, "m": 0, "v": 0}, worst


def test_no_clip_and_clip_at_one_agree():
    wl = small("gpt2_124m")
    wl = WL.scaled_down(wl, wl.sizes)
    wl.max_norm = 1e30
    a = lockstep(wl, 2)
    b = lockstep(wl, 2, clip=False)
    assert a == b == {"w": 0, "m": 0, "v": 0}


def test_nonfinite_gradients_propagate():
    for bad in (np.nan, np.inf):
        wl = WL.Workload("nonfinite", [4096 * 2 + 7, 100], 0, 0, 0, steps=1,
                         ident=13)
        arena = WL.Arena(wl, "cuda")
        arena.fill_weights()
        arena.fill_grads(1)
        arena.g[arena.offsets[0] + 5] = float(bad)
        ostate = oracle_state(arena)
        L = make_list(arena)
        nd = torch.zeros(1, device="cuda")
        cd = torch.zeros(1, device="cuda")
        L.clip_norm(1.0, nd, cd)
        L.adamw_step(wl.hparams, 1, cd)
        torch.cuda.synchronize()
        no = O.norm([o.g for o in ostate], 0)
        check_norm(np.float32(nd.item()), np.float32(cd.item()), no, 1.0)
        O.step_(ostate, 0, 0, 0, wl.lr, wl.beta1, wl.beta2, wl.eps,
                wl.weight_decay, 1, coef=np.float32(cd.item()))
        compare(arena, ostate)
        L.close()


def test_empty_list_and_empty_tensors():
    from mixed_precision_optimizer_mta_amd import MtaList
    L = MtaList([], entries=[], gtype=0, mkind=0, vkind=0)
    nd = torch.full((1,), 7.0, device="cuda")
    cd = torch.full((1,), 7.0, device="cuda")
    L.clip_norm(1.0, nd, cd)
    L.adamw_step(dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                      weight_decay=0.0), 1, cd)
    torch.cuda.synchronize()
    assert nd.item() == 0.0 and cd.item() == 1.0
    assert L.info()["tiles"] == 0
    L.close()
    wl = WL.Workload("zeros", [0, 0, 5, 0], 0, 1, 1, steps=2, ident=14)
    assert lockstep(wl, 2) == {"w": 0, "m": 0, "v": 0}


def test_deferred_scale_equals_in_place_for_f32():
    wl = WL.scaled_down(small("gpt2_124m"), SMALL["gpt2_124m"])
    res = []
    for defer in (True, False):
        arena = WL.Arena(wl, "cuda")
        arena.fill_weights()
        arena.fill_grads(1)
        L = make_list(arena)
        cd = torch.zeros(1, device="cuda")
        L.scale(0.3, defer=defer)
        L.clip_norm(0.05, None, cd)
        L.adamw_step(wl.hparams, 1, cd)
        torch.cuda.synchronize()
        res.append((arena.w.clone(), arena.m.clone(), arena.v.clone(),
                    cd.item()))
        L.close()
    (w1, m1, v1, c1), (w2, m2, v2, c2) = res
    assert c1 == c2
    assert torch.equal(w1, w2) and torch.equal(m1, m2) and torch.equal(v1, v2)


@pytest.mark.parametrize("gtype", [0, 1, 2])
def test_in_place_scale_matches_oracle(gtype):
    sizes = [1, 4096 * 3, 4097, 77]
    wl = WL.Workload("scale", sizes, gtype, 0, 0, steps=1, g_sigma=50.0,
                     ident=15)
    arena = WL.Arena(wl, "cuda")
    arena.fill_grads(1)
    gs = oracle_grads(arena)
    L = make_list(arena)
    for s in (2.0 ** -16, 0.3):
        L.scale(s, defer=False)
        torch.cuda.synchronize()
        for g in gs:
            O.scale_(g, gtype, s)
        got = oracle_grads(arena)
        for a, b in zip(got, gs):
            assert np.array_equal(a.view(np.uint16 if gtype else np.uint32),
                                  b.view(np.uint16 if gtype else np.uint32))
    L.close()


@pytest.mark.parametrize("gtype", [0, 1, 2])
def test_in_place_scale_many_tiles_and_flat_offsets(gtype):
    # over 2,200 tiles, one workgroup each: the runs of 32 tiles per XCD
    # (the first 2,048 workgroups) and the remainder taken in order, plus
    # tensors at odd flat offsets (peeled heads) and ragged tails; nothing
    # outside the tensors is written
    sizes = [4096 * 2200 + 5, 3, 4096 * 3 + 1, 300]
    offsets = [1]
    for n in sizes[:-1]:
        offsets.append(offsets[-1] + n)
    wl = WL.Workload("scale2", sizes, gtype, 0, 0, steps=1, g_sigma=50.0,
                     ident=17)
    arena = WL.Arena(wl, "cuda", offsets)
    arena.fill_grads(1)
    ity = torch.int32 if gtype == 0 else torch.int16
    before = arena.g.view(ity).clone()
    gs = oracle_grads(arena)
    L = make_list(arena)
    assert L.info()["tiles"] > 2048 + 100
    for s in (0.3, 2.0 ** 20):
        L.scale(s, defer=False)
        torch.cuda.synchronize()
        for g in gs:
            O.scale_(g, gtype, s)
        for a, b in zip(oracle_grads(arena), gs):
            assert np.array_equal(a.view(np.uint16 if gtype else np.uint32),
                                  b.view(np.uint16 if gtype else np.uint32))
    inside = torch.zeros(arena.total, dtype=torch.bool, device="cuda")
    for o, n in zip(offsets, sizes):
        inside[o:o + n] = True
    assert not bool(((arena.g.view(ity) != before) & ~inside).any())
    L.close()


def test_deferred_scale_state_machine():
    from mixed_precision_optimizer_mta_amd import MtaError
    wl = WL.Workload("defer", [100], 1, 0, 0, steps=1, ident=16)
    arena = WL.Arena(wl, "cuda")
    L = make_list(arena)
    L.scale(0.5, defer=True)
    with pytest.raises(MtaError) as e:
        L.scale(0.5, defer=True)
    assert e.value.code == -6
    with pytest.raises(MtaError):
        L.adamw_step(dict(lr=1e-3, beta1=1.0, beta2=0.999, eps=1e-8,
                          weight_decay=0.0), 1)
    L.adamw_step(wl.hparams, 1)         # consumes the factor
    L.scale(0.5, defer=True)            # allowed again
    L.adamw_step(wl.hparams, 2)
    torch.cuda.synchronize()
    L.close()


def test_deterministic_and_rearmed_ticket():
    wl = WL.scaled_down(small("gpt2_124m"), SMALL["gpt2_124m"])
    arena = WL.Arena(wl, "cuda")
    arena.fill_weights()
    arena.fill_grads(1)
    L = make_list(arena)
    norms = []
    nd = torch.zeros(1, device="cuda")
    cd = torch.zeros(1, device="cuda")
    for _ in range(20):
        L.clip_norm(1.0, nd, cd)
        norms.append(nd.clone())
    torch.cuda.synchronize()
    bits = {int(n.view(torch.int32).item()) for n in norms}
    assert len(bits) == 1
    # two identical states stepped separately end in identical bits
    w0, m0, v0 = arena.w.clone(), arena.m.clone(), arena.v.clone()
    L.adamw_step(wl.hparams, 1, cd)
    w1, m1, v1 = arena.w.clone(), arena.m.clone(), arena.v.clone()
    arena.w.copy_(w0), arena.m.copy_(m0), arena.v.copy_(v0)
    L.adamw_step(wl.hparams, 1, cd)
    torch.cuda.synchronize()
    assert torch.equal(w1, arena.w) and torch.equal(m1, arena.m) and \
        torch.equal(v1, arena.v)
    L.close()


def test_tensor_order_does_not_change_results():
    wl = small("ragged")
    arena = WL.Arena(wl, "cuda")
    arena.fill_weights()
    arena.fill_grads(1)
    ents = arena.entries()
    coef = torch.full((1,), 0.37, device="cuda")
    outs = []
    for perm in (np.arange(len(ents)), np.random.default_rng(3).permutation(
            len(ents))):
        arena.fill_weights()
        from mixed_precision_optimizer_mta_amd import MtaList
        L = MtaList([], entries=[ents[i] for i in perm], gtype=wl.gtype,
                    mkind=wl.mkind, vkind=wl.vkind)
        L.scale(wl.scale, defer=True)
        L.adamw_step(wl.hparams, 1, coef)
        torch.cuda.synchronize()
        outs.append((arena.w.clone(), arena.m.clone(), arena.v.clone()))
        L.close()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


# ---------------------------------------------------------------- full size

def test_full_tiny():
    assert lockstep(WL.get("tiny"), 10) == {"w": 0, "m": 0, "v": 0}


def test_full_gpt2_124m_every_element():
    wl = WL.get("gpt2_124m")
    worst = lockstep(wl, wl.steps)
    assert worst == {"w": 0, "m": 0, "v": 0}, worst


@pytest.mark.timeout(600)
def test_full_gpt2_124m_bf16_grads_100_steps_every_element():
    # the oracle keeps the whole list in lockstep for all 100 steps; the
    # norm is checked at every step and every element of w, m, v after
    # steps 1, 2, 10, 20, ..., 100
    wl = WL.get("gpt2_124m_bf16g")
    worst = lockstep(wl, wl.steps,
                     compare_steps={1, 2} | set(range(10, 101, 10)))
    assert worst == {"w": 0, "m": 0, "v": 0}, worst


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", ["gpt2_124m", "gpt2_124m_bf16g",
                                  "gpt2_xl_shard0of8"])
def test_full_list_on_the_element_path_every_element(name):
    # the gradients one element off w, m and v: no tensor can reach the
    # vector path, so every tile of the full list takes one-element
    # accesses (the path of tail tiles and unaligned tensors)
    wl = WL.get(name)
    arena = WL.Arena(wl, "cuda", g_shift=1)
    L = make_list(arena)
    assert L.info()["vector_tensors"] == 0
    L.close()
    del arena
    worst = lockstep(wl, 2, g_shift=1)
    assert worst == {"w": 0, "m": 0, "v": 0}, worst


@pytest.mark.timeout(600)
def test_full_gpt2_xl_packed_every_element():
    wl = WL.get("gpt2_xl")
    worst = lockstep(wl, wl.steps)
    assert worst == {"w": 0, "m": 0, "v": 0}, worst


@pytest.mark.timeout(600)
def test_full_ragged_every_element():
    wl = WL.get("ragged")
    worst = lockstep(wl, wl.steps)
    assert worst == {"w": 0, "m": 0, "v": 0}, worst


@pytest.mark.parametrize("name", ["gpt2_124m", "gpt2_124m_bf16g", "gpt2_xl",
                                  "ragged"])
def test_independent_mode_report(name):
    """Informational run: the oracle uses its own clip coefficient, from
    f32 of its own norm, instead of the device's.  The device and oracle
    norms agree to well within 1e-6, so the runs stay within a few ulp;
    the distances are printed."""
    from parity_util import bf16_ulp, dev_bf16_bits, dev_f32, f32_ulp
    wl = small(name)
    arena = WL.Arena(wl, "cuda")
    arena.fill_weights()
    L = make_list(arena)
    ostate = oracle_state(arena)
    nd = torch.zeros(1, device="cuda")
    cd = torch.zeros(1, device="cuda")
    worst = {"w": 0, "m": 0, "v": 0, "coef": 0}
    for t in range(1, 6):
        arena.fill_grads(t)
        for o, g in zip(ostate, oracle_grads(arena)):
            o.g = g
        if wl.scale != 1.0:
            L.scale(wl.scale, defer=True)
        L.clip_norm(wl.max_norm, nd, cd)
        L.adamw_step(wl.hparams, t, cd)
        torch.cuda.synchronize()
        _, c_own = O.step_(ostate, wl.gtype, wl.mkind, wl.vkind, wl.lr,
                           wl.beta1, wl.beta2, wl.eps, wl.weight_decay, t,
                           s=wl.scale, max_norm=wl.max_norm)
        worst["coef"] = max(worst["coef"], int(f32_ulp(
            np.array([cd.item()], np.float32),
            np.array([c_own], np.float32)).max()))
        for i, o in enumerate(ostate):
            n = wl.sizes[i]
            if n == 0:
                continue
            worst["w"] = max(worst["w"], int(f32_ulp(
                dev_f32(arena.view("w", i)), o.w).max()))
            for b, kind, ob in (("m", wl.mkind, o.m), ("v", wl.vkind, o.v)):
                dv = arena.view(b, i)
                if kind == WL.MOM_BF16X2:
                    d = bf16_ulp(dev_bf16_bits(dv), O.unpack_words(ob, n))
                else:
                    d = f32_ulp(dev_f32(dv), ob)
                worst[b] = max(worst[b], int(d.max()))
    L.close()
    print(f"independent mode {name}: worst {worst}", flush=True)
    assert worst["coef"] <= 8 and worst["w"] <= 4, worst
    assert worst["m"] <= 64 and worst["v"] <= 64, worst


@pytest.mark.parametrize("name", ["gpt2_124m", "gpt2_124m_bf16g",
                                  "gpt2_124m_f16amp"])
def test_norm_cache_policy_changes_no_bits(monkeypatch, name):
    # the norm's kept tiles (allocating loads) are a cache policy only:
    # every tile kept, none kept, or the default cut give the same norm,
    # coefficient and update, bit for bit, for every gradient type
    wl = small(name)
    wl = WL.scaled_down(wl, wl.sizes)
    wl.amp = False
    results = []
    for keep in (None, "0", "100000"):
        if keep is None:
            monkeypatch.delenv("MTA_NORM_KEEP_MIB", raising=False)
        else:
            monkeypatch.setenv("MTA_NORM_KEEP_MIB", keep)
        arena = WL.Arena(wl, "cuda")
        arena.fill_weights()
        arena.fill_grads(1)
        L = make_list(arena)
        info = L.info()
        if keep == "0":
            assert info["norm_kept_tiles"] == 0
        else:                      # a small list: kept whole by default
            assert info["norm_kept_tiles"] == info["tiles"]
        nd = torch.zeros(1, device="cuda")
        cd = torch.zeros(1, device="cuda")
        L.clip_norm(wl.max_norm, nd, cd)
        L.adamw_step(wl.hparams, 1, cd)
        torch.cuda.synchronize()
        results.append((nd.view(torch.int32).item(),
                        cd.view(torch.int32).item(),
                        arena.w.view(torch.int32).clone()))
        L.close()
    for r in results[1:]:
        assert r[:2] == results[0][:2]
        assert torch.equal(r[2], results[0][2])


def test_norm_keeps_the_last_256_mib_of_the_124m_list(monkeypatch):
    monkeypatch.delenv("MTA_NORM_KEEP_MIB", raising=False)
    wl = WL.get("gpt2_124m")
    arena = WL.Arena(wl, "cuda")
    L = make_list(arena)
    info = L.info()
    kept = info["norm_kept_tiles"]
    # float32 gradients of 498 MB: the last 256 MiB worth of tiles (a few
    # of them bias tiles shorter than 4096 elements)
    assert 0 < kept < info["tiles"]
    assert (256 << 20) - 4096 * 4 < kept * 4096 * 4 <= (256 << 20) + \
        64 * 4096 * 4
    L.close()


@pytest.mark.timeout(300)
def test_full_gpt2_xl_shard_in_a_flat_buffer_every_element():
    # one GPU's eighth of the 1.56B list, its 35 pieces back to back as a
    # sharded flat buffer holds them (pieces start at any element)
    wl = WL.get("gpt2_xl_shard0of8")
    offsets = [0]
    for n in wl.sizes[:-1]:
        offsets.append(offsets[-1] + n)
    worst = lockstep(wl, wl.steps, offsets=offsets)
    assert worst == {"w": 0, "m": 0, "v": 0}, worst
