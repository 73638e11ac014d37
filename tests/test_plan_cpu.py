"""mta_list_plan on the host (no GPU): the tile cuts of the list builder --
head peeling to a cache line or to 16 bytes, the element path when the
buffers' misalignments disagree, the norm's kept tiles -- checked against an
independent Python model, and the same argument errors as mta_list_create."""
import numpy as np
import pytest

import mixed_precision_optimizer_mta_amd as M
from mixed_precision_optimizer_mta_amd import workloads as WL

from parity_util import expected_tiles

BASE = [1 << 40, 2 << 40, 3 << 40, 4 << 40]   # far apart: no overlaps
SZ = {0: 4, 1: 2}


def sizes_of(gtype, mkind, vkind):
    return [4, 4 if gtype == 0 else 2, 2 if mkind else 4, 2 if vkind else 4]


def flat_entries(sizes, gtype, mkind, vkind, start=0):
    """Tensors back to back from element `start` of one flat buffer per
    kind (same element offsets in every buffer)."""
    sz = sizes_of(gtype, mkind, vkind)
    out, o = [], start
    for n in sizes:
        out.append(tuple(BASE[b] + sz[b] * o for b in range(4)) + (n,))
        o += n
    return out


@pytest.mark.parametrize("gtype,mkind,vkind", [(0, 0, 0), (1, 1, 0),
                                               (2, 0, 1), (1, 1, 1)])
@pytest.mark.parametrize("seed", range(6))
def test_flat_layouts_cut_as_the_model_says(gtype, mkind, vkind, seed):
    rng = np.random.default_rng(seed)
    sizes = [int(x) for x in rng.integers(0, 20000, size=60)]
    sizes += [int(x) for x in rng.integers(1, 9, size=10)]   # all head
    start = int(rng.integers(0, 64))
    ents = flat_entries(sizes, gtype, mkind, vkind, start=start)
    info = M.mta_list_plan(ents, gtype, mkind, vkind)
    assert (info["tiles"], info["vector_tensors"]) == \
        expected_tiles(ents, gtype, mkind, vkind)
    assert info["elements"] == sum(sizes)
    assert info["count"] == len(sizes)
    assert info["device"] == -1 and info["grid_update"] == 0
    # every tensor of 64 or more elements reaches a cache line
    assert info["vector_tensors"] >= sum(1 for n in sizes if n >= 64)


@pytest.mark.parametrize("gtype", [0, 1])
def test_disagreeing_misalignments_get_no_vector_tiles(gtype):
    # every tensor starts on a line in w, m and v, and g one element off
    sizes = [5000, 4096, 33, 9000]
    ents = []
    for i, n in enumerate(sizes):
        o = 4096 * 4 * i
        ents.append((BASE[0] + 4 * o, BASE[1] + SZ[gtype > 0] * (o + 1),
                     BASE[2] + 4 * o, BASE[3] + 4 * o, n))
    info = M.mta_list_plan(ents, gtype, 0, 0)
    assert info["vector_tensors"] == 0
    assert info["tiles"] == 2 + 1 + 1 + 3


def test_a_state_buffer_alone_can_block_the_vector_path():
    # SGD-style lists (no m, v) peel over w and g only
    ents = [(BASE[0] + 4, BASE[1] + 4, None, None, 10000)]
    info = M.mta_list_plan(ents, 0, 0, 0)
    assert info["vector_tensors"] == 1 and info["state_buffers"] == 0
    assert info["tiles"] == 1 + 3        # a 31-element head, then 3 tiles
    ents = [(BASE[0] + 4, BASE[1] + 4, BASE[2] + 8, None, 10000)]
    with pytest.raises(M.MtaError):      # m without v: a consistent list
        M.mta_list_plan(ents + [(BASE[0] + 4 * 20000, BASE[1] + 4 * 20000,
                                 None, None, 10)], 0, 0, 0)
    info = M.mta_list_plan([(BASE[0] + 4, BASE[1] + 4, BASE[2] + 8,
                             BASE[3] + 4, 10000)], 0, 0, 0)
    assert info["vector_tensors"] == 0   # m one element further than the rest


def _kept(sizes, gtype, mkind, vkind):
    """The norm's kept tiles of a padded list, from the tile lengths: the
    last tiles whose gradients fit 256 MiB, provided the update's element
    path (here the tail tiles shorter than 4096) before them moves at most
    64 MiB (w, g, m, v, read and written)."""
    lims = []
    for n in sizes:
        lims += [4096] * (n // 4096) + ([n % 4096] if n % 4096 else [])
    gsz = 4 if gtype == 0 else 2
    budget, k = 256 << 20, 0
    for lim in reversed(lims):
        if lim * gsz > budget:
            break
        budget -= lim * gsz
        k += 1
    upd = 8 + gsz + 2 * (2 if mkind else 4) + 2 * (2 if vkind else 4)
    tails = sum(lim for lim in lims[:len(lims) - k] if lim < 4096)
    return 0 if tails * upd > 64 << 20 else k


@pytest.mark.parametrize("name", ["gpt2_124m", "gpt2_124m_bf16g", "gpt2_xl",
                                  "ragged", "tiny", "gpt2_xl_shard0of8"])
def test_kept_tiles_follow_the_budget(name, monkeypatch):
    monkeypatch.delenv("MTA_NORM_KEEP_MIB", raising=False)
    wl = WL.get(name)
    sz = sizes_of(wl.gtype, wl.mkind, wl.vkind)
    ents, o = [], 0
    for n in wl.sizes:                  # padded: every tensor on a line
        ents.append(tuple(BASE[b] + sz[b] * o for b in range(4)) + (n,))
        o += -(-n // 128) * 128
    info = M.mta_list_plan(ents, wl.gtype, wl.mkind, wl.vkind)
    assert info["vector_tensors"] == sum(1 for n in wl.sizes if n)
    assert info["norm_kept_tiles"] == _kept(wl.sizes, wl.gtype, wl.mkind,
                                            wl.vkind)
    if name == "ragged":
        # 10.9M elements in tail tiles: 240 MB of element-path traffic
        assert info["norm_kept_tiles"] == 0
    if name in ("gpt2_124m", "gpt2_xl", "gpt2_xl_shard0of8"):
        assert 0 < info["norm_kept_tiles"] < info["tiles"]
    if name in ("gpt2_124m_bf16g", "tiny"):
        assert info["norm_kept_tiles"] == info["tiles"]   # all of it fits
    monkeypatch.setenv("MTA_NORM_KEEP_MIB", "0")
    assert M.mta_list_plan(ents, wl.gtype, wl.mkind,
                           wl.vkind)["norm_kept_tiles"] == 0


def test_an_unaligned_tensor_turns_the_kept_tiles_off(monkeypatch):
    # one 100M-element float32 tensor: the norm would keep its last 256 MiB
    # of gradients.  Aligned, the update takes every tile on the vector
    # path and the tiles are kept; with m one element off, every tile is on
    # the element path (28 B per element before the kept ones, far over
    # 64 MiB) and none is kept.
    monkeypatch.delenv("MTA_NORM_KEEP_MIB", raising=False)
    n = 100 * 2**20
    ok = M.mta_list_plan([tuple(BASE) + (n,)], 0, 0, 0)
    assert ok["vector_tensors"] == 1
    assert ok["norm_kept_tiles"] == (256 << 20) // (4096 * 4)
    off = M.mta_list_plan([(BASE[0], BASE[1], BASE[2] + 4, BASE[3], n)],
                          0, 0, 0)
    assert off["vector_tensors"] == 0
    assert off["norm_kept_tiles"] == 0
    monkeypatch.setenv("MTA_NORM_KEEP_MIB", "256")      # the budget wins
    assert M.mta_list_plan([(BASE[0], BASE[1], BASE[2] + 4, BASE[3], n)],
                           0, 0, 0)["norm_kept_tiles"] == ok["norm_kept_tiles"]


def test_plan_reports_the_errors_create_reports():
    ok = (0x10000, 0x20000, 0x30000, 0x40000, 64)
    cases = [([ok], 3, 0, 0, -3), ([(0x10000, 0, 0x30000, 0x40000, 64)],
                                   0, 0, 0, -1),
             ([(0x10002, 0x20000, 0x30000, 0x40000, 64)], 0, 0, 0, -2),
             ([ok, (0x10000 + 128, 0x50000, 0x60000, 0x70000, 8)], 0, 0, 0,
              -1)]
    for ents, g, m, v, code in cases:
        for fn in (M.mta_list_plan, M.mta_list_create):
            with pytest.raises(M.MtaError) as e:
                fn(ents, g, m, v)
            assert e.value.code == code, (fn.__name__, ents)


def test_gradient_only_tables():
    # g alone (w, m, v NULL on every tensor) is a valid list with no state
    # buffers and the same tile cuts as a full list over the same gradients;
    # m or v without w, or w on some tensors only, is refused
    sizes = [5, 4096, 9000, 0, 77]
    full, gonly, pos = [], [], 0
    for n in sizes:
        full.append((BASE[0] + 4 * pos, BASE[1] + 4 * pos, None, None, n))
        gonly.append((None, BASE[1] + 4 * pos, None, None, n))
        pos += -(-n // 64) * 64
    a = M.mta_list_plan(full, 0, 0, 0)
    b = M.mta_list_plan(gonly, 0, 0, 0)
    assert b["state_buffers"] == 0
    for k in ("count", "elements", "tiles", "vector_tensors"):
        assert a[k] == b[k], k
    with pytest.raises(M.MtaError):              # m without w
        M.mta_list_plan([(None, BASE[1], BASE[2], None, 8)], 0, 0, 0)
    with pytest.raises(M.MtaError):              # w on one tensor only
        M.mta_list_plan([gonly[0], full[1]], 0, 0, 0)
