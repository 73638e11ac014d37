"""Helpers of the GPU parity tests: move tensors between the device arena
and the oracle's numpy layout, run lockstep steps, measure ulp distances.

Parity protocol (lockstep): each step the device computes the norm and the
clip coefficient; the test checks the norm against the oracle's (relative
1e-6) and that the coefficient is exactly the oracle's clip rule applied to
the device norm; then the oracle runs its step with that coefficient and
w, m, v are compared element by element (float32: 2 ulp, packed bfloat16:
1 bf16 ulp).
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle as O

from mixed_precision_optimizer_mta_amd import workloads as WL

NORM_RTOL = 1e-6
F32_ULP = 2
BF16_ULP = 1

# host threads for the oracle's per-tensor work on large lists (a one-GPU
# job is given 16 cores on an MI355X node); the oracle is called through ctypes,
# which releases the GIL, so its calls on disjoint tensors run in parallel
THREADS = max(1, min(16, os.cpu_count() or 1))


def in_groups(items, fn, threads=THREADS):
    """fn(group) for `threads` disjoint groups of items (round robin by
    size, largest first), in parallel; returns the results in group
    order.  Each item is touched by exactly one call."""
    if threads <= 1 or len(items) <= 1:
        return [fn(list(items))]
    order = sorted(range(len(items)), key=lambda i: -_size(items[i]))
    groups = [[] for _ in range(min(threads, len(items)))]
    load = [0] * len(groups)
    for i in order:
        k = load.index(min(load))
        groups[k].append(items[i])
        load[k] += _size(items[i])
    with ThreadPoolExecutor(len(groups)) as ex:
        return list(ex.map(fn, groups))


def _size(x):
    return x.w.size if getattr(x, "w", None) is not None else x.g.size


def host_arena(arena, bufs="wgmv"):
    """Whole arena buffers on the host, one device-to-host copy each:
    float32 buffers as float32 arrays, 16-bit ones as uint16 bit
    patterns."""
    out = {}
    for b in bufs:
        t = getattr(arena, b).detach()
        if t.dtype == torch.float32:
            out[b] = t.cpu().numpy()
        else:
            out[b] = t.cpu().view(torch.int16).numpy().view(np.uint16)
    return out


def f32_ulp(a, b):
    """Per-element ulp distance of two float32 arrays; NaN vs NaN is 0,
    NaN vs number is huge; +0 and -0 are 0 apart."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    ia = a.view(np.int32).astype(np.int64)
    ib = b.view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    d = np.abs(ia - ib)
    na, nb = np.isnan(a), np.isnan(b)
    d = np.where(na & nb, 0, d)
    d = np.where(na ^ nb, 1 << 40, d)
    return d


def bf16_ulp(a, b):
    """Same for bfloat16 bit patterns (uint16)."""
    a = np.ascontiguousarray(a, dtype=np.uint16).astype(np.int64)
    b = np.ascontiguousarray(b, dtype=np.uint16).astype(np.int64)
    na = ((a & 0x7FFF) > 0x7F80)
    nb = ((b & 0x7FFF) > 0x7F80)
    ma = np.where(a & 0x8000, -(a & 0x7FFF), a)
    mb = np.where(b & 0x8000, -(b & 0x7FFF), b)
    d = np.abs(ma - mb)
    d = np.where(na & nb, 0, d)
    d = np.where(na ^ nb, 1 << 40, d)
    return d


def dev_f32(t):
    return t.detach().to("cpu").numpy().astype(np.float32, copy=True)


def dev_bf16_bits(t):
    return t.detach().to("cpu").view(torch.int16).numpy().view(
        np.uint16).copy()


def grad_np(t, gtype):
    """Device gradient -> oracle layout (16-bit types: their bit patterns)."""
    return dev_f32(t) if gtype == WL.F32 else dev_bf16_bits(t)


def mom_np(t, kind):
    """Device moment -> oracle layout (packed: u32 words)."""
    if kind == WL.MOM_BF16X2:
        return O.pack_halves(dev_bf16_bits(t))
    return dev_f32(t)


def oracle_state(arena, idx=None):
    """The oracle's copy of every tensor (or of the sampled positions idx,
    as one tensor) from the device arena."""
    wl = arena.wl
    if idx is not None:
        sel = torch.as_tensor(idx, device=arena.device)
        return [O.Tensor(dev_f32(arena.w[sel]),
                         grad_np(arena.g[sel], wl.gtype),
                         mom_np(arena.m[sel], wl.mkind),
                         mom_np(arena.v[sel], wl.vkind))]
    h = host_arena(arena)
    out = []
    for i, n in enumerate(wl.sizes):
        o = arena.offsets[i]
        og = o + arena.g_shift
        m, v = h["m"][o:o + n], h["v"][o:o + n]
        out.append(O.Tensor(
            h["w"][o:o + n].copy(), h["g"][og:og + n].copy(),
            O.pack_halves(m) if wl.mkind == WL.MOM_BF16X2 else m.copy(),
            O.pack_halves(v) if wl.vkind == WL.MOM_BF16X2 else v.copy()))
    return out


def oracle_grads(arena, idx=None):
    wl = arena.wl
    if idx is not None:
        sel = torch.as_tensor(idx, device=arena.device)
        return [grad_np(arena.g[sel], wl.gtype)]
    g = host_arena(arena, "g")["g"]
    sh = arena.g_shift
    return [g[o + sh:o + sh + n].copy()
            for o, n in zip(arena.offsets, wl.sizes)]


def compare(arena, ostate, idx=None, what=""):
    """Max ulp distances (w, m, v) between the device and the oracle state;
    asserts the tolerances."""
    wl = arena.wl
    if idx is not None:
        sel = torch.as_tensor(idx, device=arena.device)
        pairs = [(dev_f32(arena.w[sel]), _host_mom(arena.m[sel], wl.mkind),
                  _host_mom(arena.v[sel], wl.vkind), ostate[0], len(idx))]
    else:
        h = host_arena(arena, "wmv")
        pairs = [(h["w"][o:o + n], h["m"][o:o + n], h["v"][o:o + n],
                  ostate[i], n)
                 for i, (o, n) in enumerate(zip(arena.offsets, wl.sizes))]
    worst = {"w": 0, "m": 0, "v": 0}
    for w, m, v, o, n in pairs:
        if n == 0:
            continue
        worst["w"] = max(worst["w"], ulp_max(w, o.w, False))
        for name, t, kind, ob in (("m", m, wl.mkind, o.m),
                                  ("v", v, wl.vkind, o.v)):
            packed = kind == WL.MOM_BF16X2
            want = O.unpack_words(ob, n) if packed else ob
            worst[name] = max(worst[name], ulp_max(t, want, packed))
    assert worst["w"] <= F32_ULP, (what, worst)
    for name, kind in (("m", wl.mkind), ("v", wl.vkind)):
        tol = BF16_ULP if kind == WL.MOM_BF16X2 else F32_ULP
        assert worst[name] <= tol, (what, worst)
    return worst


def _host_mom(t, kind):
    return dev_bf16_bits(t) if kind == WL.MOM_BF16X2 else dev_f32(t)


def ulp_max(got, want, bf16):
    """Largest ulp distance between two arrays of one buffer (float32
    values, or bfloat16 bit patterns when bf16); 0 at once when they are
    the same bits."""
    it = np.uint16 if bf16 else np.uint32
    a = np.ascontiguousarray(got).view(it)
    b = np.ascontiguousarray(want).view(it)
    if a.shape == b.shape and np.array_equal(a, b):
        return 0
    d = bf16_ulp(a, b) if bf16 else f32_ulp(a.view(np.float32),
                                            b.view(np.float32))
    return int(d.max())


def check_norm(norm_gpu, coef_gpu, norm_oracle, max_norm, what=""):
    if np.isnan(norm_oracle):
        assert np.isnan(norm_gpu), what
        assert np.isnan(coef_gpu), what
        return
    if np.isinf(norm_oracle):
        assert np.isinf(norm_gpu) and coef_gpu == 0.0, what
        return
    assert abs(float(norm_gpu) - norm_oracle) <= NORM_RTOL * norm_oracle + \
        1e-38, (what, float(norm_gpu), norm_oracle)
    want = O.clip_coef(max_norm, np.float32(norm_gpu))
    assert np.float32(coef_gpu).view(np.uint32) == want.view(np.uint32), (
        what, float(coef_gpu), float(want))


def sample_positions(wl, offsets, nsample, seed=1):
    """Arena positions to compare at full size: each tensor's first and last
    8 elements plus nsample uniform draws over all elements."""
    rng = np.random.default_rng(seed)
    sizes = np.asarray(wl.sizes, dtype=np.int64)
    offs = np.asarray(offsets, dtype=np.int64)
    parts = []
    for o, n in zip(offs, sizes):
        if n == 0:
            continue
        k = min(8, int(n))
        parts.append(o + np.arange(k))
        parts.append(o + n - 1 - np.arange(k))
    cum = np.concatenate([[0], np.cumsum(sizes)])
    r = rng.integers(0, int(cum[-1]), size=nsample)
    t = np.searchsorted(cum, r, side="right") - 1
    parts.append(offs[t] + (r - cum[t]))
    return np.unique(np.concatenate(parts))


def expected_tiles(entries, gtype, mkind, vkind):
    """(tiles, vector tensors) a list of these (w, g, m, v, n) entries must
    have: a tensor whose present buffers all reach a 128-byte boundary
    after its first h elements, or else all reach 16-byte alignment (the
    smallest such h, found by trying every h up to 127, then up to 15), is
    cut into a head of h elements, if h > 0, and then 4096-element tiles;
    any other tensor into 4096-element tiles from 0."""
    sz = [4, 4 if gtype == WL.F32 else 2,
          2 if mkind == WL.MOM_BF16X2 else 4,
          2 if vkind == WL.MOM_BF16X2 else 4]
    tiles = vec = 0
    for w, g, m, v, n in entries:
        if n == 0:
            continue
        bufs = [(p, s) for p, s in zip((w, g, m, v), sz) if p]
        h = next((h for h in range(128)
                  if all((p + h * s) % 128 == 0 for p, s in bufs)), None)
        if h is None:
            h = next((h for h in range(16)
                      if all((p + h * s) % 16 == 0 for p, s in bufs)), None)
        head = min(h, n) if h else 0
        tiles += (1 if head else 0) + -(-(n - head) // 4096)
        vec += h is not None and h < n
    return tiles, vec


def make_list(arena):
    from mixed_precision_optimizer_mta_amd import MtaList
    wl = arena.wl
    return MtaList([], entries=arena.entries(), gtype=wl.gtype,
                   mkind=wl.mkind, vkind=wl.vkind)


def _bits32(x):
    return int(np.float32(x).view(np.uint32))


def check_amp_state(dev, ora, what=""):
    """The device loss-scale state equals the oracle's, field by field
    (the scale bit for bit)."""
    got = (_bits32(dev["scale"]), _bits32(dev["found_inf"]),
           dev["growth_tracker"], dev["step"])
    want = (_bits32(ora.scale), _bits32(ora.found_inf), ora.tracker,
            ora.step)
    assert got == want, (what, dev, vars(ora))


def lockstep(wl, steps, offsets=None, nsample=None, norm_steps=None,
             check_guards=False, clip=True, inject=None, g_shift=0,
             compare_steps=None):
    """Run `steps` device steps in lockstep with the oracle; returns the
    worst ulp distances seen.  Every element (or every sampled position
    when nsample is set) is compared after the steps in compare_steps
    (None: after every step) and always after the last; the norm is
    checked at norm_steps (None: every step).  The oracle's state stays in
    lockstep at every step either way.

    A loss-scaled workload (wl.amp) runs mta_amp_clip_norm,
    mta_amp_adamw_step and mta_amp_update against oracle.amp_step_ and
    AmpState.update, and also checks the found_inf flag and the state after
    every step.  inject: {step: [(arena position, value), ...]} written into
    the gradients after they are drawn (positions must be sampled ones when
    nsample is set, so the oracle sees them)."""
    from mixed_precision_optimizer_mta_amd import AmpState
    assert not (g_shift and nsample is not None), "sampling reads g unshifted"
    arena = WL.Arena(wl, "cuda", offsets, g_shift=g_shift)
    arena.fill_weights()
    L = make_list(arena)
    idx = None
    if nsample is not None:
        idx = sample_positions(wl, arena.offsets, nsample)
    ostate = oracle_state(arena, idx)
    before = None
    if check_guards:
        before = {b: getattr(arena, b).clone() for b in "wmv"}
    norm_d = torch.full((1,), -1.0, device="cuda")
    coef_d = torch.full((1,), -1.0, device="cuda")
    amp_d = amp_o = None
    if wl.amp:
        amp_d = AmpState(wl.amp_scale)
        amp_o = O.AmpState(wl.amp_scale)
    worst = {"w": 0, "m": 0, "v": 0}
    skipped = 0
    for t in range(1, steps + 1):
        arena.fill_grads(t)
        for pos, val in (inject or {}).get(t, []):
            arena.g[pos] = val
        for o, g in zip(ostate, oracle_grads(arena, idx)):
            o.g = g
        if wl.amp:
            L.amp_clip_norm(wl.max_norm, amp_d, norm_d, coef_d)
            found_d = amp_d.read()["found_inf"]
            L.amp_adamw_step(wl.hparams, amp_d, coef_d)
            amp_d.update(wl.amp_growth, wl.amp_backoff, wl.amp_interval)
        else:
            if wl.scale != 1.0:
                L.scale(wl.scale, defer=True)
            if clip:
                L.clip_norm(wl.max_norm, norm_d, coef_d)
                L.adamw_step(wl.hparams, t, coef_d)
            else:
                L.adamw_step(wl.hparams, t, None)
        torch.cuda.synchronize()
        s = O.inv_scale(amp_o.scale) if wl.amp else wl.scale
        coef = np.float32(1.0)
        if clip:
            ng = np.float32(norm_d.item())
            coef = np.float32(coef_d.item())
            if norm_steps is None or t in norm_steps:
                gs = oracle_grads(arena) if idx is not None else \
                    [o.g for o in ostate]
                no = O.norm(gs, wl.gtype, s)
                check_norm(ng, coef, no, wl.max_norm, f"{wl.name} t={t}")
            else:
                want = O.clip_coef(wl.max_norm, ng)
                assert coef.view(np.uint32) == want.view(np.uint32)
        if wl.amp:
            _, _, found_o = O.amp_step_(
                ostate, wl.gtype, wl.mkind, wl.vkind, amp_o, wl.lr,
                wl.beta1, wl.beta2, wl.eps, wl.weight_decay, wl.max_norm,
                coef=coef)
            assert found_d == (1.0 if found_o else 0.0), (wl.name, t)
            skipped += bool(found_o)
            amp_o.update(wl.amp_growth, wl.amp_backoff, wl.amp_interval)
            check_amp_state(amp_d.read(), amp_o, f"{wl.name} t={t}")
        else:
            # the oracle's own step over disjoint groups of tensors: with
            # the coefficient given, each tensor's update depends on that
            # tensor alone
            in_groups(ostate, lambda grp: O.step_(
                grp, wl.gtype, wl.mkind, wl.vkind, wl.lr, wl.beta1,
                wl.beta2, wl.eps, wl.weight_decay, t, s=s, coef=coef))
        if compare_steps is None or t in compare_steps or t == steps:
            got = compare(arena, ostate, idx, f"{wl.name} t={t}")
            worst = {k: max(worst[k], got[k]) for k in worst}
    if check_guards:
        torch.cuda.synchronize()
        inside = torch.zeros(arena.total, dtype=torch.bool, device="cuda")
        for o, n in zip(arena.offsets, wl.sizes):
            inside[o:o + n] = True
        for b in "wmv":
            now = getattr(arena, b)
            ity = torch.int16 if now.dtype == torch.bfloat16 else torch.int32
            diff = (now.view(ity) != before[b].view(ity)) & ~inside
            assert not bool(diff.any()), f"{b} written outside its tensors"
    L.close()
    extra = f" amp: {skipped} skipped, state {amp_d.read()}" if wl.amp else ""
    print(f"{wl.name}: steps={steps} worst ulp {worst}{extra}", flush=True)
    return worst


# ------------------------------------------------------------ other rules

def opt_for(kind, zero=False, lr=None):
    adam = kind in ("adamw", "adam")
    return dict(kind=kind, lr=lr if lr is not None else (3e-4 if adam
                                                          else 0.05),
                beta1=0.9, beta2=0.999, eps=1e-8,
                weight_decay=0.1 if adam else 0.0, momentum=0.9,
                zero_grad=zero)


def uses(kind):
    """(has m, has v) of a rule's list."""
    return kind != "sgd", kind in ("adamw", "adam")


def make_rule_list(arena, kind):
    from mixed_precision_optimizer_mta_amd import MtaList
    wl = arena.wl
    has_m, has_v = uses(kind)
    ents = [(w, g, m if has_m else None, v if has_v else None, n)
            for (w, g, m, v, n) in arena.entries()]
    return MtaList([], entries=ents, gtype=wl.gtype, mkind=wl.mkind,
                   vkind=wl.vkind)


def oracle_rule_state(arena, kind, idx=None):
    wl = arena.wl
    has_m, has_v = uses(kind)
    if idx is None:
        out = oracle_state(arena)
        for o in out:
            o.m = o.m if has_m else None
            o.v = o.v if has_v else None
        return out
    sel = torch.as_tensor(idx, device=arena.device)
    return [O.Tensor(dev_f32(arena.w[sel]), grad_np(arena.g[sel], wl.gtype),
                     mom_np(arena.m[sel], wl.mkind) if has_m else None,
                     mom_np(arena.v[sel], wl.vkind) if has_v else None)]


def compare_rule(arena, ost, kind, idx=None, what=""):
    """Bitwise comparison of w, g and the rule's state buffers."""
    wl = arena.wl
    has_m, has_v = uses(kind)
    if idx is not None:
        sel = torch.as_tensor(idx, device=arena.device)
        views = [(dev_f32(arena.w[sel]), grad_np(arena.g[sel], wl.gtype),
                  _host_mom(arena.m[sel], wl.mkind),
                  _host_mom(arena.v[sel], wl.vkind), len(idx))]
    else:
        h = host_arena(arena)
        sh = arena.g_shift
        views = [(h["w"][o:o + n], h["g"][o + sh:o + sh + n],
                  h["m"][o:o + n], h["v"][o:o + n], n)
                 for o, n in zip(arena.offsets, wl.sizes)]
    gbits = wl.gtype != WL.F32
    for (w, g, m, v, n), o in zip(views, ost):
        if n == 0:
            continue
        assert ulp_max(w, o.w, False) == 0, (what, "w")
        gi = np.uint16 if gbits else np.uint32
        assert np.array_equal(np.ascontiguousarray(g).view(gi),
                              np.ascontiguousarray(o.g).view(gi)), \
            (what, "g")
        for has, t, kind_, ob, name in ((has_m, m, wl.mkind, o.m, "m"),
                                        (has_v, v, wl.vkind, o.v, "v")):
            if not has:
                continue
            packed = kind_ == WL.MOM_BF16X2
            want = O.unpack_words(ob, n) if packed else ob
            d = ulp_max(t, want, packed)
            assert d == 0, (what, name, d)


def rule_lockstep(wl, opt, steps, offsets=None, nsample=None,
                  norm_steps=None, check_guards=False, g_shift=0,
                  compare_steps=None):
    """lockstep for any rule through mta_step: norm checked at norm_steps
    (None: every step), w, g and the rule's state compared bit for bit
    after compare_steps (None: every step) and after the last."""
    assert not (g_shift and nsample is not None)
    arena = WL.Arena(wl, "cuda", offsets, g_shift=g_shift)
    arena.fill_weights()
    kind, zero = opt["kind"], bool(opt.get("zero_grad"))
    L = make_rule_list(arena, kind)
    idx = None if nsample is None else sample_positions(wl, arena.offsets,
                                                        nsample)
    ost = oracle_rule_state(arena, kind, idx)
    before = None
    if check_guards:
        before = {b: getattr(arena, b).clone() for b in "wgmv"}
    nd = torch.full((1,), -1.0, device="cuda")
    cd = torch.full((1,), -1.0, device="cuda")
    for t in range(1, steps + 1):
        arena.fill_grads(t)
        if check_guards:
            before["g"] = arena.g.clone()
        for o, g in zip(ost, oracle_grads(arena, idx)):
            o.g = g
        full_g = None
        if idx is not None and (norm_steps is None or t in norm_steps):
            full_g = oracle_grads(arena)     # before a zeroing step runs
        if wl.scale != 1.0:
            L.scale(wl.scale, defer=True)
        L.clip_norm(wl.max_norm, nd, cd)
        L.step(opt, t, cd)
        torch.cuda.synchronize()
        ng, coef = np.float32(nd.item()), np.float32(cd.item())
        if norm_steps is None or t in norm_steps:
            # the oracle's step below may zero its copies: read them first
            gs = [o.g for o in ost] if idx is None else full_g
            check_norm(ng, coef, O.norm(gs, wl.gtype, wl.scale), wl.max_norm,
                       f"{wl.name} {kind} t={t}")
        else:
            want = O.clip_coef(wl.max_norm, ng)
            assert coef.view(np.uint32) == want.view(np.uint32)
        in_groups(ost, lambda grp: O.opt_step_(
            grp, opt, wl.gtype, wl.mkind, wl.vkind, t, s=wl.scale,
            coef=coef, zero=zero))
        if compare_steps is None or t in compare_steps or t == steps:
            compare_rule(arena, ost, kind, idx, f"{wl.name} {kind} t={t}")
        if check_guards:
            has_m, has_v = uses(kind)
            for b in "wgmv":
                sh = arena.g_shift if b == "g" else 0
                inside = torch.zeros(arena.total, dtype=torch.bool,
                                     device="cuda")
                for o, n in zip(arena.offsets, wl.sizes):
                    inside[o + sh:o + sh + n] = True
                now = getattr(arena, b)
                ity = torch.int32 if now.dtype == torch.float32 else \
                    torch.int16
                diff = now.view(ity) != before[b].view(ity)
                if b in "wg" or (b == "m" and has_m) or (b == "v" and has_v):
                    diff = diff & ~inside    # only inside its tensors
                assert not bool(diff.any()), f"{kind}: {b} written outside"
    L.close()
    print(f"{wl.name} {kind} zero={zero}: {steps} steps bitwise",
          flush=True)
