"""Pins for the CPU oracle: values fixed by the pages or by mathematics.

None of these compares the oracle with a retyped copy of itself.  They use
hand-derived exact steps (tests/golden), closed forms of the AdamW
recurrence, exact sums (math.fsum), an independent distance-based
nearest-even rounding, and library routines (torch) for the special cases
they share with the method.  Each test names the page passage it pins.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def f32bits(x):
    return int(np.asarray(x, dtype=np.float32).view(np.uint32))


def ulp_dist(a, b):
    """ulp distance between float32 arrays (monotone integer map)."""
    a = np.asarray(a, dtype=np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, dtype=np.float32).view(np.int32).astype(np.int64)
    a = np.where(a < 0, -(a & 0x7FFFFFFF), a)
    b = np.where(b < 0, -(b & 0x7FFFFFFF), b)
    return np.abs(a - b)


# ---------------------------------------------------------------------------
# bfloat16 rounding ("BendTorch main.bend", Optimizers, ph_of_bits / ph_to)
# ---------------------------------------------------------------------------

def test_bf16_golden_cases():
    for row in _golden_rows("bf16_cases.txt"):
        u, h = int(row[0], 16), int(row[1], 16)
        assert O.bf16_of_bits(u) == h, row


def _rne_by_distance(bits):
    """Nearest-even bfloat16 by comparing exact distances (no bit tricks
    beyond truncation): an independent reference for non-NaN inputs."""
    bits = bits.astype(np.uint32)
    x = bits.view(np.float32).astype(np.float64)
    lo = (bits >> np.uint32(16)).astype(np.uint32)        # toward zero
    hi = lo + np.uint32(1)                                  # away from zero
    vlo = (lo << np.uint32(16)).view(np.float32).astype(np.float64)
    hi_exp_all_ones = (hi & np.uint32(0x7F80)) == np.uint32(0x7F80)
    with np.errstate(invalid="ignore"):
        vhi = np.where(hi_exp_all_ones,
                       np.copysign(2.0 ** 128, x),
                       (hi << np.uint32(16)).view(np.float32)
                       .astype(np.float64))
    with np.errstate(invalid="ignore"):
        dlo = np.abs(x - vlo)
        dhi = np.abs(vhi - x)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((lo & np.uint32(1)) == 1))
    out = np.where(pick_hi, hi, lo)
    inf = np.isinf(x)
    out = np.where(inf, lo, out)
    return out.astype(np.uint32)


def test_bf16_rne_against_distance_rounding():
    # every bfloat16 high half, with low halves that cover exact values,
    # ties, both sides of a tie and the extremes, plus random ones
    rng = np.random.default_rng(20261202)
    lows = np.concatenate([
        np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000,
                  0xC000], dtype=np.uint32),
        rng.integers(0, 0x10000, size=24, dtype=np.uint32)])
    highs = np.arange(0x10000, dtype=np.uint32)
    bits = (highs[:, None] << np.uint32(16) | lows[None, :]).ravel()
    x = bits.view(np.float32)
    got = O.bf16_of_f32(x).astype(np.uint32)
    nan = np.isnan(x)
    assert np.all(got[nan] == 0xFFFF)
    want = _rne_by_distance(bits[~nan])
    bad = np.nonzero(got[~nan] != want)[0]
    assert bad.size == 0, [hex(int(b)) for b in bits[~nan][bad[:5]]]


def test_bf16_rne_matches_torch_on_finite():
    # torch's float32 -> bfloat16 conversion is round-to-nearest-even too;
    # it differs only in the NaN pattern it writes
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(
        np.uint32)
    x = bits.view(np.float32)
    keep = ~np.isnan(x)
    x = x[keep]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_of_f32(x), ref)


def test_bf16_round_trip_identity():
    h = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    x = O.f32_of_bf16(h)
    back = O.bf16_of_f32(x)
    nan = np.isnan(x)
    assert np.array_equal(back[~nan], h[~nan])
    assert np.all(back[nan] == 0xFFFF)
    # bf16 -> f32 is the value torch gives for the same bits
    t = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).float()
    tn = t.numpy()
    assert np.array_equal(tn[~nan].view(np.uint32), x[~nan].view(np.uint32))


def test_packed_layout_is_little_endian_bf16_array():
    # PTree comment: element 2k in the low half of word k.  That is exactly
    # the memory of a bfloat16 array of n elements on a little-endian host.
    h = np.array([0x1111, 0x2222, 0x3333, 0x4444, 0x5555], dtype=np.uint16)
    words = O.pack_halves(h)
    assert [hex(int(w)) for w in words] == ["0x22221111", "0x44443333",
                                            "0x5555"]
    assert np.array_equal(words[:2].view(np.uint16), h[:4])
    assert np.array_equal(O.unpack_words(words, 5), h)


# ---------------------------------------------------------------------------
# scalars ("BendTorch main.bend": Opt type comment, Opt.at, comment on
# adam_m; Training: q1 = 1 - b1^t, q2 = 1 - b2^t, t = 1 first)
# ---------------------------------------------------------------------------

def _f32_nearest(fr):
    """The float32 nearest to an exact Fraction (via float64 is enough for
    these magnitudes only when no double rounding occurs; checked below by
    comparing neighbours exactly)."""
    cand = np.float32(float(fr))
    best, bd = cand, abs(Fraction(float(cand)) - fr)
    for nb in (np.nextafter(cand, np.float32(np.inf)),
               np.nextafter(cand, np.float32(-np.inf))):
        d = abs(Fraction(float(nb)) - fr)
        if d < bd:
            best, bd = nb, d
    return best


def test_scalars_first_step_closed_form():
    sc = dict(zip(O.SCALAR_NAMES, O.scalars(3e-4, 0.9, 0.999, 1e-8, 0.1, 1)))
    # t = 1: step = lr / (1 - b1) = 0.003, bc2 = sqrt(0.001)
    assert sc["step"] == np.float32(0.003)
    assert sc["bc2"] == np.float32(0.0316227766016838)   # sqrt(1/1000)
    assert sc["c1"] == np.float32(0.1)
    assert sc["c2"] == np.float32(0.001)
    assert sc["b2"] == np.float32(0.999)
    assert sc["eps"] == np.float32(1e-8)
    assert sc["dec"] == np.float32(0.99997)               # 1 - 3e-4 * 0.1


def test_scalars_late_steps_tend_to_lr_and_one():
    sc = dict(zip(O.SCALAR_NAMES,
                  O.scalars(3e-4, 0.9, 0.999, 1e-8, 0.1, 10 ** 6)))
    assert sc["step"] == np.float32(3e-4)
    assert sc["bc2"] == np.float32(1.0)


def test_c2_formed_in_float64_not_float32():
    # comment on adam_m: 1 - b2 taken in F32 from b2 = 0.999 is 1.3e-5 too
    # small; the constant must be the float32 nearest 0.001 instead
    c2 = O.scalars(3e-4, 0.9, 0.999, 1e-8, 0.1, 1)[3]
    assert c2 == np.float32(0.001)
    f32_way = np.float32(1.0) - np.float32(0.999)
    rel = (float(f32_way) - 0.001) / 0.001
    assert -1.35e-5 < rel < -1.25e-5        # the page's 1.3e-5, too small
    assert f32_way != c2


@pytest.mark.parametrize("t", [1, 2, 3, 10, 100, 1000, 12345])
def test_scalars_against_exact_rationals(t):
    lr, b1, b2, wd = 3e-4, 0.9, 0.999, 0.1
    sc = dict(zip(O.SCALAR_NAMES, O.scalars(lr, b1, b2, 1e-8, wd, t)))
    L, B1, B2, WD = (Fraction(x) for x in (lr, b1, b2, wd))
    step = L / (1 - B1 ** t)
    # float64 pow and division then one float32 rounding: within 1 ulp of
    # the float32 nearest the exact value
    assert ulp_dist(sc["step"], _f32_nearest(step)) <= 1
    bc2_sq = 1 - B2 ** t
    near = _f32_nearest(Fraction(math.sqrt(float(bc2_sq))))
    assert ulp_dist(sc["bc2"], near) <= 1
    # and bc2^2 brackets 1 - b2^t
    lo = Fraction(float(np.nextafter(sc["bc2"], np.float32(0))))
    hi = Fraction(float(np.nextafter(sc["bc2"], np.float32(2))))
    assert lo * lo < bc2_sq < hi * hi
    assert sc["dec"] == _f32_nearest(1 - L * WD)
    assert sc["c1"] == _f32_nearest(1 - B1)
    assert sc["c2"] == _f32_nearest(1 - B2)


def test_scalars_reject_step_zero():
    with pytest.raises(ValueError):
        O.scalars(3e-4, 0.9, 0.999, 1e-8, 0.1, 0)


# ---------------------------------------------------------------------------
# AdamW element steps (hand-derived, exact)
# ---------------------------------------------------------------------------

def _kind(s):
    return O.MOM_BF16X2 if s == "bf16x2" else O.MOM_F32


def _mom_buf(kind, val):
    if kind == O.MOM_BF16X2:
        return O.pack_halves(O.bf16_of_f32(np.array([val], np.float32)))
    return np.array([val], dtype=np.float32)


def _mom_val(kind, buf):
    if kind == O.MOM_BF16X2:
        return float(O.f32_of_bf16(O.unpack_words(buf, 1))[0])
    return float(buf[0])


@pytest.mark.parametrize("row", _golden_rows("hand_steps.txt"),
                         ids=lambda r: f"{r[0]}-t{r[1]}")
def test_hand_derived_steps(row):
    case, t, mk, vk, eps, w0, g0, m0, v0, w1, m1, v1 = row
    mkind, vkind = _kind(mk), _kind(vk)
    w = np.array([float(w0)], np.float32)
    g = np.array([float(g0)], np.float32)
    assert float(g[0]) == float(Fraction(g0))          # exact input
    m, v = _mom_buf(mkind, float(m0)), _mom_buf(vkind, float(v0))
    sc = O.scalars(0.125, 0.5, 0.75, float(eps), 0.5, int(t))
    O.adamw_(w, g, m, v, O.F32, mkind, vkind, sc)
    assert float(w[0]) == float(Fraction(w1))
    assert _mom_val(mkind, m) == float(Fraction(m1))
    assert _mom_val(vkind, v) == float(Fraction(v1))


def test_packed_element_layout_and_pad_half_untouched():
    # g_k = 2^-k with c1 = 0.5 gives m_k = 2^-(k+1), exact in bfloat16:
    # bits 0x3F00 - 0x80*k.  Element 2k sits in the low half of word k and
    # the pad half of the last word keeps whatever it held.
    n = 5
    g = np.array([2.0 ** -k for k in range(n)], np.float32)
    w = np.ones(n, np.float32)
    m = np.zeros(3, np.uint32)
    v = np.zeros(3, np.uint32)
    m[2] = 0xBEEF0000
    v[2] = 0xCAFE0000
    sc = O.scalars(0.125, 0.5, 0.75, 0.5, 0.5, 1)
    O.adamw_(w, g, m, v, O.F32, O.MOM_BF16X2, O.MOM_BF16X2, sc)
    want = [0x3F00 - 0x80 * k for k in range(n)]
    assert int(m[0]) == (want[1] << 16) | want[0]
    assert int(m[1]) == (want[3] << 16) | want[2]
    assert int(m[2]) == 0xBEEF0000 | want[4]
    assert int(v[2]) >> 16 == 0xCAFE


# ---------------------------------------------------------------------------
# AdamW against the textbook recurrence (closed forms; float64)
# ---------------------------------------------------------------------------

def test_first_step_closed_form():
    # From zero moments at t = 1, exact arithmetic gives
    #   w1 = w * (1 - lr*wd) - lr * g / (|g| + eps)
    rng = np.random.default_rng(1)
    n = 4096
    w = rng.normal(0, 0.02, n).astype(np.float32)
    g = rng.normal(0, 1e-3, n).astype(np.float32)
    g[:16] = 0.0
    lr, b1, b2, eps, wd = 3e-4, 0.9, 0.999, 1e-8, 0.1
    want = (w.astype(np.float64) * (1 - lr * wd)
            - lr * g.astype(np.float64) / (np.abs(g.astype(np.float64)) + eps))
    ww = w.copy()
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    O.adamw_(ww, g, m, v, O.F32, O.MOM_F32, O.MOM_F32,
             O.scalars(lr, b1, b2, eps, wd, 1))
    err = np.abs(ww.astype(np.float64) - want)
    # a few float32 roundings of w1, plus a few relative roundings of the
    # update term (about lr in size) itself
    tol = (4 * np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
           + 16 * 2.0 ** -24 * lr)
    assert np.all(err <= tol)
    # a zero gradient leaves exactly the decayed weight
    dec = np.float32(1 - lr * wd)
    assert np.array_equal(ww[:16], w[:16] * dec)


def _textbook_adamw(w, gs, lr, b1, b2, eps, wd):
    """Loshchilov & Hutter's AdamW in float64, bias-corrected moments."""
    w = w.astype(np.float64).copy()
    m = np.zeros_like(w)
    v = np.zeros_like(w)
    for t, g in enumerate(gs, start=1):
        g = g.astype(np.float64)
        w = w * (1 - lr * wd)
        m = b1 * m + (1 - b1) * g
        v = b2 * v + (1 - b2) * g * g
        mh = m / (1 - b1 ** t)
        vh = v / (1 - b2 ** t)
        w = w - lr * mh / (np.sqrt(vh) + eps)
    return w, m, v


@pytest.mark.parametrize("mk,vk", [("f32", "f32"), ("bf16x2", "bf16x2"),
                                   ("bf16x2", "f32")])
def test_multi_step_against_textbook_float64(mk, vk):
    rng = np.random.default_rng(2)
    n, steps = 2048, 12
    lr, b1, b2, eps, wd = 3e-4, 0.9, 0.999, 1e-8, 0.1
    w0 = rng.normal(0, 0.02, n).astype(np.float32)
    gs = [rng.normal(0, 1e-3, n).astype(np.float32) for _ in range(steps)]
    mkind, vkind = _kind(mk), _kind(vk)
    w = w0.copy()
    m = np.zeros(O.packed_words(n) if mkind else n,
                 np.uint32 if mkind else np.float32)
    v = np.zeros(O.packed_words(n) if vkind else n,
                 np.uint32 if vkind else np.float32)
    for t, g in enumerate(gs, start=1):
        O.adamw_(w, g, m, v, O.F32, mkind, vkind,
                 O.scalars(lr, b1, b2, eps, wd, t))
    wt, mt, vt = _textbook_adamw(w0, gs, lr, b1, b2, eps, wd)
    # per-step displacement is ~lr; float32 rounding of the update
    # (f32 moments) or bfloat16 moments (relative 2^-9) bound the drift
    rel = 2.0 ** -20 if mkind == O.MOM_F32 and vkind == O.MOM_F32 else 2.0 ** -7
    bound = steps * lr * rel * 4 + 4 * np.spacing(np.abs(wt).astype(np.float32))
    assert np.all(np.abs(w - wt) <= bound)
    mm = (O.f32_of_bf16(O.unpack_words(m, n)) if mkind else m)
    vv = (O.f32_of_bf16(O.unpack_words(v, n)) if vkind else v)
    mrel = 2.0 ** -7 if mkind else 2.0 ** -18
    vrel = 2.0 ** -7 if vkind else 2.0 ** -18
    # m is a signed sum: its rounding error scales with the terms (about
    # c1 * |g| = 1e-4), not with |m| itself
    assert np.all(np.abs(mm - mt) <= mrel * (np.abs(mt) + 1e-4) * steps)
    assert np.all(np.abs(vv - vt) <= vrel * np.abs(vt) * steps + 1e-30)


def test_adamw_against_torch_cpu():
    # torch.optim.AdamW (single-tensor path) performs the same operations in
    # the same order; its lerp may use a fused multiply-add on this CPU, so
    # agreement is to a few ulp rather than bitwise.
    rng = np.random.default_rng(3)
    n, steps = 4096, 10
    lr, b1, b2, eps, wd = 3e-4, 0.9, 0.999, 1e-8, 0.1
    w0 = rng.normal(0, 0.02, n).astype(np.float32)
    gs = [rng.normal(0, 1e-2, n).astype(np.float32) for _ in range(steps)]
    p = torch.nn.Parameter(torch.from_numpy(w0.copy()))
    opt = torch.optim.AdamW([p], lr=lr, betas=(b1, b2), eps=eps,
                            weight_decay=wd, foreach=False, fused=False)
    w = w0.copy()
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    for t, g in enumerate(gs, start=1):
        p.grad = torch.from_numpy(g.copy())
        opt.step()
        O.adamw_(w, g, m, v, O.F32, O.MOM_F32, O.MOM_F32,
                 O.scalars(lr, b1, b2, eps, wd, t))
    st = opt.state[p]
    wt = p.detach().numpy()
    mt = st["exp_avg"].numpy()
    # the fused lerp differs by an ulp of the terms (c1*|g| ~ 1e-3), which
    # is many ulps of an m that cancels to near zero; so compare on the
    # scale of the terms, and w on its own scale plus that of the update
    u = 2.0 ** -24
    # each step rounds w at the size it had then (at most |w0| + t*lr)
    wscale = np.abs(w0) + steps * lr
    assert np.all(np.abs(w - wt) <= steps * (np.spacing(wscale) + 4 * u * lr))
    assert np.all(np.abs(m - mt) <= steps * 2 * u * (np.abs(mt) + 1e-2))
    assert ulp_dist(v, st["exp_avg_sq"].numpy()).max() <= 4


# ---------------------------------------------------------------------------
# joint norm and clip (Mica: ClipGradNorms, one threshold over the joint norm)
# ---------------------------------------------------------------------------

def test_norm_is_exact_sum_of_squares():
    rng = np.random.default_rng(4)
    gs = [rng.normal(0, 1e-3, n).astype(np.float32) for n in (0, 1, 7, 1000,
                                                              65537)]
    s = O.sumsq(gs, O.F32)
    exact = math.fsum(float(x) * float(x) for g in gs for x in g)
    assert abs(s - exact) <= 1e-15 * exact


def test_norm_closed_forms():
    a = np.float32(0.75)
    for n in (1, 3, 1024, 1000003):
        g = np.full(n, a, np.float32)
        assert O.sumsq([g], O.F32) == n * 0.5625
        assert abs(O.norm([g], O.F32) - 0.75 * math.sqrt(n)) <= \
            1e-15 * math.sqrt(n)
    assert O.norm([], O.F32) == 0.0
    assert O.norm([np.zeros(10, np.float32)], O.F32) == 0.0


def test_norm_power_of_two_scaling_and_bf16_unscale():
    rng = np.random.default_rng(5)
    g = rng.normal(0, 1e-3, 50000).astype(np.float32)
    gb = O.bf16_of_f32(g * np.float32(65536.0))
    # unscaling by 2^-16 in registers is exact: the norm scales exactly
    n_raw = O.norm([gb], O.BF16, 1.0)
    n_uns = O.norm([gb], O.BF16, 2.0 ** -16)
    assert n_uns == n_raw * 2.0 ** -16
    # bf16 values are the same numbers torch reads from the same bits
    tv = torch.from_numpy(gb.view(np.int16).copy()).view(torch.bfloat16)
    exact = math.fsum(float(x) ** 2 for x in tv.float().numpy())
    assert abs(O.sumsq([gb], O.BF16) - exact) <= 1e-15 * exact


def test_clip_coef_special_cases():
    assert O.clip_coef(1.0, 0.0) == 1.0            # all-zero list
    assert O.clip_coef(1.0, 0.5) == 1.0
    assert O.clip_coef(1.0, np.float32(1.0) - np.float32(1e-6)) == 1.0
    assert O.clip_coef(1.0, np.inf) == 0.0
    assert np.isnan(O.clip_coef(1.0, np.nan))
    assert O.clip_coef(2.0, 4.0) < 0.5


def test_clip_matches_torch_clip_grad_norm():
    # torch.nn.utils.clip_grad_norm_: coef = max/(norm + 1e-6), clamp at 1,
    # gradients multiplied in float32.  With max = 1 its reciprocal-multiply
    # is the same correctly rounded quotient.
    rng = np.random.default_rng(6)
    gs = [rng.normal(0, 0.05, n).astype(np.float32) for n in (100, 333, 4096)]
    ps = [torch.nn.Parameter(torch.zeros(len(g))) for g in gs]
    for p, g in zip(ps, gs):
        p.grad = torch.from_numpy(g.copy())
    tn = torch.nn.utils.clip_grad_norm_(ps, 1.0, foreach=False)
    nrm = O.norm(gs, O.F32)
    assert abs(float(tn) - nrm) <= 1e-6 * nrm
    c = O.clip_coef(1.0, np.float32(float(tn)))
    for p, g in zip(ps, gs):
        assert np.array_equal(p.grad.numpy(), (g * c).astype(np.float32))


@pytest.mark.parametrize("seed", range(5))
def test_clip_invariant_post_clip_norm(seed):
    rng = np.random.default_rng(100 + seed)
    scale = [1e-4, 1e-2, 1.0, 10.0, 1e3][seed]
    gs = [rng.normal(0, scale, n).astype(np.float32) for n in (17, 500, 3000)]
    max_norm = 1.0
    nrm = O.norm(gs, O.F32)
    c = O.clip_coef(max_norm, np.float32(nrm))
    post = math.sqrt(math.fsum(float(x) ** 2 for g in gs
                               for x in (g * c).astype(np.float32)))
    assert post <= max_norm * (1 + 1e-6)
    if nrm <= max_norm - 1e-6:
        assert c == 1.0


def test_step_with_no_clip_leaves_gradient_bitwise():
    # coef = 1 must leave ge == x bitwise, so a step with a huge max_norm
    # equals a step with no clip at all
    rng = np.random.default_rng(8)
    n = 999
    mk = lambda: O.Tensor(rng.normal(0, .02, n).astype(np.float32),
                          rng.normal(0, 1e-3, n).astype(np.float32),
                          np.zeros(n, np.float32), np.zeros(n, np.float32))
    a = mk()
    b = O.Tensor(a.w.copy(), a.g.copy(), a.m.copy(), a.v.copy())
    hp = (3e-4, 0.9, 0.999, 1e-8, 0.1)
    O.step_([a], O.F32, O.MOM_F32, O.MOM_F32, *hp, t=1, max_norm=1e6)
    O.step_([b], O.F32, O.MOM_F32, O.MOM_F32, *hp, t=1)
    assert np.array_equal(a.w, b.w) and np.array_equal(a.m, b.m)


# ---------------------------------------------------------------------------
# multi-tensor == per-tensor (Mica: each group updated as AdamWStep alone)
# ---------------------------------------------------------------------------

def _rand_list(rng, sizes, gtype, mkind, vkind):
    out = []
    for n in sizes:
        w = rng.normal(0, 0.02, n).astype(np.float32)
        g = rng.normal(0, 1e-2, n).astype(np.float32)
        if gtype == O.BF16:
            g = O.bf16_of_f32(g)
        m = (O.pack_halves(O.bf16_of_f32(rng.normal(0, 1e-3, n)
                                         .astype(np.float32)))
             if mkind else rng.normal(0, 1e-3, n).astype(np.float32))
        v = (O.pack_halves(O.bf16_of_f32(np.abs(rng.normal(0, 1e-5, n))
                                         .astype(np.float32)))
             if vkind else np.abs(rng.normal(0, 1e-5, n)).astype(np.float32))
        out.append(O.Tensor(w, g, m, v))
    return out


def _copy(ts):
    return [O.Tensor(x.w.copy(), x.g.copy(), x.m.copy(), x.v.copy())
            for x in ts]


@pytest.mark.parametrize("gtype,mkind,vkind",
                         [(0, 0, 0), (1, 0, 0), (0, 1, 1), (1, 1, 0)])
def test_multi_tensor_equals_per_tensor(gtype, mkind, vkind):
    rng = np.random.default_rng(9)
    for trial in range(20):
        k = rng.integers(1, 7)
        sizes = rng.integers(0, 18, size=k)
        ts = _rand_list(rng, sizes, gtype, mkind, vkind)
        hp = (3e-4, 0.9, 0.999, 1e-8, 0.1)
        joint = _copy(ts)
        nrm, c = O.step_(joint, gtype, mkind, vkind, *hp, t=3, s=0.5,
                         max_norm=0.01)
        perm = rng.permutation(k)
        for i in perm:                          # any order, one at a time
            one = _copy([ts[i]])
            O.step_(one, gtype, mkind, vkind, *hp, t=3, s=0.5, coef=c)
            for a, b in ((one[0].w, joint[i].w), (one[0].m, joint[i].m),
                         (one[0].v, joint[i].v)):
                assert np.array_equal(a.view(np.uint32) if a.dtype ==
                                      np.float32 else a,
                                      b.view(np.uint32) if b.dtype ==
                                      np.float32 else b)


def test_deferred_unscale_equals_in_place_scale_f32():
    # ScaleTensors then AdamW: for float32 gradients, scaling in registers
    # and scaling the stored gradient first give the same bits
    rng = np.random.default_rng(10)
    ts = _rand_list(rng, [1000, 31], O.F32, 0, 0)
    a, b = _copy(ts), _copy(ts)
    hp = (3e-4, 0.9, 0.999, 1e-8, 0.1)
    s = np.float32(1.0 / 3.0)
    O.step_(a, O.F32, 0, 0, *hp, t=2, s=s, max_norm=0.05)
    for x in b:
        O.scale_(x.g, O.F32, s)
    O.step_(b, O.F32, 0, 0, *hp, t=2, s=1.0, max_norm=0.05)
    for x, y in zip(a, b):
        assert np.array_equal(x.w, y.w) and np.array_equal(x.v, y.v)


def test_in_place_scale_bf16_matches_torch_rounding():
    rng = np.random.default_rng(11)
    g = O.bf16_of_f32(rng.normal(0, 60.0, 10000).astype(np.float32))
    for s in (2.0 ** -16, 0.3):
        x = g.copy()
        O.scale_(x, O.BF16, s)
        t = torch.from_numpy(g.view(np.int16).copy()).view(torch.bfloat16)
        ref = (t.float() * np.float32(s)).to(torch.bfloat16)
        assert np.array_equal(x, ref.view(torch.int16).numpy().view(np.uint16))


def test_nonfinite_gradient_propagates():
    g = np.array([1.0, np.nan, 2.0], np.float32)
    nrm = O.norm([g], O.F32)
    assert math.isnan(nrm)
    c = O.clip_coef(1.0, np.float32(nrm))
    assert np.isnan(c)
    g = np.array([1.0, np.inf], np.float32)
    assert O.norm([g], O.F32) == math.inf
    assert O.clip_coef(1.0, np.float32(O.norm([g], O.F32))) == 0.0
    g = np.array([np.inf, 1.0, -np.inf], np.float32)
    assert O.norm([g], O.F32) == math.inf


# ---------------------------------------------------------------------------
# bfloat16 weight copy ("Mica 7.7", float16 and bfloat16, whole: a product
# reads the float32 weights as bfloat16; "Precision and numerics": the cast
# is nearest-even)
# ---------------------------------------------------------------------------

def test_weight_copy_is_nearest_even_bfloat16():
    rng = np.random.default_rng(12)
    w = rng.normal(0, 0.02, 1 << 16).astype(np.float32)
    w[:4] = [0.8671875, np.float32(1.00390625), -0.0, np.inf]
    out = np.zeros(w.size, np.uint16)
    O.weight_copy(w, out)
    assert out[0] == 0x3F5E          # 0.8671875 = 1.1011110b * 2^-1, exact
    assert out[1] == 0x3F80          # tie between 0x3F80 and 0x3F81: even
    assert out[2] == 0x8000 and out[3] == 0x7F80
    ref = torch.from_numpy(w.copy()).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, ref)
    w[5] = np.nan
    O.weight_copy(w, out)
    assert out[5] == 0xFFFF


def test_step_writes_the_copy_of_the_new_weights():
    row = _golden_rows("hand_steps.txt")[2]      # case B: w -> 0.8671875
    w = np.array([1.0], np.float32)
    g = np.array([float(Fraction(row[6]))], np.float32)
    m, v = _mom_buf(O.MOM_BF16X2, 0.0), _mom_buf(O.MOM_BF16X2, 0.0)
    t = O.Tensor(w, g, m, v, w16=np.zeros(1, np.uint16))
    O.step_([t], O.F32, O.MOM_BF16X2, O.MOM_BF16X2, 0.125, 0.5, 0.75, 0.875,
            0.5, 1)
    assert float(t.w[0]) == 0.8671875 and t.w16[0] == 0x3F5E


# ---------------------------------------------------------------------------
# float16 ("Mica 7.7": float16 beside float32 everywhere; the unscaling a
# float16 step needs before its clip)
# ---------------------------------------------------------------------------

def test_f16_decode_all_patterns_match_numpy():
    h = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    got = O.f32_of_f16(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f16_encode_nearest_even_matches_numpy():
    # every float16 value, every midpoint between neighbours (ties), points
    # just either side of the midpoints, and random float32 over the range
    h = np.arange(0x7C00, dtype=np.uint32).astype(np.uint16)    # +0 .. max
    v = h.view(np.float16).astype(np.float64)
    mids = (v[:-1] + v[1:]) / 2                                # exact in f64
    rng = np.random.default_rng(13)
    xs = np.concatenate([
        v, -v, mids, -mids,
        np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
        np.nextafter(mids.astype(np.float32), np.float32(0)),
        rng.normal(0, 1, 1 << 16) * 10.0 ** rng.uniform(-9, 5, 1 << 16),
        [65504.0, 65519.99, 65520.0, 1e6, np.inf, -np.inf, 2.0 ** -25,
         2.0 ** -25 * 1.0000001, 3 * 2.0 ** -25]]).astype(np.float32)
    got = O.f16_of_f32(xs)
    with np.errstate(over="ignore"):
        ref = xs.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)
    assert O.f16_of_f32(np.array([np.nan, -np.nan], np.float32)).tolist() == [
        0xFFFF, 0xFFFF]


# ---------------------------------------------------------------------------
# loss scaling state (reading: PyTorch's GradScaler)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("b", [0.9, 0.999, 0.95, 0.5, 0.123456789])
def test_pow_rn_is_the_correctly_rounded_power(b):
    for t in list(range(1, 40)) + [64, 127, 500, 1000]:
        exact = Fraction(b) ** t
        assert O.pow_rn(b, t) == float(exact), (b, t)   # Fraction rounds RN


def test_scalars_rn_agree_with_the_host_form():
    # the two forms differ only where libm's pow is not correctly rounded
    diff = 0
    for t in range(1, 3000):
        a = O.scalars(3e-4, 0.9, 0.999, 1e-8, 0.1, t)
        b = O.scalars_rn(3e-4, 0.9, 0.999, 1e-8, 0.1, t)
        diff += int(np.any(a.view(np.uint32) != b.view(np.uint32)))
    assert diff <= 3


def test_amp_update_matches_torch_amp_update_scale():
    rng = np.random.default_rng(14)
    flags = rng.random(300) < 0.1
    amp = O.AmpState(65536.0)
    scale = torch.full((1,), 65536.0)
    tracker = torch.zeros(1, dtype=torch.int32)
    good = 0
    for f in flags:
        found = torch.full((1,), 1.0 if f else 0.0)
        torch._amp_update_scale_(scale, tracker, found, 2.0, 0.5, 7)
        amp.found_inf = np.float32(1.0 if f else 0.0)
        amp.update(2.0, 0.5, 7)
        good += int(not f)
        assert amp.scale == np.float32(scale.item())
        assert amp.tracker == int(tracker.item())
        assert amp.step == good and amp.found_inf == 0.0


def test_amp_update_keeps_the_scale_finite():
    amp = O.AmpState(np.float32(3e38))
    amp.update(2.0, 0.5, 1)                # 6e38 is not finite: no growth
    assert amp.scale == np.float32(3e38) and amp.tracker == 0


def test_amp_step_skips_on_non_finite_and_matches_plain_step_otherwise():
    rng = np.random.default_rng(15)
    n = 3000
    g = (rng.normal(0, 1e-3, n) * 1024).astype(np.float32)
    gh = O.f16_of_f32(g)
    mk = lambda: O.Tensor(rng.normal(0, .02, n).astype(np.float32), gh.copy(),
                          np.zeros(n, np.float32), np.zeros(n, np.float32))
    a = mk()
    b = O.Tensor(a.w.copy(), a.g.copy(), a.m.copy(), a.v.copy())
    amp = O.AmpState(1024.0, step=4)
    nrm, c, found = O.amp_step_([a], O.F16, 0, 0, amp, 3e-4, 0.9, 0.999,
                                1e-8, 0.1, 1.0)
    assert not found and amp.found_inf == 0.0
    # the same step through the plain path: unscale by 1/1024, t = 5
    O.step_([b], O.F16, 0, 0, 3e-4, 0.9, 0.999, 1e-8, 0.1, 5,
            s=1.0 / 1024, max_norm=1.0)
    assert np.array_equal(a.w, b.w) and np.array_equal(a.v, b.v)
    # an Inf gradient: found_inf, nothing written
    a.g[7] = 0x7C00
    w0 = a.w.copy()
    nrm, c, found = O.amp_step_([a], O.F16, 0, 0, amp, 3e-4, 0.9, 0.999,
                                1e-8, 0.1, 1.0)
    assert found and amp.found_inf == 1.0 and np.array_equal(a.w, w0)


# ---------------------------------------------------------------------------
# the other optimizers of "BendTorch main.bend", Optimizers: Adam with
# coupled decay (adam_grad / adam_decay with dec = False), SGD (sgd_l),
# momentum SGD (mom_l), and the zeroed gradient every step loop leaves
# ---------------------------------------------------------------------------

def test_sgd_exact_dyadic_step():
    # every product and sum below is exact in float32
    w = np.array([1.0, -2.0, 0.75, 0.0], np.float32)
    g = np.array([0.5, 0.25, -1.0, 3.0], np.float32)
    O.sgd_(w, g, O.F32, lr=0.5, s=0.5, coef=0.5)      # g' = g / 4
    assert w.tolist() == [1.0 - 0.0625, -2.0 - 0.03125, 0.75 + 0.125,
                          -0.375]
    assert g.tolist() == [0.5, 0.25, -1.0, 3.0]          # read only


def test_sgd_against_torch_cpu():
    rng = np.random.default_rng(31)
    n, lr = 4096, 0.01
    w = rng.normal(0, 0.02, n).astype(np.float32)
    p = torch.nn.Parameter(torch.from_numpy(w.copy()))
    opt = torch.optim.SGD([p], lr=lr, foreach=False)
    for _ in range(10):
        g = rng.normal(0, 1e-2, n).astype(np.float32)
        p.grad = torch.from_numpy(g.copy())
        opt.step()
        w_prev = w.copy()
        O.sgd_(w, g, O.F32, lr)
        # torch's add with alpha may fuse the multiply: the two differ by
        # the product's rounding, an ulp of the larger term at most
        scale = np.maximum(np.abs(w_prev), np.abs(np.float32(lr) * g))
        scale = np.maximum(scale, np.abs(w))       # the result's binade
        assert np.all(np.abs(w - p.detach().numpy()) <= np.spacing(scale))
        p.data.copy_(torch.from_numpy(w))          # restart from ours


def test_momentum_geometric_series_is_exact():
    # constant g = 1, mu = 1/2: buf_t = 2 (1 - 2^-t) and
    # w_t = w0 - lr * sum_k buf_k, all exact dyadic numbers here
    w = np.array([8.0], np.float32)
    buf = np.zeros(1, np.float32)
    g = np.ones(1, np.float32)
    lr, mu = 0.25, 0.5
    total = Fraction(0)
    for t in range(1, 21):
        O.momentum_(w, g, buf, O.F32, lr, mu)
        bt = 2 * (1 - Fraction(1, 2 ** t))
        total += bt
        assert Fraction(float(buf[0])) == bt, t
        assert Fraction(float(w[0])) == 8 - Fraction(1, 4) * total, t


def test_momentum_against_torch_cpu():
    rng = np.random.default_rng(32)
    n, lr, mu = 4096, 0.01, 0.9
    w = rng.normal(0, 0.02, n).astype(np.float32)
    buf = np.zeros(n, np.float32)
    p = torch.nn.Parameter(torch.from_numpy(w.copy()))
    opt = torch.optim.SGD([p], lr=lr, momentum=mu, foreach=False)
    for t in range(10):
        g = rng.normal(0, 1e-2, n).astype(np.float32)
        p.grad = torch.from_numpy(g.copy())
        opt.step()
        w_prev, b_prev = w.copy(), buf.copy()
        O.momentum_(w, g, buf, O.F32, lr, mu)
        tb = opt.state[p]["momentum_buffer"].numpy()
        # torch's first step clones g (ours: 0*mu + g, the same value); the
        # later ones are buf*mu + g, as here, where an FMA would differ by
        # the product's rounding; the weight update likewise
        bscale = np.maximum(np.abs(b_prev * np.float32(mu)), np.abs(g))
        bscale = np.maximum(bscale, np.abs(buf))
        assert np.all(np.abs(buf - tb) <= np.spacing(bscale))
        scale = np.maximum(np.abs(w_prev), np.abs(np.float32(lr) * buf))
        scale = np.maximum(scale, np.abs(w))
        assert np.all(np.abs(w - p.detach().numpy()) <= np.spacing(scale))
        p.data.copy_(torch.from_numpy(w))
        opt.state[p]["momentum_buffer"].copy_(torch.from_numpy(buf))


def _adam_scalars(t, lr=3e-4, b1=0.9, b2=0.999, eps=1e-8, wd=0.1):
    return O.scalars(lr, b1, b2, eps, wd, t)


def test_adam_coupled_decay_first_step_direction():
    # Adam's decay enters the gradient: g' = g + wd*w.  With w = 1,
    # g = -0.1, wd = 0.5 the step follows g' = 0.4 and moves w DOWN by about
    # lr; AdamW would move it up (g < 0) and decay it separately.
    lr, wd = 1e-2, 0.5
    sc = O.scalars(lr, 0.9, 0.999, 1e-8, wd, 1)
    w = np.array([1.0], np.float32)
    g = np.array([-0.1], np.float32)
    m = np.zeros(1, np.float32)
    v = np.zeros(1, np.float32)
    O.adam_(w, g, m, v, O.F32, 0, 0, sc, coupled=True, l2=wd)
    # first step from zero moments: w1 = w - lr * g'/(|g'| + eps), no decay
    gp = -0.1 + 0.5
    assert abs(float(w[0]) - (1.0 - lr * gp / (abs(gp) + 1e-8))) < 4e-7
    assert abs(float(m[0]) - 0.1 * gp) < 1e-7
    assert abs(float(v[0]) - 0.001 * gp * gp) < 1e-9
    ww = np.array([1.0], np.float32)
    O.adamw_(ww, g, np.zeros(1, np.float32), np.zeros(1, np.float32), O.F32,
             0, 0, sc)
    assert ww[0] > 1.0 - lr * wd and w[0] < 1.0 - 0.9 * lr


def test_adam_with_zero_decay_equals_adamw_with_zero_decay():
    rng = np.random.default_rng(33)
    n = 3000
    for t in (1, 2, 7):
        w = rng.normal(0, 0.02, n).astype(np.float32)
        g = rng.normal(0, 1e-3, n).astype(np.float32)
        m = rng.normal(0, 1e-3, n).astype(np.float32)
        v = np.abs(rng.normal(0, 1e-6, n)).astype(np.float32)
        a = [x.copy() for x in (w, g, m, v)]
        b = [x.copy() for x in (w, g, m, v)]
        sc = O.scalars(3e-4, 0.9, 0.999, 1e-8, 0.0, t)
        O.adam_(*a, O.F32, 0, 0, sc, coupled=True, l2=0.0)
        O.adamw_(*b, O.F32, 0, 0, sc)
        for x, y in zip(a, b):
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


def test_adam_against_torch_cpu():
    rng = np.random.default_rng(34)
    n, steps = 4096, 10
    lr, b1, b2, eps, wd = 3e-4, 0.9, 0.999, 1e-8, 0.1
    w0 = rng.normal(0, 0.02, n).astype(np.float32)
    p = torch.nn.Parameter(torch.from_numpy(w0.copy()))
    opt = torch.optim.Adam([p], lr=lr, betas=(b1, b2), eps=eps,
                           weight_decay=wd, foreach=False, fused=False)
    w = w0.copy()
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    for t in range(1, steps + 1):
        g = rng.normal(0, 1e-2, n).astype(np.float32)
        p.grad = torch.from_numpy(g.copy())
        opt.step()
        O.adam_(w, g, m, v, O.F32, 0, 0, O.scalars(lr, b1, b2, eps, wd, t),
                coupled=True, l2=wd)
    st = opt.state[p]
    u = 2.0 ** -24
    wscale = np.abs(w0) + steps * lr
    assert np.all(np.abs(w - p.detach().numpy()) <=
                  steps * (np.spacing(wscale) + 4 * u * lr))
    assert np.all(np.abs(m - st["exp_avg"].numpy()) <=
                  steps * 2 * u * (np.abs(st["exp_avg"].numpy()) + 1e-2))
    assert ulp_dist(v, st["exp_avg_sq"].numpy()).max() <= 4


@pytest.mark.parametrize("gtype", [O.F32, O.BF16, O.F16])
@pytest.mark.parametrize("kind", O.OPT_KINDS)
def test_zeroing_writes_plus_zero_and_changes_nothing_else(kind, gtype):
    rng = np.random.default_rng(35)
    n = 1001
    opt = dict(kind=kind, lr=1e-2, beta1=0.9, beta2=0.999, eps=1e-8,
               weight_decay=0.1 if kind.startswith("adam") else 0.0,
               momentum=0.9)

    def mk():
        r = np.random.default_rng(36)
        g = r.normal(0, 1e-2, n).astype(np.float32)
        g[::7] = -0.0
        if gtype == O.BF16:
            g = O.bf16_of_f32(g)
        elif gtype == O.F16:
            g = O.f16_of_f32(g)
        m = r.normal(0, 1e-3, n).astype(np.float32)
        v = np.abs(r.normal(0, 1e-5, n)).astype(np.float32)
        return O.Tensor(r.normal(0, .02, n).astype(np.float32), g, m, v)

    a, b = mk(), mk()
    O.opt_step_([a], opt, gtype, 0, 0, 3, s=0.5, max_norm=1.0, zero=False)
    O.opt_step_([b], opt, gtype, 0, 0, 3, s=0.5, max_norm=1.0, zero=True)
    assert not np.any(b.g.view(np.uint16 if gtype else np.uint32))
    for x, y in ((a.w, b.w), (a.m, b.m), (a.v, b.v)):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    assert rng is not None


@pytest.mark.parametrize("kind", O.OPT_KINDS)
def test_amp_opt_step_skip_zeroes_only_the_gradient(kind):
    n = 500
    r = np.random.default_rng(37)
    g = O.f16_of_f32((r.normal(0, 1e-3, n) * 1024).astype(np.float32))
    g[3] = 0x7C00                                       # +Inf
    x = O.Tensor(r.normal(0, .02, n).astype(np.float32), g,
                 r.normal(0, 1e-3, n).astype(np.float32),
                 np.abs(r.normal(0, 1e-5, n)).astype(np.float32))
    before = [x.w.copy(), x.m.copy(), x.v.copy()]
    amp = O.AmpState(1024.0, step=9)
    opt = dict(kind=kind, lr=1e-2, beta1=0.9, beta2=0.999, eps=1e-8,
               weight_decay=0.0, momentum=0.9)
    nrm, c, found = O.amp_opt_step_([x], opt, O.F16, 0, 0, amp, 1.0,
                                    zero=True)
    assert found and amp.found_inf == 1.0 and not np.any(x.g)
    for a, b in zip(before, (x.w, x.m, x.v)):
        assert np.array_equal(a, b)


def test_amp_opt_step_equals_plain_step_at_the_next_t():
    n = 700
    r = np.random.default_rng(38)
    g = O.f16_of_f32((r.normal(0, 1e-3, n) * 256).astype(np.float32))
    for kind in O.OPT_KINDS:
        opt = dict(kind=kind, lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8,
                   weight_decay=0.05 if kind.startswith("adam") else 0.0,
                   momentum=0.5)
        mk = lambda: O.Tensor(np.full(n, 0.01, np.float32), g.copy(),
                              np.full(n, 1e-4, np.float32),
                              np.full(n, 1e-8, np.float32))
        a, b = mk(), mk()
        amp = O.AmpState(256.0, step=4)
        O.amp_opt_step_([a], opt, O.F16, 0, 0, amp, 1.0)
        O.opt_step_([b], opt, O.F16, 0, 0, 5, s=1.0 / 256, max_norm=1.0)
        assert np.array_equal(a.w, b.w) and np.array_equal(a.m, b.m), kind


def test_float16_weight_copy_is_numpys_nearest_even():
    # "float16 and bfloat16, whole": a float16 step's product reads the
    # float32 weights as float16; the copy is numpy's conversion bit for bit
    rng = np.random.default_rng(41)
    w = np.concatenate([rng.normal(0, 0.02, 50000),
                        rng.normal(0, 1e4, 5000),
                        [65504.0, 65520.0, 1e-8, -0.0, np.inf]]).astype(
                            np.float32)
    out = np.zeros(w.size, np.uint16)
    O.weight_copy(w, out, O.F16)
    with np.errstate(over="ignore"):
        want = w.astype(np.float16).view(np.uint16)
    assert np.array_equal(out, want)
    nan = np.array([np.nan], np.float32)
    o1 = np.zeros(1, np.uint16)
    O.weight_copy(nan, o1, O.F16)
    assert o1[0] == 0xFFFF


def test_step_writes_a_float16_copy_when_asked():
    rng = np.random.default_rng(42)
    n = 1001
    x = O.Tensor(rng.normal(0, 0.02, n).astype(np.float32),
                 rng.normal(0, 1e-3, n).astype(np.float32),
                 np.zeros(n, np.float32), np.zeros(n, np.float32),
                 np.zeros(n, np.uint16), O.F16)
    O.step_([x], O.F32, 0, 0, 3e-4, 0.9, 0.999, 1e-8, 0.1, 1)
    assert np.array_equal(x.w16, x.w.astype(np.float16).view(np.uint16))


def test_joint_norm_over_mixed_gradient_types_is_the_exact_norm():
    # brute force: exact rational sum of the squares of f32(g*s) over a
    # float32 list, a bfloat16 list and a float16 list, each with its own
    # unscale factor; the oracle's compensated float64 sum must be the
    # correctly rounded sum to within a couple of float64 ulps
    from fractions import Fraction
    rng = np.random.default_rng(51)
    a = [rng.normal(0, 3, 40).astype(np.float32),
         rng.normal(0, 1e-3, 7).astype(np.float32)]
    b = [O.bf16_of_f32(rng.normal(0, 50, 33).astype(np.float32))]
    c = [O.f16_of_f32(rng.normal(0, 2, 21).astype(np.float32))]
    parts = [(a, O.F32, 1.0), (b, O.BF16, 2.0 ** -6), (c, O.F16, 0.3)]
    exact = Fraction(0)
    for grads, gtype, s in parts:
        for g in grads:
            x = g if gtype == O.F32 else (O.f32_of_bf16(g) if gtype == O.BF16
                                          else O.f32_of_f16(g))
            xs = (x.astype(np.float32) * np.float32(s)).astype(np.float32)
            exact += sum(Fraction(float(v)) ** 2 for v in xs)
    got = O.joint_sumsq(parts)
    assert abs(Fraction(got) - exact) <= exact * Fraction(1, 2 ** 51)
    # one type throughout: the joint sum is the plain sum of the
    # concatenation, bit for bit (the same terms in the same order)
    assert O.joint_sumsq([(a[:1], O.F32, 1.0), (a[1:], O.F32, 1.0)]) == \
        O.sumsq(a, O.F32)
    # a missing part changes the result: every part is counted
    assert O.joint_sumsq(parts[:2]) < got


@pytest.mark.parametrize("kind", ["adamw", "adam"])
def test_zero_decay_keeps_a_zero_gradient_tensor_exactly(kind):
    # The reading behind per-tensor no-decay flags: a flagged tensor takes
    # the step with weight_decay = 0.  Closed form from zero gradient and
    # zero moments: m1 = v1 = 0, so the Adam term is (-step * 0) / eps = -0
    # and w_new = w' exactly.  With weight_decay = 0, AdamW's factor is
    # f32(1 - lr*0) = 1 and Adam's coupled term is w*0 = +-0, so w keeps
    # every bit; with weight_decay > 0, AdamW gives w * f32(1 - lr*wd)
    # exactly and Adam's coupled term moves w.
    rng = np.random.default_rng(12)
    w = (rng.standard_normal(257) * 0.02).astype(np.float32)
    lr, wd = 3e-4, 0.1
    out = {}
    for decay in (0.0, wd):
        x = O.Tensor(w.copy(), np.zeros(257, np.float32),
                     np.zeros(257, np.float32), np.zeros(257, np.float32))
        O.opt_step_([x], dict(kind=kind, lr=lr, beta1=0.9, beta2=0.999,
                              eps=1e-8, weight_decay=decay, momentum=0.0),
                    O.F32, O.MOM_F32, O.MOM_F32, 1)
        out[decay] = x.w
    assert np.array_equal(out[0.0].view(np.uint32), w.view(np.uint32))
    if kind == "adamw":
        dec = np.float32(1.0 - lr * wd)
        assert np.array_equal(out[wd].view(np.uint32),
                              (w * dec).view(np.uint32))
    else:
        assert not np.array_equal(out[wd], w)
