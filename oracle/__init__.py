"""CPU oracle for the fused mixed-precision clip + multi-tensor AdamW step.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product path never imports this
package, and this package imports nothing from the product.

The arithmetic lives in ``mta_oracle.c`` (plain loops, one IEEE float32
operation at a time, compiled without FMA contraction); this module marshals
numpy arrays into it and drives a whole tensor list in list order.

Sources, by page title and section:
  * "Mica 7.7: a training step on the card, in every float type",
    "The whole model in one call": ClipGradNorms (joint L2 norm, one cap),
    AdamWSteps (each group updated as AdamWStep alone), ScaleTensors.
  * "BendTorch main.bend", "Optimizers": the Adam-family element arithmetic
    in PyTorch's order, the packed-bfloat16 moments, the bias-correction
    scalars; "Training": q1 = 1 - b1^t, q2 = 1 - b2^t with t = 1 first.

Layouts accepted here:
  * float32 arrays: ``numpy.float32``;
  * bfloat16 gradients: ``numpy.uint16`` bit patterns, one per element;
  * packed bfloat16 moments: ``numpy.uint32`` words, ceil(n / 2) of them,
    element 2k in the low half of word k.

Pins: every function here is checked in ``tests/test_oracle_pins.py``
against values fixed by the pages or by mathematics (closed forms, exact
sums, hand-computed steps, library routines for the special cases they
share).  Nothing here is "parity unpinned" except bitwise agreement with
PyTorch's own kernels, which the pages do not fix.
"""
import ctypes
import math
import os

import numpy as np

from . import build as _build

F32, BF16, F16 = 0, 1, 2
MOM_F32, MOM_BF16X2 = 0, 1

_lib = None


def lib():
    """Load the oracle library, compiling it first if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        vp, i64, f32, f64 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_double)
        L.mto_bf16_of_bits.argtypes = [ctypes.c_uint32]
        L.mto_bf16_of_bits.restype = ctypes.c_uint32
        L.mto_f32_of_bf16.argtypes = [ctypes.c_uint32]
        L.mto_f32_of_bf16.restype = f32
        L.mto_bf16_of_bits_array.argtypes = [i64, vp, vp]
        L.mto_bf16_of_bits_array.restype = None
        L.mto_scalars.argtypes = [f64, f64, f64, f64, f64, i64, vp]
        L.mto_scalars.restype = None
        L.mto_scale_tensor.argtypes = [i64, vp, ctypes.c_int, f32]
        L.mto_scale_tensor.restype = None
        L.mto_sumsq_accumulate.argtypes = [i64, vp, ctypes.c_int, f32, vp]
        L.mto_sumsq_accumulate.restype = None
        L.mto_clip_coef.argtypes = [f32, f32]
        L.mto_clip_coef.restype = f32
        L.mto_adamw_tensor.argtypes = [i64, vp, vp, ctypes.c_int, vp,
                                       ctypes.c_int, vp, ctypes.c_int, f32,
                                       f32, vp]
        L.mto_adamw_tensor.restype = None
        L.mto_adam_tensor.argtypes = [i64, vp, vp, ctypes.c_int, vp,
                                      ctypes.c_int, vp, ctypes.c_int, f32,
                                      f32, vp, ctypes.c_int, f32,
                                      ctypes.c_int]
        L.mto_adam_tensor.restype = None
        L.mto_sgd_tensor.argtypes = [i64, vp, vp, ctypes.c_int, f32, f32,
                                     f32, ctypes.c_int]
        L.mto_sgd_tensor.restype = None
        L.mto_momentum_tensor.argtypes = [i64, vp, vp, ctypes.c_int, vp, f32,
                                          f32, f32, f32, ctypes.c_int]
        L.mto_momentum_tensor.restype = None
        L.mto_weight_copy.argtypes = [i64, vp, vp]
        L.mto_weight_copy.restype = None
        L.mto_f32_of_f16.argtypes = [ctypes.c_uint32]
        L.mto_f32_of_f16.restype = f32
        L.mto_f16_of_f32.argtypes = [f32]
        L.mto_f16_of_f32.restype = ctypes.c_uint32
        L.mto_f16_of_f32_array.argtypes = [i64, vp, vp]
        L.mto_f16_of_f32_array.restype = None
        L.mto_f32_of_f16_array.argtypes = [i64, vp, vp]
        L.mto_f32_of_f16_array.restype = None
        L.mto_pow_rn.argtypes = [f64, i64]
        L.mto_pow_rn.restype = f64
        L.mto_scalars_rn.argtypes = [f64, f64, f64, f64, f64, i64, vp]
        L.mto_scalars_rn.restype = None
        L.mto_inv_scale.argtypes = [f32]
        L.mto_inv_scale.restype = f32
        i32p = ctypes.POINTER(ctypes.c_int32)
        f32p = ctypes.POINTER(ctypes.c_float)
        L.mto_amp_update.argtypes = [f32p, i32p, f32p,
                                     ctypes.POINTER(ctypes.c_int64), f64, f64,
                                     ctypes.c_int32]
        L.mto_amp_update.restype = None
        _lib = L
    return _lib


def _ptr(a, dtype):
    if not isinstance(a, np.ndarray) or a.dtype != dtype:
        raise TypeError(f"expected a numpy {np.dtype(dtype).name} array")
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError("array must be C-contiguous")
    return a.ctypes.data_as(ctypes.c_void_p)


def _grad_dtype(gtype):
    return np.uint16 if gtype in (BF16, F16) else np.float32


def _mom_dtype(kind):
    return np.uint32 if kind == MOM_BF16X2 else np.float32


def packed_words(n):
    """Number of u32 words that hold n packed bfloat16 values: ceil(n/2)."""
    return (n + 1) // 2


# ---------------------------------------------------------------- bfloat16

def bf16_of_bits(u):
    """float32 bit pattern -> bfloat16 bit pattern (RNE, NaN -> 0xFFFF)."""
    return int(lib().mto_bf16_of_bits(int(u) & 0xFFFFFFFF))


def bf16_of_f32(x):
    """Round a float32 array to bfloat16 bit patterns (numpy uint16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().mto_bf16_of_bits_array(x.size, _ptr(x.view(np.uint32), np.uint32),
                                 _ptr(out, np.uint16))
    return out


def f32_of_bf16(h):
    """bfloat16 bit patterns -> float32 (exact: the bits move up 16)."""
    h = np.asarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def unpack_words(words, n):
    """Packed u32 words -> n bfloat16 bit patterns, element order."""
    words = np.asarray(words, dtype=np.uint32)
    out = np.empty(2 * words.size, dtype=np.uint16)
    out[0::2] = (words & np.uint32(0xFFFF)).astype(np.uint16)
    out[1::2] = (words >> np.uint32(16)).astype(np.uint16)
    return out[:n]


def pack_halves(h):
    """n bfloat16 bit patterns -> ceil(n/2) u32 words (pad half zero)."""
    h = np.asarray(h, dtype=np.uint16)
    n = h.size
    padded = np.zeros(2 * packed_words(n), dtype=np.uint32)
    padded[:n] = h
    return (padded[0::2] | (padded[1::2] << np.uint32(16))).astype(np.uint32)


# ---------------------------------------------------------------- scalars

def scalars(lr, beta1, beta2, eps, weight_decay, t):
    """{step, bc2, c1, c2, b2, eps, dec} as float32, formed in float64."""
    if t < 1:
        raise ValueError("t counts from 1")
    out = np.zeros(7, dtype=np.float32)
    lib().mto_scalars(lr, beta1, beta2, eps, weight_decay, int(t),
                      _ptr(out, np.float32))
    return out


SCALAR_NAMES = ("step", "bc2", "c1", "c2", "b2", "eps", "dec")


# ---------------------------------------------------------------- scale

def scale_(g, gtype, s):
    """ScaleTensors in place on one gradient array (bf16 rounds back)."""
    lib().mto_scale_tensor(g.size, _ptr(g, _grad_dtype(gtype)), gtype,
                           float(s))


# ---------------------------------------------------------------- norm

def joint_sumsq(parts):
    """Joint sum of squares over several gradient lists, each with its own
    gradient type and unscale factor: parts = [(grads, gtype, s), ...].
    The one cap of ClipGradNorms is over the joint length of every gradient
    the step names ("Mica 7.7", "The whole model in one call"), whatever
    type each is stored in (under bfloat16, a high-numerics parameter keeps
    a float32 gradient: "Precision and numerics", Parameters).  Every
    f32(g*s)^2 goes into one compensated float64 sum, in list order."""
    state = np.zeros(2, dtype=np.float64)
    L = lib()
    for grads, gtype, s in parts:
        for g in grads:
            L.mto_sumsq_accumulate(g.size, _ptr(g, _grad_dtype(gtype)),
                                   gtype, float(s), _ptr(state, np.float64))
    return float(state[0] + state[1])


def joint_norm(parts):
    """L2 norm of joint_sumsq(parts) (float64, effectively exact)."""
    return math.sqrt(joint_sumsq(parts))


def sumsq(grads, gtype, s=1.0):
    """Joint sum of squares of f32(g*s) over a list of gradient arrays."""
    return joint_sumsq([(grads, gtype, s)])


def norm(grads, gtype, s=1.0):
    """Joint L2 norm (float64, effectively exact)."""
    return math.sqrt(sumsq(grads, gtype, s))


def clip_coef(max_norm, norm_f32):
    """min(1, max/(norm + 1e-6)) in float32; NaN passes through."""
    return np.float32(lib().mto_clip_coef(float(np.float32(max_norm)),
                                          float(np.float32(norm_f32))))


# ---------------------------------------------------------------- AdamW

def adamw_(w, g, m, v, gtype, mkind, vkind, sc, s=1.0, coef=1.0):
    """One AdamW step over one tensor, in place on w, m, v."""
    n = w.size
    if g.size != n:
        raise ValueError("gradient size differs from the weight's")
    for buf, kind in ((m, mkind), (v, vkind)):
        want = packed_words(n) if kind == MOM_BF16X2 else n
        if buf.size != want:
            raise ValueError("moment buffer has the wrong size")
    sc = np.ascontiguousarray(sc, dtype=np.float32)
    lib().mto_adamw_tensor(n, _ptr(w, np.float32), _ptr(g, _grad_dtype(gtype)),
                           gtype, _ptr(m, _mom_dtype(mkind)), mkind,
                           _ptr(v, _mom_dtype(vkind)), vkind,
                           float(np.float32(s)), float(np.float32(coef)),
                           _ptr(sc, np.float32))


def adam_(w, g, m, v, gtype, mkind, vkind, sc, s=1.0, coef=1.0,
          coupled=False, l2=0.0, zero=False):
    """One Adam-family step over one tensor, in place on w, m, v (and g when
    ``zero``).  coupled=False is AdamW (decay factor sc[6]); coupled=True is
    Adam with g' = g + f32(w * l2) and no decay of w."""
    n = w.size
    if g.size != n:
        raise ValueError("gradient size differs from the weight's")
    for buf, kind in ((m, mkind), (v, vkind)):
        want = packed_words(n) if kind == MOM_BF16X2 else n
        if buf.size != want:
            raise ValueError("moment buffer has the wrong size")
    sc = np.ascontiguousarray(sc, dtype=np.float32)
    lib().mto_adam_tensor(n, _ptr(w, np.float32), _ptr(g, _grad_dtype(gtype)),
                          gtype, _ptr(m, _mom_dtype(mkind)), mkind,
                          _ptr(v, _mom_dtype(vkind)), vkind,
                          float(np.float32(s)), float(np.float32(coef)),
                          _ptr(sc, np.float32), int(bool(coupled)),
                          float(np.float32(l2)), int(bool(zero)))


def sgd_(w, g, gtype, lr, s=1.0, coef=1.0, zero=False):
    """SGD over one tensor: w <- w + (-lr) * f32(f32(g*s)*coef)."""
    if g.size != w.size:
        raise ValueError("gradient size differs from the weight's")
    lib().mto_sgd_tensor(w.size, _ptr(w, np.float32),
                         _ptr(g, _grad_dtype(gtype)), gtype,
                         float(np.float32(s)), float(np.float32(coef)),
                         float(np.float32(lr)), int(bool(zero)))


def momentum_(w, g, buf, gtype, lr, mu, s=1.0, coef=1.0, zero=False):
    """SGD with momentum over one tensor: buf <- buf*mu + g';
    w <- w + (-lr)*buf (float32 buffer)."""
    if g.size != w.size or buf.size != w.size:
        raise ValueError("buffer sizes differ from the weight's")
    lib().mto_momentum_tensor(w.size, _ptr(w, np.float32),
                              _ptr(g, _grad_dtype(gtype)), gtype,
                              _ptr(buf, np.float32), float(np.float32(s)),
                              float(np.float32(coef)), float(np.float32(lr)),
                              float(np.float32(mu)), int(bool(zero)))


def weight_copy(w, out, ctype=BF16):
    """16-bit copy of float32 weights: bfloat16 (ctype BF16, the default) or
    IEEE float16 (ctype F16), nearest-even, NaN -> 0xFFFF."""
    if out.size != w.size:
        raise ValueError("copy buffer has the wrong size")
    if ctype == F16:
        out[...] = f16_of_f32(w)
    elif ctype == BF16:
        lib().mto_weight_copy(w.size, _ptr(w, np.float32),
                              _ptr(out, np.uint16))
    else:
        raise ValueError("a weight copy is bfloat16 or float16")


class Tensor:
    """One parameter group: weight, gradient and the two moments, and an
    optional 16-bit copy of the weight (numpy uint16, bfloat16 or float16
    by w16_type, written after each step when present)."""

    def __init__(self, w, g, m, v, w16=None, w16_type=BF16):
        self.w, self.g, self.m, self.v, self.w16 = w, g, m, v, w16
        self.w16_type = w16_type

    @property
    def n(self):
        return self.w.size


def step_(tensors, gtype, mkind, vkind, lr, beta1, beta2, eps, weight_decay,
          t, s=1.0, max_norm=None, coef=None):
    """The whole step over a tensor list, in list order.

    Unscale by ``s`` (in registers), clip by the joint norm when
    ``max_norm`` is given, then AdamW every group.  ``coef`` overrides the
    coefficient the oracle would compute (used to compare against a device
    run in lockstep).  Returns ``(norm_f64, coef_f32)``; the norm is None
    when no clip is asked for.
    """
    nrm = None
    c = np.float32(1.0)
    if max_norm is not None:
        nrm = norm([x.g for x in tensors], gtype, s)
        c = clip_coef(max_norm, np.float32(nrm))
    if coef is not None:
        c = np.float32(coef)
    sc = scalars(lr, beta1, beta2, eps, weight_decay, t)
    for x in tensors:
        adamw_(x.w, x.g, x.m, x.v, gtype, mkind, vkind, sc, s, c)
        if getattr(x, "w16", None) is not None:
            weight_copy(x.w, x.w16, getattr(x, "w16_type", BF16))
    return nrm, c


# ---------------------------------------------------------------- float16

def f32_of_f16(h):
    """float16 bit patterns -> float32 (exact)."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib().mto_f32_of_f16_array(h.size, _ptr(h, np.uint16),
                               _ptr(out, np.float32))
    return out


def f16_of_f32(x):
    """float32 -> float16 bit patterns (nearest-even, NaN -> 0xFFFF)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().mto_f16_of_f32_array(x.size, _ptr(x, np.float32),
                               _ptr(out, np.uint16))
    return out


# ---------------------------------------------------------------- AMP

def pow_rn(b, t):
    """b^t rounded once to the nearest float64."""
    return float(lib().mto_pow_rn(float(b), int(t)))


def scalars_rn(lr, beta1, beta2, eps, weight_decay, t):
    """As scalars(), with 1 - b^t from the correctly rounded power (the form
    the device computes from its own step counter)."""
    if t < 1:
        raise ValueError("t counts from 1")
    out = np.zeros(7, dtype=np.float32)
    lib().mto_scalars_rn(lr, beta1, beta2, eps, weight_decay, int(t),
                         _ptr(out, np.float32))
    return out


def inv_scale(scale):
    return np.float32(lib().mto_inv_scale(float(np.float32(scale))))


class AmpState:
    """The loss-scale state a caller keeps next to the tensors."""

    def __init__(self, scale, step=0, tracker=0, found_inf=0.0):
        self.scale = np.float32(scale)
        self.step = int(step)
        self.tracker = int(tracker)
        self.found_inf = np.float32(found_inf)

    def update(self, growth=2.0, backoff=0.5, interval=2000):
        sc = ctypes.c_float(self.scale)
        tr = ctypes.c_int32(self.tracker)
        fi = ctypes.c_float(self.found_inf)
        st = ctypes.c_int64(self.step)
        lib().mto_amp_update(ctypes.byref(sc), ctypes.byref(tr),
                             ctypes.byref(fi), ctypes.byref(st), growth,
                             backoff, interval)
        self.scale, self.tracker = np.float32(sc.value), tr.value
        self.found_inf, self.step = np.float32(fi.value), st.value


def amp_step_(tensors, gtype, mkind, vkind, amp, lr, beta1, beta2, eps,
              weight_decay, max_norm, coef=None):
    """One loss-scaled step: unscale by 1/S, joint norm, found_inf, clip,
    and the AdamW update at t = step + 1 unless a gradient is not finite.
    Does not call amp.update().  Returns (norm, coef, found_inf)."""
    s = inv_scale(amp.scale)
    nrm = norm([x.g for x in tensors], gtype, s)
    found = not math.isfinite(nrm)
    c = clip_coef(max_norm, np.float32(nrm)) if coef is None else \
        np.float32(coef)
    amp.found_inf = np.float32(1.0 if found else 0.0)
    if not found:
        sc = scalars_rn(lr, beta1, beta2, eps, weight_decay, amp.step + 1)
        for x in tensors:
            adamw_(x.w, x.g, x.m, x.v, gtype, mkind, vkind, sc, s, c)
            if getattr(x, "w16", None) is not None:
                weight_copy(x.w, x.w16, getattr(x, "w16_type", BF16))
    return nrm, c, found


# ---------------------------------------------------------------- optimizers

OPT_KINDS = ("adamw", "adam", "sgd", "momentum")


def _apply_opt(x, opt, gtype, mkind, vkind, sc, s, c, zero):
    kind = opt["kind"]
    if kind in ("adamw", "adam"):
        adam_(x.w, x.g, x.m, x.v, gtype, mkind, vkind, sc, s, c,
              coupled=(kind == "adam"), l2=opt["weight_decay"], zero=zero)
    elif kind == "sgd":
        sgd_(x.w, x.g, gtype, opt["lr"], s, c, zero)
    elif kind == "momentum":
        momentum_(x.w, x.g, x.m, gtype, opt["lr"], opt["momentum"], s, c,
                  zero)
    else:
        raise ValueError(f"unknown optimizer {kind!r}")
    if getattr(x, "w16", None) is not None:
        weight_copy(x.w, x.w16, getattr(x, "w16_type", BF16))


def opt_step_(tensors, opt, gtype, mkind, vkind, t, s=1.0, max_norm=None,
              coef=None, zero=False):
    """The whole step over a tensor list for any optimizer of the
    Optimizers section ("BendTorch main.bend"): opt is a dict with kind
    ("adamw", "adam", "sgd", "momentum"), lr, beta1, beta2, eps,
    weight_decay, momentum.  Unscale by s, clip by the joint norm when
    max_norm is given (coef overrides the coefficient), update every group,
    zero the gradients when asked.  Returns (norm_f64, coef_f32)."""
    nrm = None
    c = np.float32(1.0)
    if max_norm is not None:
        nrm = norm([x.g for x in tensors], gtype, s)
        c = clip_coef(max_norm, np.float32(nrm))
    if coef is not None:
        c = np.float32(coef)
    sc = None
    if opt["kind"] in ("adamw", "adam"):
        sc = scalars(opt["lr"], opt["beta1"], opt["beta2"], opt["eps"],
                     opt["weight_decay"], t)
    for x in tensors:
        _apply_opt(x, opt, gtype, mkind, vkind, sc, s, c, zero)
    return nrm, c


def amp_opt_step_(tensors, opt, gtype, mkind, vkind, amp, max_norm,
                  coef=None, zero=False):
    """opt_step_ under a loss-scale state: unscale by 1/S; when the norm is
    not finite the update is skipped (the gradients are still zeroed when
    asked); otherwise Adam-family constants come from t = amp.step + 1 with
    the correctly rounded power.  Does not call amp.update().  Returns
    (norm, coef, found_inf)."""
    s = inv_scale(amp.scale)
    nrm = norm([x.g for x in tensors], gtype, s)
    found = not math.isfinite(nrm)
    c = clip_coef(max_norm, np.float32(nrm)) if coef is None else \
        np.float32(coef)
    amp.found_inf = np.float32(1.0 if found else 0.0)
    if found:
        if zero:
            for x in tensors:
                x.g[...] = 0
        return nrm, c, found
    sc = None
    if opt["kind"] in ("adamw", "adam"):
        sc = scalars_rn(opt["lr"], opt["beta1"], opt["beta2"], opt["eps"],
                        opt["weight_decay"], amp.step + 1)
    for x in tensors:
        _apply_opt(x, opt, gtype, mkind, vkind, sc, s, c, zero)
    return nrm, c, found
