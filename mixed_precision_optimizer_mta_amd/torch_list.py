"""MtaList: a libmta tensor-list handle over PyTorch tensors.

Marshalling only.  It checks that the tensors are what the C ABI expects
(device, dtype, contiguity, element counts), passes their data pointers and
the current HIP stream, and owns the handle.  The tensors must keep their
storage for the handle's life (the library holds their addresses).
"""
import struct

import torch

from . import _binding as B

_G = {torch.float32: B.MTA_F32, torch.bfloat16: B.MTA_BF16,
      torch.float16: B.MTA_F16}
_M = {torch.float32: B.MTA_MOM_F32, torch.bfloat16: B.MTA_MOM_BF16X2}


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def current_stream():
    """The current HIP stream of the current device, as an integer handle
    (torch's raw-stream query when it has one: it skips building a Stream
    object, a few microseconds per call on a launch-bound loop)."""
    if _raw_stream is not None:
        return _raw_stream(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


class MtaList:
    """groups: sequence of (w, g, m, v) tensors.  w is float32; g float32,
    bfloat16 or float16; m and v float32 or bfloat16 (bfloat16 = packed
    moments), or None when the list's rule has no such state (SGD: neither,
    momentum: no v); all groups share the gradient type and each moment
    kind."""

    def __init__(self, groups, entries=None, gtype=None, mkind=None,
                 vkind=None):
        self._keep = list(groups)
        if entries is None:
            if not self._keep:
                raise ValueError("empty list: pass gtype/mkind/vkind and "
                                 "entries=[] explicitly")
            g0, m0, v0 = self._keep[0][1], self._keep[0][2], self._keep[0][3]

            def kind(t):
                return B.MTA_MOM_F32 if t is None else _M[t.dtype]

            gtype, mkind, vkind = _G[g0.dtype], kind(m0), kind(v0)
            entries = []
            for w, g, m, v in self._keep:
                for t in (w, g, m, v):
                    if t is not None and (not t.is_cuda or
                                          not t.is_contiguous()):
                        raise ValueError("tensors must be contiguous on the GPU")
                if w.dtype != torch.float32:
                    raise TypeError("w must be float32")
                if (_G.get(g.dtype), kind(m), kind(v)) != (
                        gtype, mkind, vkind):
                    raise TypeError("all groups must share g, m, v dtypes")
                n = w.numel()
                if g.numel() != n or any(t is not None and t.numel() != n
                                         for t in (m, v)):
                    raise ValueError("w, g, m, v must have the same numel")
                entries.append((w.data_ptr(), g.data_ptr(),
                                None if m is None else m.data_ptr(),
                                None if v is None else v.data_ptr(), n))
        self.gtype, self.mkind, self.vkind = gtype, mkind, vkind
        self.sizes = [int(e[4]) for e in entries]
        self.device = torch.cuda.current_device()
        self.handle = B.mta_list_create(entries, gtype, mkind, vkind,
                                        current_stream())

    def info(self):
        return B.mta_list_info(self.handle)

    def scale(self, factor, defer=True):
        B.mta_scale(self.handle, factor,
                    B.MTA_SCALE_DEFER if defer else B.MTA_SCALE_INPLACE,
                    current_stream())

    def scale_device(self, factor):
        """g = g * factor in place, factor a one-element float32 GPU tensor
        (for instance the coef a clip_norm left)."""
        if factor.dtype != torch.float32 or not factor.is_cuda:
            raise TypeError("the factor is a float32 GPU tensor")
        B.mta_scale_device(self.handle, factor.data_ptr(), current_stream())

    def clip_norm(self, max_norm, norm_out, coef_out):
        """norm_out (may be None) and coef_out: float32 device tensors."""
        for t in (norm_out, coef_out):
            if t is not None and (t.dtype != torch.float32 or not t.is_cuda):
                raise TypeError("norm/coef outputs are float32 GPU tensors")
        B.mta_clip_norm(self.handle, max_norm,
                        None if norm_out is None else norm_out.data_ptr(),
                        coef_out.data_ptr(), current_stream())

    def set_weight_copies(self, copies):
        """copies: one bfloat16 or float16 GPU tensor (or None) per group,
        each with the weight's numel and all of one dtype, written with the
        16-bit rounding of w by every later step; None detaches them all."""
        ptrs = None
        ctype = B.MTA_BF16
        if copies is not None:
            if len(copies) != len(self.sizes):
                raise ValueError("one copy (or None) per tensor of the list")
            ptrs = []
            for c, n in zip(copies, self.sizes):
                if c is None:
                    ptrs.append(None)
                    continue
                if c.numel() != n:
                    raise ValueError("a weight copy must have the weight's numel")
                if c.dtype not in (torch.bfloat16, torch.float16) or \
                        not c.is_cuda or not c.is_contiguous():
                    raise TypeError("weight copies are contiguous bfloat16 "
                                    "or float16 GPU tensors")
                ptrs.append(c.data_ptr())
            dts = {c.dtype for c in copies if c is not None}
            if len(dts) > 1:
                raise TypeError("the weight copies of a list share one dtype")
            if dts == {torch.float16}:
                ctype = B.MTA_F16
        B.mta_list_set_weight_copies_as(self.handle, ptrs, ctype,
                                        current_stream())
        # the list holds raw addresses: keep the tensors alive with it
        self._copies = None if copies is None else list(copies)

    def set_no_decay(self, flags):
        """flags: one truth value per group (True: that tensor's step
        takes weight_decay = 0, in the same launch as the others), or None
        to clear them."""
        if flags is not None and len(flags) != len(self.sizes):
            raise ValueError("one flag per tensor of the list")
        B.mta_list_set_no_decay(self.handle, flags, current_stream())
        self.no_decay = None if flags is None else [bool(f) for f in flags]

    def adamw_step(self, hparams, t, coef=None):
        if coef is not None and (coef.dtype != torch.float32 or
                                 not coef.is_cuda):
            raise TypeError("coef is a float32 GPU tensor")
        B.mta_adamw_step(self.handle, hparams, t,
                         None if coef is None else coef.data_ptr(),
                         current_stream())

    def step(self, opt, t, coef=None):
        """One step of any rule: opt is a dict (kind "adamw" / "adam" /
        "sgd" / "momentum", lr, beta1, beta2, eps, weight_decay, momentum,
        zero_grad)."""
        if coef is not None and (coef.dtype != torch.float32 or
                                 not coef.is_cuda):
            raise TypeError("coef is a float32 GPU tensor")
        B.mta_step(self.handle, opt, t,
                   None if coef is None else coef.data_ptr(),
                   current_stream())

    def amp_step(self, opt, amp, coef=None):
        """Loss-scaled step of any rule (see step)."""
        if coef is not None and (coef.dtype != torch.float32 or
                                 not coef.is_cuda):
            raise TypeError("coef is a float32 GPU tensor")
        B.mta_amp_step(self.handle, opt, amp.ptr,
                       None if coef is None else coef.data_ptr(),
                       current_stream())

    def amp_clip_norm(self, max_norm, amp, norm_out, coef_out):
        """Loss-scaled norm: unscales by 1/amp.scale on the device and sets
        amp's found_inf flag."""
        for t in (norm_out, coef_out):
            if t is not None and (t.dtype != torch.float32 or not t.is_cuda):
                raise TypeError("norm/coef outputs are float32 GPU tensors")
        B.mta_amp_clip_norm(self.handle, max_norm, amp.ptr,
                            None if norm_out is None else norm_out.data_ptr(),
                            coef_out.data_ptr(), current_stream())

    def amp_adamw_step(self, hparams, amp, coef=None):
        """Loss-scaled AdamW step: t and 1/scale come from amp on the
        device; no-op when its found_inf flag is set."""
        if coef is not None and (coef.dtype != torch.float32 or
                                 not coef.is_cuda):
            raise TypeError("coef is a float32 GPU tensor")
        B.mta_amp_adamw_step(self.handle, hparams, amp.ptr,
                             None if coef is None else coef.data_ptr(),
                             current_stream())

    def close(self):
        """Free the handle's device tables once the device is done with
        them: mta_list_destroy requires every stream that used the list to
        be synchronized, and work launched earlier may still be queued."""
        if self.handle is not None:
            torch.cuda.synchronize(self.device)
            B.mta_list_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def clip_norm_joint(lists, max_norm, norm_out, coef_out, amp=None):
    """One clip over the joint norm of several MtaLists (each with its own
    gradient type): mta_clip_norm_joint, or mta_amp_clip_norm_joint with
    a loss-scale state."""
    for t in (norm_out, coef_out):
        if t is not None and (t.dtype != torch.float32 or not t.is_cuda):
            raise TypeError("norm/coef outputs are float32 GPU tensors")
    handles = [L.handle for L in lists]
    nptr = None if norm_out is None else norm_out.data_ptr()
    if amp is None:
        B.mta_clip_norm_joint(handles, max_norm, nptr, coef_out.data_ptr(),
                              current_stream())
    else:
        B.mta_amp_clip_norm_joint(handles, max_norm, amp.ptr, nptr,
                                  coef_out.data_ptr(), current_stream())


class GradClipper:
    """Gradient clipping on the device, for gradients an optimizer of
    another kind will read: the joint L2 norm of every gradient, the
    coefficient min(1, max_norm / (norm + 1e-6)) and every gradient scaled by
    it in place (ClipGradNorms with the norm, the coefficient and the scaling
    all on the device).  For float32 gradients this is PyTorch's
    clip_grad_norm_ (same coefficient rule, in float32).  For bfloat16 and
    float16 gradients the norm here is the float64-accumulated norm of the
    exact values, rounded once to float32, while PyTorch's clip_grad_norm_
    forms per-tensor norms and the total in the gradients' own dtype; the
    two can then differ by about one ulp of that 16-bit dtype, and so can
    the coefficients.
    One gradient-only list per gradient dtype (built once, on the first call
    and again whenever a gradient moves); a call launches one norm per list
    (chained to a joint norm) and one in-place scale per list, and reads
    nothing back: the norm and the coefficient stay in device tensors."""

    def __init__(self, params):
        self.params = [p for p in params]
        self._lists, self._key = [], None
        self.norm = self.coef = None

    def _build(self, ps):
        for L in self._lists:
            L.close()
        self._lists = []
        for dt in _G:
            gs = [p.grad for p in ps if p.grad.dtype == dt]
            if gs:
                L = MtaList([], entries=[(None, g.data_ptr(), None, None,
                                          g.numel()) for g in gs],
                            gtype=_G[dt], mkind=B.MTA_MOM_F32,
                            vkind=B.MTA_MOM_F32)
                L._keep = gs
                self._lists.append(L)

    def __call__(self, max_norm):
        """Clip every gradient in place; returns the pre-clip joint norm as
        a one-element float32 device tensor (coef in ``self.coef``)."""
        ps = [p for p in self.params if p.grad is not None]
        for p in ps:
            g = p.grad
            if g.dtype not in _G or not g.is_cuda or not g.is_contiguous():
                raise TypeError("gradients are contiguous float32, bfloat16 "
                                "or float16 GPU tensors")
        key = tuple((p.grad.data_ptr(), p.grad.dtype, p.grad.numel())
                    for p in ps)
        if key != self._key:
            self._build(ps)
            self._key = key
        if not self._lists:
            return None
        dev = ps[0].grad.device
        if self.norm is None or self.norm.device != dev:
            self.norm = torch.zeros(1, device=dev)
            self.coef = torch.zeros(1, device=dev)
        clip_norm_joint(self._lists, float(max_norm), self.norm, self.coef)
        for L in self._lists:
            L.scale_device(self.coef)
        return self.norm

    def close(self):
        for L in self._lists:
            L.close()
        self._lists, self._key = [], None


class AmpState:
    """The 24-byte device loss-scale state of include/mta.h (mta_amp_state):
    scale, found_inf, growth_tracker, step.  Lives in device memory; reading
    it back (``read``) synchronizes the stream."""

    _FMT = "<ffiiq"

    def __init__(self, scale=65536.0, step=0, growth_tracker=0,
                 found_inf=0.0, device=None):
        self.buf = torch.empty(3, dtype=torch.int64,
                               device=device or torch.device("cuda"))
        self.write(scale, step, growth_tracker, found_inf)

    @property
    def ptr(self):
        return self.buf.data_ptr()

    def write(self, scale, step=0, growth_tracker=0, found_inf=0.0):
        raw = struct.pack(self._FMT, scale, found_inf, growth_tracker, 0, step)
        host = torch.frombuffer(bytearray(raw), dtype=torch.int64)
        self.buf.copy_(host)

    def read(self):
        raw = self.buf.cpu().numpy().tobytes()
        scale, found_inf, tracker, _, step = struct.unpack(self._FMT, raw)
        return {"scale": scale, "found_inf": found_inf,
                "growth_tracker": tracker, "step": step}

    def update(self, growth_factor=2.0, backoff_factor=0.5,
               growth_interval=2000):
        B.mta_amp_update(self.ptr, growth_factor, backoff_factor,
                         growth_interval, current_stream())
