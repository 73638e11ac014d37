"""MtaList: a libmta tensor-list handle over PyTorch tensors.

Marshalling only.  It checks that the tensors are what the C ABI expects
(device, dtype, contiguity, element counts), passes their data pointers and
the current HIP stream, and owns the handle.  The tensors must keep their
storage for the handle's life (the library holds their addresses).
"""
import torch

from . import _binding as B

_G = {torch.float32: B.MTA_F32, torch.bfloat16: B.MTA_BF16}
_M = {torch.float32: B.MTA_MOM_F32, torch.bfloat16: B.MTA_MOM_BF16X2}


def current_stream():
    return torch.cuda.current_stream().cuda_stream


class MtaList:
    """groups: sequence of (w, g, m, v) tensors.  w is float32; g float32 or
    bfloat16; m and v float32 or bfloat16 (bfloat16 = packed moments); all
    groups share the gradient type and each moment kind."""

    def __init__(self, groups, entries=None, gtype=None, mkind=None,
                 vkind=None):
        self._keep = list(groups)
        if entries is None:
            if not self._keep:
                raise ValueError("empty list: pass gtype/mkind/vkind and "
                                 "entries=[] explicitly")
            g0, m0, v0 = self._keep[0][1], self._keep[0][2], self._keep[0][3]
            gtype, mkind, vkind = _G[g0.dtype], _M[m0.dtype], _M[v0.dtype]
            entries = []
            for w, g, m, v in self._keep:
                for t in (w, g, m, v):
                    if not t.is_cuda or not t.is_contiguous():
                        raise ValueError("tensors must be contiguous on the GPU")
                if w.dtype != torch.float32:
                    raise TypeError("w must be float32")
                if (_G.get(g.dtype), _M.get(m.dtype), _M.get(v.dtype)) != (
                        gtype, mkind, vkind):
                    raise TypeError("all groups must share g, m, v dtypes")
                n = w.numel()
                if g.numel() != n or m.numel() != n or v.numel() != n:
                    raise ValueError("w, g, m, v must have the same numel")
                entries.append((w.data_ptr(), g.data_ptr(), m.data_ptr(),
                                v.data_ptr(), n))
        self.gtype, self.mkind, self.vkind = gtype, mkind, vkind
        self.sizes = [int(e[4]) for e in entries]
        self.handle = B.mta_list_create(entries, gtype, mkind, vkind,
                                        current_stream())

    def info(self):
        return B.mta_list_info(self.handle)

    def scale(self, factor, defer=True):
        B.mta_scale(self.handle, factor,
                    B.MTA_SCALE_DEFER if defer else B.MTA_SCALE_INPLACE,
                    current_stream())

    def clip_norm(self, max_norm, norm_out, coef_out):
        """norm_out (may be None) and coef_out: float32 device tensors."""
        for t in (norm_out, coef_out):
            if t is not None and (t.dtype != torch.float32 or not t.is_cuda):
                raise TypeError("norm/coef outputs are float32 GPU tensors")
        B.mta_clip_norm(self.handle, max_norm,
                        None if norm_out is None else norm_out.data_ptr(),
                        coef_out.data_ptr(), current_stream())

    def set_weight_copies(self, copies):
        """copies: one bfloat16 GPU tensor (or None) per group, each with the
        weight's numel, written with bfloat16(w) by every later AdamW step;
        None detaches them all."""
        ptrs = None
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
                if c.dtype != torch.bfloat16 or not c.is_cuda or \
                        not c.is_contiguous():
                    raise TypeError("weight copies are contiguous bfloat16 "
                                    "GPU tensors")
                ptrs.append(c.data_ptr())
            self._copies = list(copies)
        B.mta_list_set_weight_copies(self.handle, ptrs, current_stream())

    def adamw_step(self, hparams, t, coef=None):
        if coef is not None and (coef.dtype != torch.float32 or
                                 not coef.is_cuda):
            raise TypeError("coef is a float32 GPU tensor")
        B.mta_adamw_step(self.handle, hparams, t,
                         None if coef is None else coef.data_ptr(),
                         current_stream())

    def close(self):
        if self.handle is not None:
            B.mta_list_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
