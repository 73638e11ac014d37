"""ctypes binding of libmta.so: the C ABI of include/mta.h, same names.

Argument marshalling only: every step of the optimizer runs in the HIP
library.  If the library is not built, loading fails loudly; there is no
fallback of any kind.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmta.so")

MTA_F32, MTA_BF16, MTA_F16 = 0, 1, 2
MTA_MOM_F32, MTA_MOM_BF16X2 = 0, 1
MTA_SCALE_INPLACE, MTA_SCALE_DEFER = 1, 2
MTA_OPT_ADAMW, MTA_OPT_ADAM, MTA_OPT_SGD, MTA_OPT_MOMENTUM = 0, 1, 2, 3
OPT_KINDS = {"adamw": MTA_OPT_ADAMW, "adam": MTA_OPT_ADAM,
             "sgd": MTA_OPT_SGD, "momentum": MTA_OPT_MOMENTUM}
MTA_STEP_ZERO_GRAD = 1

MTA_OK = 0
STATUS_NAMES = {0: "MTA_OK", -1: "MTA_EINVAL", -2: "MTA_EALIGN",
                -3: "MTA_EDTYPE", -4: "MTA_ENOMEM", -5: "MTA_EHIP",
                -6: "MTA_ESTATE"}

# MTA_ABI_VERSION of include/mta.h that these structs mirror
ABI_VERSION = 5

# every symbol include/mta.h declares
EXPORTS = ("mta_list_create", "mta_list_destroy", "mta_scale",
           "mta_clip_norm", "mta_adamw_step", "mta_list_set_weight_copies",
           "mta_adamw_scalars", "mta_list_info", "mta_last_error",
           "mta_abi_version", "mta_amp_clip_norm", "mta_amp_adamw_step",
           "mta_amp_update", "mta_step", "mta_amp_step",
           "mta_list_set_weight_copies_as", "mta_list_plan",
           "mta_clip_norm_joint", "mta_amp_clip_norm_joint",
           "mta_list_set_no_decay", "mta_scale_device",
           "mta_clip_norm_noalloc")


class mta_tensor(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("g", ctypes.c_void_p),
                ("m", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("n", ctypes.c_int64)]


class mta_adamw_hparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double),
                ("beta2", ctypes.c_double), ("eps", ctypes.c_double),
                ("weight_decay", ctypes.c_double)]


class mta_opt(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("lr", ctypes.c_double), ("beta1", ctypes.c_double),
                ("beta2", ctypes.c_double), ("eps", ctypes.c_double),
                ("weight_decay", ctypes.c_double),
                ("momentum", ctypes.c_double)]


class mta_amp_state(ctypes.Structure):
    """Host image of the 24-byte device loss-scale state."""
    _fields_ = [("scale", ctypes.c_float), ("found_inf", ctypes.c_float),
                ("growth_tracker", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("step", ctypes.c_int64)]


class mta_list_info_t(ctypes.Structure):
    _fields_ = [("count", ctypes.c_int64), ("elements", ctypes.c_int64),
                ("tiles", ctypes.c_int64), ("tile_elems", ctypes.c_int32),
                ("grid_update", ctypes.c_int32), ("grid_norm", ctypes.c_int32),
                ("device", ctypes.c_int32), ("vector_tensors", ctypes.c_int32),
                ("gtype", ctypes.c_int32), ("mkind", ctypes.c_int32),
                ("vkind", ctypes.c_int32), ("weight_copies", ctypes.c_int32),
                ("state_buffers", ctypes.c_int32),
                ("weight_copy_type", ctypes.c_int32),
                ("norm_kept_tiles", ctypes.c_int32)]


class MtaError(RuntimeError):
    """A libmta call returned a negative mta_status."""

    def __init__(self, code, func, msg):
        self.code = code
        super().__init__(f"{func}: {STATUS_NAMES.get(code, code)}: {msg}")


_lib = None


def lib():
    """The loaded libmta.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built: run `python -m "
                "mixed_precision_optimizer_mta_amd.build` (or "
                "__graft_entry__.build()) first")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, c_int, f32 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                               ctypes.c_float)
        L.mta_list_create.argtypes = [ctypes.POINTER(mta_tensor), i64, c_int,
                                      c_int, c_int, vp,
                                      ctypes.POINTER(vp)]
        L.mta_list_destroy.argtypes = [vp]
        L.mta_scale.argtypes = [vp, f32, c_int, vp]
        L.mta_scale_device.argtypes = [vp, vp, vp]
        L.mta_clip_norm.argtypes = [vp, f32, vp, vp, vp]
        L.mta_clip_norm_joint.argtypes = [ctypes.POINTER(vp), i64, f32, vp,
                                          vp, vp]
        L.mta_amp_clip_norm_joint.argtypes = [ctypes.POINTER(vp), i64, f32,
                                              vp, vp, vp, vp]
        L.mta_adamw_step.argtypes = [vp, ctypes.POINTER(mta_adamw_hparams),
                                     i64, vp, vp]
        L.mta_list_set_weight_copies.argtypes = [vp, ctypes.POINTER(vp), vp]
        L.mta_list_set_weight_copies_as.argtypes = [vp, ctypes.POINTER(vp),
                                                    ctypes.c_int32, vp]
        L.mta_list_set_no_decay.argtypes = [vp, ctypes.POINTER(
            ctypes.c_uint8), vp]
        L.mta_adamw_scalars.argtypes = [ctypes.POINTER(mta_adamw_hparams),
                                        i64, ctypes.POINTER(ctypes.c_float)]
        L.mta_list_info.argtypes = [vp, ctypes.POINTER(mta_list_info_t)]
        L.mta_list_plan.argtypes = [ctypes.POINTER(mta_tensor), i64, c_int,
                                    c_int, c_int,
                                    ctypes.POINTER(mta_list_info_t)]
        L.mta_clip_norm_noalloc.argtypes = [ctypes.POINTER(mta_tensor), i64,
                                            c_int, f32, f32, vp, vp, vp]
        L.mta_amp_clip_norm.argtypes = [vp, f32, vp, vp, vp, vp]
        L.mta_amp_adamw_step.argtypes = [vp,
                                         ctypes.POINTER(mta_adamw_hparams),
                                         vp, vp, vp]
        L.mta_amp_update.argtypes = [vp, ctypes.c_double, ctypes.c_double,
                                     ctypes.c_int32, vp]
        L.mta_step.argtypes = [vp, ctypes.POINTER(mta_opt), i64, vp, vp]
        L.mta_amp_step.argtypes = [vp, ctypes.POINTER(mta_opt), vp, vp, vp]
        L.mta_last_error.argtypes = []
        L.mta_last_error.restype = ctypes.c_char_p
        L.mta_abi_version.argtypes = []
        for name in EXPORTS:
            if name != "mta_last_error":
                getattr(L, name).restype = ctypes.c_int
        if L.mta_abi_version() != ABI_VERSION:
            raise RuntimeError(
                f"{LIB_PATH} has ABI {L.mta_abi_version()}, this binding "
                f"speaks {ABI_VERSION}: rebuild the library")
        _lib = L
    return _lib


def _check(rc, func):
    if rc != MTA_OK:
        raise MtaError(rc, func, mta_last_error())


def mta_last_error():
    return lib().mta_last_error().decode()


def mta_abi_version():
    return lib().mta_abi_version()


def _hparams(hp):
    if isinstance(hp, mta_adamw_hparams):
        return hp
    if isinstance(hp, dict):
        return mta_adamw_hparams(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                                 hp["weight_decay"])
    return mta_adamw_hparams(*hp)


def _tensor_table(tensors):
    arr = (mta_tensor * max(1, len(tensors)))()
    for i, (w, g, m, v, n) in enumerate(tensors):
        arr[i] = mta_tensor(w, g, m, v, n)
    return arr


def mta_list_create(tensors, gtype, mkind, vkind, stream=0):
    """tensors: sequence of (w_ptr, g_ptr, m_ptr, v_ptr, n).  Returns the
    opaque handle (an int)."""
    arr = _tensor_table(tensors)
    out = ctypes.c_void_p()
    rc = lib().mta_list_create(arr, len(tensors), gtype, mkind, vkind,
                               stream, ctypes.byref(out))
    _check(rc, "mta_list_create")
    return out.value


def mta_list_destroy(handle):
    _check(lib().mta_list_destroy(handle), "mta_list_destroy")


def mta_scale(handle, factor, flags, stream=0):
    _check(lib().mta_scale(handle, factor, flags, stream), "mta_scale")


def mta_scale_device(handle, d_factor, stream=0):
    """g = g * (*d_factor) in place; d_factor a device pointer."""
    _check(lib().mta_scale_device(handle, d_factor, stream),
           "mta_scale_device")


def mta_clip_norm(handle, max_norm, d_norm, d_coef, stream=0):
    _check(lib().mta_clip_norm(handle, max_norm, d_norm, d_coef, stream),
           "mta_clip_norm")


def mta_clip_norm_noalloc(tensors, gtype, scale, max_norm, d_norm, d_coef,
                          stream=0):
    """The allocation-free norm: tensors as for mta_list_create (only g is
    read); d_norm (or None) and d_coef device pointers."""
    arr = _tensor_table(tensors)
    _check(lib().mta_clip_norm_noalloc(arr, len(tensors), gtype, scale,
                                       max_norm, d_norm, d_coef, stream),
           "mta_clip_norm_noalloc")


def _handles(handles):
    return (ctypes.c_void_p * max(1, len(handles)))(*handles)


def mta_clip_norm_joint(handles, max_norm, d_norm, d_coef, stream=0):
    """handles: list handles in the order their norms are summed."""
    _check(lib().mta_clip_norm_joint(_handles(handles), len(handles),
                                     max_norm, d_norm, d_coef, stream),
           "mta_clip_norm_joint")


def mta_adamw_step(handle, hp, t, d_coef, stream=0):
    h = _hparams(hp)
    _check(lib().mta_adamw_step(handle, ctypes.byref(h), t, d_coef, stream),
           "mta_adamw_step")


def _copy_array(w16):
    if w16 is None:
        return None
    return (ctypes.c_void_p * max(1, len(w16)))(*[p or None for p in w16])


def mta_list_set_weight_copies(handle, w16, stream=0):
    """w16: one device pointer (or None) per tensor of the list, or None to
    detach every copy."""
    _check(lib().mta_list_set_weight_copies(handle, _copy_array(w16), stream),
           "mta_list_set_weight_copies")


def mta_list_set_weight_copies_as(handle, w16, copy_type, stream=0):
    """As mta_list_set_weight_copies; copy_type MTA_BF16 or MTA_F16."""
    _check(lib().mta_list_set_weight_copies_as(handle, _copy_array(w16),
                                               copy_type, stream),
           "mta_list_set_weight_copies_as")


def mta_list_set_no_decay(handle, no_decay, stream=0):
    """no_decay: one truth value per tensor of the list (True: the tensor
    takes weight_decay = 0), or None to clear every flag."""
    arr = None
    if no_decay is not None and handle:
        count = mta_list_info(handle)["count"]
        if len(no_decay) != count:
            raise ValueError(f"no_decay has {len(no_decay)} entries, the "
                             f"list {count} tensors")
        arr = (ctypes.c_uint8 * max(1, count))(
            *[1 if f else 0 for f in no_decay])
    _check(lib().mta_list_set_no_decay(handle, arr, stream),
           "mta_list_set_no_decay")


def mta_adamw_scalars(hp, t):
    h = _hparams(hp)
    out = (ctypes.c_float * 7)()
    _check(lib().mta_adamw_scalars(ctypes.byref(h), t, out),
           "mta_adamw_scalars")
    return [out[i] for i in range(7)]


def mta_list_info(handle):
    info = mta_list_info_t()
    _check(lib().mta_list_info(handle, ctypes.byref(info)), "mta_list_info")
    return {name: getattr(info, name) for name, _ in mta_list_info_t._fields_}


def mta_list_plan(tensors, gtype, mkind, vkind):
    """The shape mta_list_create would give these (w, g, m, v, n) entries
    (pointers as ints, m / v may be None); no device is touched."""
    info = mta_list_info_t()
    _check(lib().mta_list_plan(_tensor_table(tensors), len(tensors), gtype,
                               mkind, vkind, ctypes.byref(info)),
           "mta_list_plan")
    return {name: getattr(info, name) for name, _ in mta_list_info_t._fields_}


def mta_amp_clip_norm(handle, max_norm, d_amp, d_norm, d_coef, stream=0):
    _check(lib().mta_amp_clip_norm(handle, max_norm, d_amp, d_norm, d_coef,
                                   stream), "mta_amp_clip_norm")


def mta_amp_clip_norm_joint(handles, max_norm, d_amp, d_norm, d_coef,
                            stream=0):
    _check(lib().mta_amp_clip_norm_joint(_handles(handles), len(handles),
                                         max_norm, d_amp, d_norm, d_coef,
                                         stream), "mta_amp_clip_norm_joint")


def mta_amp_adamw_step(handle, hp, d_amp, d_coef, stream=0):
    h = _hparams(hp)
    _check(lib().mta_amp_adamw_step(handle, ctypes.byref(h), d_amp, d_coef,
                                    stream), "mta_amp_adamw_step")


def mta_amp_update(d_amp, growth_factor, backoff_factor, growth_interval,
                   stream=0):
    _check(lib().mta_amp_update(d_amp, growth_factor, backoff_factor,
                                growth_interval, stream), "mta_amp_update")


def _opt(opt):
    """An mta_opt from a dict: kind ("adamw", "adam", "sgd", "momentum" or
    the enum value), lr, and the fields the rule reads; zero_grad (bool)."""
    if isinstance(opt, mta_opt):
        return opt
    kind = opt["kind"]
    kind = OPT_KINDS[kind] if isinstance(kind, str) else int(kind)
    flags = MTA_STEP_ZERO_GRAD if opt.get("zero_grad") else 0
    return mta_opt(kind, flags, opt.get("lr", 0.0), opt.get("beta1", 0.0),
                   opt.get("beta2", 0.0), opt.get("eps", 0.0),
                   opt.get("weight_decay", 0.0), opt.get("momentum", 0.0))


def mta_step(handle, opt, t, d_coef, stream=0):
    o = _opt(opt)
    _check(lib().mta_step(handle, ctypes.byref(o), t, d_coef, stream),
           "mta_step")


def mta_amp_step(handle, opt, d_amp, d_coef, stream=0):
    o = _opt(opt)
    _check(lib().mta_amp_step(handle, ctypes.byref(o), d_amp, d_coef, stream),
           "mta_amp_step")
