"""Fused mixed-precision gradient clip + multi-tensor AdamW for MI355X.

The work runs in libmta.so (HIP, gfx950) behind the C ABI of include/mta.h.
``_binding`` mirrors that ABI name for name; ``MtaList`` marshals PyTorch
tensors and the current HIP stream into it.  Nothing here computes any part
of the step, and nothing falls back to another implementation: if
libmta.so is missing the first call raises.
"""
from ._binding import (  # noqa: F401
    EXPORTS, LIB_PATH, MTA_BF16, MTA_F16, MTA_F32, MTA_MOM_BF16X2,
    MTA_MOM_F32, MTA_OPT_ADAM, MTA_OPT_ADAMW, MTA_OPT_MOMENTUM, MTA_OPT_SGD,
    MTA_SCALE_DEFER, MTA_SCALE_INPLACE, MTA_STEP_ZERO_GRAD, MtaError, lib,
    mta_abi_version, mta_adamw_scalars, mta_adamw_step, mta_amp_adamw_step,
    mta_amp_clip_norm, mta_amp_clip_norm_joint, mta_amp_step, mta_amp_update,
    mta_clip_norm, mta_clip_norm_joint, mta_clip_norm_noalloc,
    mta_last_error, mta_list_create, mta_list_destroy, mta_list_info,
    mta_list_plan, mta_list_set_no_decay, mta_list_set_weight_copies,
    mta_list_set_weight_copies_as, mta_scale, mta_scale_device, mta_step)
from .torch_list import (AmpState, GradClipper, MtaList,  # noqa: F401
                         clip_norm_joint)
from .optim import MtaOptimizer  # noqa: F401
