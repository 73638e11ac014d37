"""C-ABI checks that need no GPU: the library loads, exports every function
include/mta.h declares, validates arguments before touching the device, and
prepares the step's float32 constants exactly as the oracle does."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
import mixed_precision_optimizer_mta_amd as M
from mixed_precision_optimizer_mta_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mta.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mta_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 9
    lib = ctypes.CDLL(B.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name
    assert sorted(B.EXPORTS) == names


def test_abi_version():
    assert M.mta_abi_version() == 5 == B.ABI_VERSION
    # the binding's mirror of mta_list_info_t has the header's size
    assert ctypes.sizeof(B.mta_list_info_t) == 72


def _err(fn, *a):
    with pytest.raises(M.MtaError) as e:
        fn(*a)
    return e.value.code


def test_create_rejects_bad_arguments_before_device_work():
    ok = (0x10000, 0x20000, 0x30000, 0x40000, 64)
    assert _err(M.mta_list_create, [ok], 3, 0, 0) == -3            # gtype
    assert _err(M.mta_list_create, [ok], 0, 5, 0) == -3            # mkind
    assert _err(M.mta_list_create, [ok], 0, 0, -1) == -3           # vkind
    assert _err(M.mta_list_create, [(0x10000, 0, 0x30000, 0x40000, 64)],
                0, 0, 0) == -1                                      # NULL g
    assert _err(M.mta_list_create, [(0x10000, 0x20000, 0x30000, 0x40000,
                                      -1)], 0, 0, 0) == -1          # n < 0
    assert _err(M.mta_list_create, [(0x10002, 0x20000, 0x30000, 0x40000,
                                      64)], 0, 0, 0) == -2          # w align
    assert _err(M.mta_list_create, [(0x10000, 0x20001, 0x30000, 0x40000,
                                      64)], 1, 0, 0) == -2          # bf16 g
    assert _err(M.mta_list_create, [(0x10000, 0x20001, 0x30000, 0x40000,
                                      64)], 2, 0, 0) == -2          # f16 g
    # packed moments need only 2-byte alignment; f32 ones 4
    assert _err(M.mta_list_create, [(0x10000, 0x20000, 0x30002, 0x40000,
                                      64)], 0, 0, 0) == -2
    # overlap inside a tensor and across tensors
    assert _err(M.mta_list_create, [(0x10000, 0x10010, 0x30000, 0x40000,
                                      64)], 0, 0, 0) == -1
    assert _err(M.mta_list_create, [ok, (0x10080, 0x50000, 0x60000,
                                         0x70000, 8)], 0, 0, 0) == -1
    assert "overlap" in M.mta_last_error()


def test_adjacent_buffers_are_not_overlap_and_empty_tensors_skip_checks():
    # w of 64 float32 ends exactly where g starts: allowed.  Without a GPU
    # the call then fails at the device step, not at validation.
    ents = [(0x10000, 0x10100, 0x10200, 0x10300, 64), (0, 0, 0, 0, 0)]
    try:
        h = M.mta_list_create(ents, 0, 0, 0)
    except M.MtaError as e:
        assert e.code == -5, e            # no device here
    else:                                   # a GPU is present
        M.mta_list_destroy(h)


def test_calls_on_a_null_handle_fail_cleanly():
    assert _err(M.mta_clip_norm, None, 1.0, None, 0x1000) == -1
    assert _err(M.mta_adamw_step, None, (1e-3, .9, .999, 1e-8, 0.), 1,
                None) == -1
    assert _err(M.mta_scale, None, 0.5, M.MTA_SCALE_DEFER) == -1
    assert _err(M.mta_amp_clip_norm, None, 1.0, 0x1000, None, 0x2000) == -1
    assert _err(M.mta_amp_adamw_step, None, (1e-3, .9, .999, 1e-8, 0.),
                0x1000, None) == -1
    assert _err(M.mta_list_set_no_decay, None, [True, False]) == -1
    assert _err(M.mta_list_set_no_decay, None, None) == -1
    assert _err(M.mta_scale_device, None, 0x1000) == -1
    assert _err(M.mta_list_set_weight_copies, None, None) == -1
    M.mta_list_destroy(None)


@pytest.mark.parametrize("args,code", [
    ((None, 2.0, 0.5, 2000), -1),            # NULL state
    ((0x1004, 2.0, 0.5, 2000), -2),          # state not 8-byte aligned
    ((0x1000, 1.0, 0.5, 2000), -1),          # growth must be > 1
    ((0x1000, float("inf"), 0.5, 2000), -1),
    ((0x1000, 2.0, 1.0, 2000), -1),          # backoff must be < 1
    ((0x1000, 2.0, 0.0, 2000), -1),          # and > 0
    ((0x1000, 2.0, 0.5, 0), -1),             # interval >= 1
])
def test_amp_update_validation(args, code):
    # every case fails in validation, before any device work
    assert _err(M.mta_amp_update, *args) == code


def test_amp_state_layout():
    assert ctypes.sizeof(B.mta_amp_state) == 24
    assert B.mta_amp_state.step.offset == 16


@pytest.mark.parametrize("hp,t", [
    ((1e-3, 1.0, 0.999, 1e-8, 0.0), 1),      # beta1 = 1
    ((1e-3, 0.9, -0.1, 1e-8, 0.0), 1),       # beta2 < 0
    ((-1e-3, 0.9, 0.999, 1e-8, 0.0), 1),     # lr < 0
    ((float("nan"), 0.9, 0.999, 1e-8, 0.0), 1),
    ((1e-3, 0.9, 0.999, -1e-8, 0.0), 1),     # eps < 0
    ((1e-3, 0.9, 0.999, 1e-8, -0.1), 1),     # wd < 0
    ((1e-3, 0.9, 0.999, 1e-8, 0.1), 0),      # t = 0
])
def test_hparams_validation(hp, t):
    assert _err(M.mta_adamw_scalars, hp, t) == -1


@pytest.mark.parametrize("hp", [(3e-4, 0.9, 0.999, 1e-8, 0.1),
                                (3e-4, 0.9, 0.999, 1e-8, 0.01),
                                (1e-2, 0.5, 0.75, 0.5, 0.5),
                                (6e-4, 0.95, 0.98, 1e-6, 0.0),
                                (1.0, 0.0, 0.0, 0.0, 0.0)])
def test_scalars_match_the_oracle_bitwise(hp):
    for t in list(range(1, 60)) + [100, 1000, 4567, 10 ** 6]:
        got = np.array(M.mta_adamw_scalars(hp, t), dtype=np.float32)
        want = O.scalars(*hp, t)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (
            hp, t, got, want)


@pytest.mark.parametrize("opt,t,msg", [
    (dict(kind=7, lr=1e-3), 1, "unknown optimizer kind"),
    (dict(kind="sgd", lr=1e-3, weight_decay=0.1), 1, "no weight decay"),
    (dict(kind="momentum", lr=1e-3, weight_decay=0.1), 1, "no weight decay"),
    (dict(kind="momentum", lr=1e-3, momentum=-0.5), 1, "momentum"),
    (dict(kind="momentum", lr=1e-3, momentum=float("nan")), 1, "momentum"),
    (dict(kind="sgd", lr=-1.0), 1, "lr"),
    (dict(kind="sgd", lr=float("inf")), 1, "lr"),
    (dict(kind="sgd", lr=1e-3), 0, "step t"),
    (dict(kind="adam", lr=1e-3, beta1=1.0, beta2=0.999), 1, "beta1"),
    (dict(kind="adamw", lr=1e-3, beta1=0.9, beta2=0.999, eps=-1.0), 1,
     "eps"),
])
def test_step_validation_before_any_device_work(opt, t, msg):
    # the optimizer is checked before the list: these fail on a NULL list
    # with the optimizer's message
    assert _err(M.mta_step, None, opt, t, None) == -1
    assert msg in M.mta_last_error(), M.mta_last_error()


def test_step_rejects_unknown_flags():
    o = B.mta_opt(B.MTA_OPT_SGD, 0x10, 1e-3, 0, 0, 0, 0, 0)
    assert _err(M.mta_step, None, o, 1, None) == -1
    assert "flags" in M.mta_last_error()


def test_opt_struct_layout():
    assert ctypes.sizeof(B.mta_opt) == 56
    assert B.mta_opt.lr.offset == 8 and B.mta_opt.momentum.offset == 48


def test_last_error_is_per_host_thread():
    # each thread's failing call leaves its own message; another thread's
    # failure does not overwrite it
    import threading
    barrier = threading.Barrier(8)
    results = {}

    def worker(k):
        barrier.wait()
        lr = -1.0 - k            # a distinct invalid lr per thread
        try:
            M.mta_adamw_scalars((lr, 0.9, 0.999, 1e-8, 0.0), 1)
        except M.MtaError:
            pass
        barrier.wait()           # every thread has failed by now
        results[k] = M.mta_last_error()

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    for k in range(8):
        assert f"(got {-1.0 - k:g})" in results[k], (k, results[k])


def test_success_clears_the_last_error():
    with pytest.raises(M.MtaError):
        M.mta_adamw_scalars((-1.0, 0.9, 0.999, 1e-8, 0.0), 1)
    assert M.mta_last_error() != ""
    M.mta_adamw_scalars((1e-3, 0.9, 0.999, 1e-8, 0.0), 1)
    assert M.mta_last_error() == ""


def test_joint_norm_validation_before_any_device_work():
    assert _err(M.mta_clip_norm_joint, [], 1.0, None, 0x1000) == -1
    assert _err(M.mta_clip_norm_joint, [None], 1.0, None, 0x1000) == -1
    assert _err(M.mta_clip_norm_joint, [None, None], 1.0, None,
                0x1000) == -1
    assert _err(M.mta_clip_norm_joint, [None], 0.0, None, 0x1000) == -1
    assert _err(M.mta_clip_norm_joint, [None], 1.0, None, None) == -1
    assert _err(M.mta_clip_norm_joint, [None], 1.0, None, 0x1002) == -2
    assert _err(M.mta_amp_clip_norm_joint, [None], 1.0, None, None,
                0x1000) == -1
    assert _err(M.mta_amp_clip_norm_joint, [None], 1.0, 0x1004, None,
                0x1000) == -2
