"""Benchmark of the fused clip + multi-tensor AdamW step on one MI355X.

One step = mta_clip_norm (joint norm + clip coefficient, one launch) and
mta_adamw_step (AdamW over every tensor, one launch), plus the deferred
unscale where the workload has one (no launch), over inputs resident in HBM.
A loss-scaled workload runs mta_amp_clip_norm, mta_amp_adamw_step and
mta_amp_update (a one-thread launch) instead.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

The default workload is gpt2_xl, the 1.56B-parameter list with packed
bfloat16 moments: the largest of the workloads, and one that fits one GPU.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published
KERNEL_SRC = os.path.join(ROOT, "mixed_precision_optimizer_mta_amd", "csrc",
                          "mta_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_sha():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter runs, or
    None when there are none for this workload or the kernel source changed
    since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    rec = data.get(workload, {}).get(kernel)
    if not rec or rec.get("kernel_source_sha") != kernel_source_sha():
        return None
    return rec.get("bytes_per_launch")


# --no-decay flags tensors below this many elements: in the GPT-2 layouts
# exactly the biases and layer-norm gains (the largest, 6400, in gpt2_xl),
# none of the weight matrices or embeddings (the smallest, 589,824)
NO_DECAY_BELOW = 1 << 14

KERNEL_OF = {"adamw": "k_adamw", "adam": "k_adamw", "sgd": "k_sgd",
             "momentum": "k_momentum"}


def opt_of(wl, kind, zero):
    """The update rule's configuration for a workload (SGD and momentum take
    the workload's lr, no weight decay, momentum 0.9)."""
    adam = kind in ("adamw", "adam")
    return dict(kind=kind, lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2,
                eps=wl.eps, weight_decay=wl.weight_decay if adam else 0.0,
                momentum=0.9, zero_grad=zero)


def traffic_key(wl, kind, zero):
    """The key of a configuration in profiles/traffic.json."""
    if kind == "adamw" and not zero:
        return wl.name
    return f"{wl.name}+{kind}" + ("+zero" if zero else "")


def update_bytes(wl, kind, zero, copy):
    """Algorithmic HBM bytes per parameter of one update launch."""
    gb = 4 if wl.gtype == 0 else 2
    mb = 2 if wl.mkind == 1 else 4
    vb = 2 if wl.vkind == 1 else 4
    b = {"adamw": wl.bytes_per_param()["update"],
         "adam": wl.bytes_per_param()["update"],
         "sgd": 4 + gb + 4,                       # read w, g; write w
         "momentum": 4 + gb + mb + 4 + mb}[kind]  # + read/write buf
    return b + (gb if zero else 0) + (2 if copy else 0)


PROBE_LIB = os.path.join(ROOT, "bench_probes", "libmta_probe.so")


def independent_ceiling(wl, reps=5):
    """HBM rates of AMD- and PyTorch-owned kernels (none of this library's
    code) on float32 buffers of the workload's parameter count, on the same
    GPU: torch's fill_ (write only), Tensor.copy_ (a hipMemcpy device to
    device), torch.add(a, b, out=c) (2 reads : 1 write) and
    torch.addcmul(a, b, c, out=d) (3 : 1).  Best of `reps` launches after
    two warm-ups, algorithmic bytes / event time."""
    import torch
    n = wl.n
    bufs = [torch.ones(n, device="cuda") for _ in range(4)]
    a, b, c, d = bufs
    s = torch.cuda.current_stream()

    def best(fn, nbytes):
        for _ in range(2):
            fn()
        out = 0.0
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s)
            fn()
            e1.record(s)
            torch.cuda.synchronize()
            out = max(out, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        return out

    res = {
        "fill_gbs": best(lambda: d.fill_(0.5), 4 * n),
        "copy_gbs": best(lambda: d.copy_(a), 8 * n),
        "add_gbs": best(lambda: torch.add(a, b, out=d), 12 * n),
        "addcmul_gbs": best(lambda: torch.addcmul(a, b, c, out=d), 16 * n),
    }
    del bufs, a, b, c, d
    torch.cuda.empty_cache()
    out = {"kernels": "torch " + torch.__version__ + ": fill_, copy_ "
                      "(hipMemcpy device to device), add(out=), "
                      "addcmul(out=); float32 buffers of the workload's "
                      "parameter count; best of %d launches" % reps}
    for k, v in res.items():
        out[k] = v
        out[k.replace("_gbs", "_frac")] = v / HBM_PEAK_GBS
    return out


def probe_ceiling(wl, reps=10):
    """Best HBM rates of this project's ceiling probes
    (bench_probes/libmta_probe.so: no optimizer arithmetic) on buffers of
    the workload's size: a stream with the update's exact bytes (read w, g,
    m, v; write w, m, v), a read-only stream, a write-only stream and a
    copy, each over grids of 1, 2, 4 and 8 workgroups per CU (the
    write-only one also over half the CUs).  These share the update's lane
    mapping, so they bound that design, not the device."""
    import ctypes

    import torch

    if not os.path.exists(PROBE_LIB):
        raise SystemExit(f"{PROBE_LIB} is not built: python "
                         "bench_probes/build.py")
    P = ctypes.CDLL(PROBE_LIB)
    vp, i64, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    P.mta_probe_mix.argtypes = [vp, vp, vp, vp, i64, c_int, c_int, c_int,
                                c_int, vp]
    P.mta_probe_read.argtypes = [vp, i64, vp, c_int, vp]
    P.mta_probe_copy.argtypes = [vp, vp, i64, c_int, vp]
    P.mta_probe_write.argtypes = [vp, i64, c_int, vp]
    n = -(-wl.n // 4096) * 4096
    gb = 4 if wl.gtype == 0 else 2
    mb = 2 if wl.mkind == 1 else 4
    vb = 2 if wl.vkind == 1 else 4

    def buf(b):
        return torch.zeros(n, device="cuda",
                           dtype=torch.float32 if b == 4 else torch.int16)

    w, g, m, v = buf(4), buf(gb), buf(mb), buf(vb)
    w2 = buf(4)
    sink = torch.zeros(256, device="cuda")
    s = torch.cuda.current_stream()
    cus = torch.cuda.get_device_properties(0).multi_processor_count

    def best(launch, nbytes, per_cu=(1, 2, 4, 8)):
        out = (0.0, 0)
        for bpc in per_cu:
            grid = max(1, int(cus * bpc))
            for _ in range(2):
                assert launch(grid) == 0
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(s)
            for _ in range(reps):
                launch(grid)
            b.record(s)
            torch.cuda.synchronize()
            gbs = nbytes / (a.elapsed_time(b) / reps * 1e-3) / 1e9
            out = max(out, (gbs, bpc))
        return out

    sp = s.cuda_stream
    mix = best(lambda gr: P.mta_probe_mix(w.data_ptr(), g.data_ptr(),
                                          m.data_ptr(), v.data_ptr(), n, gb,
                                          mb, vb, gr, sp),
               n * (4 + gb + mb + vb + 4 + mb + vb))
    rd = best(lambda gr: P.mta_probe_read(w.data_ptr(), n, sink.data_ptr(),
                                          gr, sp), n * 4)
    cp = best(lambda gr: P.mta_probe_copy(w.data_ptr(), w2.data_ptr(), n, gr,
                                          sp), n * 8)
    wr = best(lambda gr: P.mta_probe_write(w2.data_ptr(), n, gr, sp), n * 4,
              per_cu=(0.5, 1, 2, 4))
    rbytes, wbytes = 4 + gb + mb + vb, 4 + mb + vb
    serial = (rbytes + wbytes) / (rbytes / rd[0] + wbytes / wr[0])
    return {"probe": "bench_probes/libmta_probe.so, trivial arithmetic, "
                     "best of 1/2/4/8 workgroups per CU",
            "update_mix_gbs": mix[0], "update_mix_frac": mix[0] / HBM_PEAK_GBS,
            "update_mix_blocks_per_cu": mix[1],
            "read_gbs": rd[0], "read_frac": rd[0] / HBM_PEAK_GBS,
            "copy_gbs": cp[0], "copy_frac": cp[0] / HBM_PEAK_GBS,
            "write_gbs": wr[0], "write_frac": wr[0] / HBM_PEAK_GBS,
            "write_blocks_per_cu": wr[1],
            "serial_bound_gbs": serial,
            "serial_bound_frac": serial / HBM_PEAK_GBS}


def cpu_model():
    """The host CPU as /proc/cpuinfo names it: model name, family, model
    and stepping (the latter three identify the generation when a virtual
    machine shortens the name), and the logical CPUs this process may use
    against those the machine shows."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break                  # the first processor is enough
                k, _, v = line.partition(":")
                info[k.strip()] = v.strip()
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return (f"{info.get('model name', 'unknown')} (family "
            f"{info.get('cpu family', '?')}, model {info.get('model', '?')}, "
            f"stepping {info.get('stepping', '?')}); {usable} of "
            f"{os.cpu_count()} logical CPUs usable")


def cpu_baseline_parallel(arena, wl, steps, threads):
    """The same oracle functions, unchanged, run by `threads` host threads
    over disjoint element ranges of the list (AdamW, deferred unscale, joint
    clip): each thread's float64 sum-of-squares state for its ranges, the
    states summed in thread order, then every thread's AdamW on its ranges.
    Plain AdamW workloads only."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch

    import oracle as O

    def host(t, bits16):
        t = t.detach().cpu()
        if bits16:
            return t.view(torch.int16).numpy().view(np.uint16).copy()
        return t.numpy().copy()

    chunk = max(4096, (wl.n // (threads * 8)) // 2 * 2)  # even: packed words
    parts = []
    for i in range(wl.count):
        n = wl.sizes[i]
        if n == 0:
            continue
        w = host(arena.view("w", i), False)
        g = host(arena.view("g", i), wl.gtype != 0)
        m = host(arena.view("m", i), wl.mkind == 1)
        v = host(arena.view("v", i), wl.vkind == 1)
        m = O.pack_halves(m) if wl.mkind == 1 else m
        v = O.pack_halves(v) if wl.vkind == 1 else v
        for a in range(0, n, chunk):
            b = min(n, a + chunk)
            mm = m[a // 2:(b + 1) // 2] if wl.mkind == 1 else m[a:b]
            vv = v[a // 2:(b + 1) // 2] if wl.vkind == 1 else v[a:b]
            parts.append(O.Tensor(w[a:b], g[a:b], mm, vv))
    groups = [parts[k::threads] for k in range(threads)]
    O.lib()
    pool = ThreadPoolExecutor(threads)
    t0 = time.perf_counter()
    for t in range(1, steps + 1):
        sums = list(pool.map(
            lambda grp: O.sumsq([x.g for x in grp], wl.gtype, wl.scale),
            groups))
        nrm = float(np.sqrt(sum(sums)))
        c = O.clip_coef(wl.max_norm, np.float32(nrm))
        sc = O.scalars(wl.lr, wl.beta1, wl.beta2, wl.eps, wl.weight_decay, t)

        def update(grp):
            for x in grp:
                O.adamw_(x.w, x.g, x.m, x.v, wl.gtype, wl.mkind, wl.vkind,
                         sc, wl.scale, c)
        list(pool.map(update, groups))
    dt = time.perf_counter() - t0
    pool.shutdown()
    return {"value": wl.n * steps / dt, "unit": "params/s", "cores": threads,
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"{steps} whole steps of the full {wl.n:,}-param "
                      f"list, the oracle's own functions over disjoint "
                      f"ranges of {chunk:,} elements on {threads} host "
                      f"threads, {dt:.2f} s"}


def torch_reference(arena, wl, steps=100, warmup=10):
    """PyTorch's own step on the same tensors, for context: every tensor a
    torch Parameter over its slice of the arena (its gradient the slice of
    g), then torch.nn.utils.clip_grad_norm_ + torch.optim.AdamW(fused=True)
    with the workload's hyperparameters (PyTorch keeps float32 moments of
    its own).  Device time per step from HIP events over `steps` steps.
    Float32 gradients only (PyTorch needs the parameter's dtype)."""
    import torch
    ps = []
    for i, n in enumerate(wl.sizes):
        if n:
            p = torch.nn.Parameter(arena.view("w", i))
            p.grad = arena.view("g", i)
            ps.append(p)
    opt = torch.optim.AdamW(ps, lr=wl.lr, betas=(wl.beta1, wl.beta2),
                            eps=wl.eps, weight_decay=wl.weight_decay,
                            fused=True)

    def step():
        torch.nn.utils.clip_grad_norm_(ps, wl.max_norm)
        opt.step()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        step()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    return {"kind": "torch.nn.utils.clip_grad_norm_ + "
                    "torch.optim.AdamW(fused=True), float32 moments",
            "torch": torch.__version__, "steps": steps, "ms_per_step": ms,
            "params_per_s": wl.n / (ms * 1e-3)}


def cpu_baseline(arena, wl, steps, opt=None):
    """The oracle as it stands (single thread) on host copies of the same
    list: `steps` whole steps (norm + update), or, with steps None, as many
    as cpu_steps_after() picks from the first step's time."""
    import numpy as np
    import torch

    import oracle as O

    def host(t, bits16):
        t = t.detach().cpu()
        if bits16:
            return t.view(torch.int16).numpy().view(np.uint16).copy()
        return t.numpy().copy()

    ts = []
    for i in range(wl.count):
        m = host(arena.view("m", i), wl.mkind == 1)
        v = host(arena.view("v", i), wl.vkind == 1)
        ts.append(O.Tensor(host(arena.view("w", i), False),
                           host(arena.view("g", i), wl.gtype != 0),
                           O.pack_halves(m) if wl.mkind == 1 else m,
                           O.pack_halves(v) if wl.vkind == 1 else v))
    O.lib()
    amp = O.AmpState(wl.amp_scale) if wl.amp else None
    general = opt is not None and (opt["kind"] != "adamw" or
                                   opt["zero_grad"])
    zero = bool(opt and opt["zero_grad"])
    t0 = time.perf_counter()
    t = 0
    while steps is None or t < steps:
        t += 1
        if general and amp is not None:
            O.amp_opt_step_(ts, opt, wl.gtype, wl.mkind, wl.vkind, amp,
                            wl.max_norm, zero=zero)
            amp.update(wl.amp_growth, wl.amp_backoff, wl.amp_interval)
        elif general:
            O.opt_step_(ts, opt, wl.gtype, wl.mkind, wl.vkind, t,
                        s=wl.scale, max_norm=wl.max_norm, zero=zero)
        elif amp is not None:
            O.amp_step_(ts, wl.gtype, wl.mkind, wl.vkind, amp, wl.lr,
                        wl.beta1, wl.beta2, wl.eps, wl.weight_decay,
                        wl.max_norm)
            amp.update(wl.amp_growth, wl.amp_backoff, wl.amp_interval)
        else:
            O.step_(ts, wl.gtype, wl.mkind, wl.vkind, wl.lr, wl.beta1,
                    wl.beta2, wl.eps, wl.weight_decay, t, s=wl.scale,
                    max_norm=wl.max_norm)
        if steps is None:
            steps = cpu_steps_after(time.perf_counter() - t0)
    dt = time.perf_counter() - t0
    return {"value": wl.n * steps / dt, "unit": "params/s", "cores": 1,
            "kind": "oracle", "cpu": cpu_model(), "steps": steps,
            "sample": f"{steps} whole steps (joint norm + clip + "
                      f"{opt['kind'] if opt else 'adamw'} update"
                      f"{' + loss-scale update' if amp else ''}) of "
                      f"the full {wl.n:,}-param list, one host thread, "
                      f"{dt:.2f} s"}


def cpu_steps_after(first_s, target_s=20.0):
    """Whole oracle steps of the CPU baseline by default, given the first
    step's time: about target_s of one host core in all, at least 1 (the
    step already taken), at most 60.  The oracle's rate depends on the
    list's kinds (packed 16-bit moments cost it about 3x per parameter), so
    the count is taken from the list itself rather than from its size."""
    return max(1, min(60, round(target_s / max(first_s, 1e-9))))


def make_parser():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="gpt2_xl",
                    help="default gpt2_xl: the 1.56B-parameter list, the "
                         "largest workload that fits one GPU")
    ap.add_argument("--layout", default="padded", choices=["padded", "flat"],
                    help="padded: every tensor starts 16-byte aligned in "
                         "each buffer; flat: tensors back to back in one "
                         "buffer per kind, as a flat parameter / gradient "
                         "buffer holds them (a tensor may start anywhere)")
    ap.add_argument("--cpu-steps", type=int, default=None,
                    help="oracle steps of the CPU baseline (0 = skip); by "
                         "default as many whole steps as take about 20 s "
                         "of one host core, counted from the first step's "
                         "time (1 on the 1.56B packed list, about 55 on "
                         "the 124M one), at least 1")
    ap.add_argument("--weight-copy", nargs="?", const="bf16", default=None,
                    choices=["bf16", "f16"],
                    help="also write a 16-bit copy (bfloat16 by default, or "
                         "float16) of every updated weight "
                         "(mta_list_set_weight_copies_as): +2 B/param")
    ap.add_argument("--scale-inplace", action="store_true",
                    help="workloads with an unscale factor s (not loss-"
                         "scaled): apply it with an in-place mta_scale "
                         "launch (k_scale: reads and writes g) instead of "
                         "deferring it into the norm and the update; the "
                         "factor alternates s, 1/s from step to step so "
                         "the gradients keep their values (s is a power of "
                         "two)")
    ap.add_argument("--joint-norm", type=int, default=1, metavar="K",
                    help="clip over the joint norm of K lists (the tensors "
                         "cut into K runs of consecutive tensors, norms "
                         "chained by mta_clip_norm_joint) instead of one; "
                         "the update stays one list")
    ap.add_argument("--no-decay", action="store_true",
                    help="flag the tensors of under 2^14 elements (in the "
                         "GPT-2 layouts: the biases and layer-norm gains) "
                         "to take no weight decay, in the same update "
                         "launch (mta_list_set_no_decay)")
    ap.add_argument("--torch-reference", action="store_true",
                    help="after the timed steps, also time PyTorch's own "
                         "clip_grad_norm_ + AdamW(fused=True) on the same "
                         "tensors (float32-gradient AdamW workloads only), "
                         "reported as torch_reference")
    ap.add_argument("--opt", default="adamw",
                    choices=["adamw", "adam", "sgd", "momentum"],
                    help="update rule (mta_step); adamw runs mta_adamw_step")
    ap.add_argument("--zero-grad", action="store_true",
                    help="also zero every gradient in the update launch")
    ap.add_argument("--graph", action="store_true",
                    help="loss-scaled workloads only: after the eager pass, "
                         "capture one whole step in a HIP graph and time K "
                         "replays (value and ms_per_step then come from the "
                         "replays; per-kernel times from the eager pass)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the independent ceiling (AMD- and "
                         "PyTorch-owned kernels on buffers of the "
                         "workload's size)")
    ap.add_argument("--probes", action="store_true",
                    help="also time this project's ceiling probes "
                         "(bench_probes/libmta_probe.so, built by "
                         "python bench_probes/build.py)")
    ap.add_argument("--ceiling-only", action="store_true",
                    help="only time the independent ceiling (AMD- and "
                         "PyTorch-owned kernels on buffers of the "
                         "workload's size) and print it as one JSON line: "
                         "a trace of this run holds those kernels alone")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run torch's device copy of 1 GiB, 5 times: "
                         "the known-size kernel that scales the HBM byte "
                         "counters of a profile")
    return ap


def main():
    args = make_parser().parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU "
              "path (the step measured here is one GPU's; how it would shard "
              "is described, not built)", file=sys.stderr)
        sys.exit(2)

    import torch

    import mixed_precision_optimizer_mta_amd as M
    from mixed_precision_optimizer_mta_amd import workloads as WL

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        n = 1 << 28                      # 1 GiB of float32 each way
        src = torch.ones(n, device="cuda")
        dst = torch.empty(n, device="cuda")
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": 4 * n,
                          "calibrate_copy_bytes_written": 4 * n,
                          "launches": 5}), flush=True)
        return
    wl = WL.get(args.workload)
    if args.ceiling_only:
        print(json.dumps({"workload": wl.name, "params": wl.n,
                          "ceiling": independent_ceiling(wl)}), flush=True)
        return
    M.lib()
    if args.joint_norm > 1 and args.scale_inplace:
        print("--joint-norm with --scale-inplace is not measured",
              file=sys.stderr)
        sys.exit(2)
    if args.scale_inplace and (wl.amp or wl.scale == 1.0):
        print("--scale-inplace needs a workload with a fixed unscale factor "
              "(not loss-scaled): e.g. --workload gpt2_124m_bf16g",
              file=sys.stderr)
        sys.exit(2)
    # PyTorch's step on the same tensors needs float32 gradients (its
    # optimizers take the parameter's dtype) and is the AdamW step itself
    ref_ok = wl.gtype == WL.F32 and not wl.amp and args.opt == "adamw" \
        and not args.zero_grad and not args.weight_copy and \
        not args.scale_inplace
    if args.torch_reference and not ref_ok:
        print("--torch-reference needs a plain AdamW step on float32 "
              "gradients", file=sys.stderr)
        sys.exit(2)
    torch_ref = args.torch_reference
    if args.graph and not wl.amp:
        print("--graph needs a loss-scaled workload (its step counter and "
              "scale live on the device, so a captured step can be "
              "replayed): e.g. --workload gpt2_124m_f16amp", file=sys.stderr)
        sys.exit(2)
    offsets = None
    if args.layout == "flat":
        offsets = [0]
        for n in wl.sizes[:-1]:
            offsets.append(offsets[-1] + n)
    arena = WL.Arena(wl, "cuda", offsets)
    arena.fill_weights()
    arena.fill_grads(1)
    opt = opt_of(wl, args.opt, args.zero_grad)
    general = args.opt != "adamw" or args.zero_grad
    has_m, has_v = args.opt != "sgd", args.opt in ("adamw", "adam")
    ents = [(w, g, m if has_m else None, v if has_v else None, n)
            for (w, g, m, v, n) in arena.entries()]
    L = M.MtaList([], entries=ents, gtype=wl.gtype, mkind=wl.mkind,
                  vkind=wl.vkind)
    copies = None
    if args.weight_copy:
        cdt = torch.float16 if args.weight_copy == "f16" else torch.bfloat16
        copies = torch.empty(arena.total, dtype=cdt, device="cuda")
        L.set_weight_copies([copies[o:o + n] for o, n in
                             zip(arena.offsets, wl.sizes)])
    no_decay = [n < NO_DECAY_BELOW for n in wl.sizes] if args.no_decay \
        else None
    if no_decay:
        L.set_no_decay(no_decay)
    info = L.info()
    norm_lists = [L]
    if args.joint_norm > 1:
        k = args.joint_norm
        cuts = [round(i * len(ents) / k) for i in range(k + 1)]
        norm_lists = [M.MtaList([], entries=[e[:2] + (None, None, e[4])
                                             for e in ents[a:b]],
                                gtype=wl.gtype, mkind=wl.mkind,
                                vkind=wl.vkind)
                      for a, b in zip(cuts, cuts[1:]) if b > a]
    norm_d = torch.zeros(1, device="cuda")
    coef_d = torch.zeros(1, device="cuda")
    stream = torch.cuda.current_stream()
    hp = M._binding.mta_adamw_hparams(wl.lr, wl.beta1, wl.beta2, wl.eps,
                                      wl.weight_decay)
    inplace = bool(args.scale_inplace)
    defer = wl.scale != 1.0 and not inplace
    amp = M.AmpState(wl.amp_scale) if wl.amp else None
    if defer and len(norm_lists) > 1:
        # norm-only lists never step, so a deferred factor set once stays
        # pending and applies to every later norm
        for x in norm_lists:
            x.scale(wl.scale, defer=True)

    def step(t, ev=None):
        if ev is not None and inplace:
            ev[3].record(stream)
        if inplace:
            L.scale(wl.scale if t % 2 else 1.0 / wl.scale, defer=False)
        if defer:
            L.scale(wl.scale, defer=True)
        if ev is not None:
            ev[0].record(stream)
        if len(norm_lists) > 1:
            M.clip_norm_joint(norm_lists, wl.max_norm, norm_d, coef_d,
                              amp=amp)
        elif amp is not None:
            L.amp_clip_norm(wl.max_norm, amp, norm_d, coef_d)
        else:
            L.clip_norm(wl.max_norm, norm_d, coef_d)
        if ev is not None:
            ev[1].record(stream)
        if general and amp is not None:
            L.amp_step(opt, amp, coef_d)
        elif general:
            L.step(opt, t, coef_d)
        elif amp is not None:
            L.amp_adamw_step(hp, amp, coef_d)
        else:
            L.adamw_step(hp, t, coef_d)
        if ev is not None:
            ev[2].record(stream)
        if amp is not None:      # one thread; not part of the update's time
            amp.update(wl.amp_growth, wl.amp_backoff, wl.amp_interval)

    t = 0
    for _ in range(args.warmup):
        t += 1
        step(t)
    torch.cuda.synchronize()

    # per-kernel events on an evenly spaced sample of ~50 timed steps: each
    # record costs the host a few microseconds, which a launch-bound list
    # (tiny) would otherwise pay every step
    every = max(1, args.steps // 50)
    evs = {k: [torch.cuda.Event(enable_timing=True) for _ in range(4)]
           for k in range(0, args.steps, every)}
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        t += 1
        step(t, evs.get(k))
    end.record(stream)
    torch.cuda.synchronize()
    host_s = time.perf_counter() - h0
    dev_ms = start.elapsed_time(end)
    ms_per_step = dev_ms / args.steps
    norm_ms = sum(e[0].elapsed_time(e[1]) for e in evs.values()) / len(evs)
    adamw_ms = sum(e[1].elapsed_time(e[2]) for e in evs.values()) / len(evs)
    first = 3 if inplace else 0
    per_step = sorted(e[first].elapsed_time(e[2]) for e in evs.values())
    scale_ms = (sum(e[3].elapsed_time(e[0]) for e in evs.values()) /
                len(evs)) if inplace else None

    def pct(q):
        return per_step[min(len(per_step) - 1, int(q * len(per_step)))]
    assert torch.isfinite(norm_d).all() and torch.isfinite(coef_d).all()
    if amp is not None:      # every timed step was taken, none skipped
        st = amp.read()
        assert st["step"] == t and st["found_inf"] == 0.0, st
    if args.graph:
        # one whole step captured once; every replay reads t and the scale
        # from the device state, so replays are successive steps
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(graph, stream=side):
            step(0)
        torch.cuda.current_stream().wait_stream(side)
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        start.record(stream)
        h0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        end.record(stream)
        torch.cuda.synchronize()
        host_s = time.perf_counter() - h0
        dev_ms = start.elapsed_time(end)
        ms_per_step = dev_ms / args.steps
        st = amp.read()
        assert st["step"] == t + args.warmup + args.steps, st
        assert st["found_inf"] == 0.0, st

    bpp = {"norm": wl.bytes_per_param()["norm"],
           "update": update_bytes(wl, args.opt, args.zero_grad,
                                  args.weight_copy)}
    kernel = KERNEL_OF[args.opt]
    scale_bytes = wl.n * 2 * (4 if wl.gtype == WL.F32 else 2) if inplace \
        else 0
    step_bytes = wl.n * (bpp["norm"] + bpp["update"]) + scale_bytes
    adamw_bytes = wl.n * bpp["update"]
    norm_bytes = wl.n * bpp["norm"]
    value = wl.n * args.steps / (host_s)
    achieved = adamw_bytes / (adamw_ms * 1e-3) / 1e9
    traffic = (None if args.weight_copy or args.layout != "padded" or inplace
               or args.no_decay else measured_traffic(traffic_key(wl, args.opt, args.zero_grad),
                                     kernel))
    out = {
        "metric": "params updated/sec and achieved HBM GB/s (% of peak) per "
                  "fused clip+AdamW step",
        "value": value,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": host_s * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "params": wl.n, "tensors": wl.count,
            "layout": args.layout, "vector_tensors": info["vector_tensors"],
            "grad": ["f32", "bf16", "f16"][wl.gtype],
            "loss_scaling": "dynamic (device state)" if wl.amp else "none",
            "m": ["f32", "bf16x2"][wl.mkind], "v": ["f32", "bf16x2"][wl.vkind],
            "unscale": ("in place (k_scale)" if inplace else "deferred"
                        if defer else "none"),
            "bytes_per_param": bpp["norm"] + bpp["update"] +
            scale_bytes // wl.n,
            "tiles": info["tiles"], "grid_update": info["grid_update"],
            "grid_norm": info["grid_norm"],
            "norm_kept_tiles": info["norm_kept_tiles"],
            "parallelism": "single GPU",
            "weight_copy": args.weight_copy,
            "optimizer": args.opt, "zero_grad": bool(args.zero_grad),
            "graph": bool(args.graph),
            "joint_norm_lists": len(norm_lists),
            "no_decay_tensors": sum(no_decay) if no_decay else 0,
        },
        "step_gbs": step_bytes / (dev_ms * 1e-3 / args.steps) / 1e9,
        "step_hbm_frac": step_bytes / (dev_ms * 1e-3 / args.steps) / 1e9
        / HBM_PEAK_GBS,
        "device_ms_per_step": ms_per_step,
        "step_ms_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
        "kernels_ms": {"k_sumsq": norm_ms, kernel: adamw_ms,
                       **({"k_scale": scale_ms} if inplace else {})},
        "norm_gbs": norm_bytes / (norm_ms * 1e-3) / 1e9,
        # the second kernel of the step, measured the same way
        "norm_roofline": {
            "kernel": "k_sumsq", "bound": "hbm",
            "achieved": norm_bytes / (norm_ms * 1e-3) / 1e9,
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": norm_bytes / (norm_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "traffic": (None if args.layout != "padded" or inplace or
                        len(norm_lists) > 1
                        else measured_traffic(traffic_key(
                            wl, args.opt, args.zero_grad), "k_sumsq")),
            "bytes_per_launch": norm_bytes,
        },
        **({"scale_gbs": scale_bytes / (scale_ms * 1e-3) / 1e9}
           if inplace else {}),
        "roofline": {
            "kernel": kernel, "bound": "hbm", "achieved": achieved,
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
            "bytes_per_launch": adamw_bytes,
        },
    }
    # the counters' HBM bytes per launch at the same live launch time
    for key, ms in (("norm_roofline", norm_ms), ("roofline", adamw_ms)):
        r = out[key]
        r["traffic_gbs"] = (None if r["traffic"] is None
                            else r["traffic"] / (ms * 1e-3) / 1e9)
    L.close()
    for x in norm_lists[1:] if len(norm_lists) > 1 else []:
        x.close()
    if not args.no_ceiling:
        c = independent_ceiling(wl)
        c["update_of_add"] = achieved / c["add_gbs"]
        c["update_of_addcmul"] = achieved / c["addcmul_gbs"]
        out["ceiling"] = c
    if args.probes and args.opt in ("adamw", "adam") and \
            not args.zero_grad and not args.weight_copy:
        c = probe_ceiling(wl)
        c["update_of_mix"] = achieved / c["update_mix_gbs"]
        c["update_of_serial_bound"] = achieved / c["serial_bound_gbs"]
        out["probe_ceiling"] = c
    if args.cpu_steps is None or args.cpu_steps > 0:
        out["cpu_baseline"] = cpu_baseline(arena, wl, args.cpu_steps, opt)
        cpu_steps = out["cpu_baseline"]["steps"]
        if not general and not wl.amp and not args.weight_copy:
            # a one-GPU job is given 16 cores on an MI355X node: the pool
            # takes at most that many, and no more than this process may use
            try:
                usable = len(os.sched_getaffinity(0))
            except (AttributeError, OSError):
                usable = os.cpu_count() or 1
            threads = max(1, min(16, usable))
            out["cpu_baseline_parallel"] = cpu_baseline_parallel(
                arena, wl, cpu_steps, threads)
    if torch_ref:
        out["torch_reference"] = torch_reference(arena, wl)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
