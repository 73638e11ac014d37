"""MtaOptimizer: a torch.optim-style front end over the C ABI.

Marshalling only, like MtaList: it allocates the state buffers a rule needs
(float32, or bfloat16 for packed Adam-family moments), keeps them in
``self.state`` under PyTorch's names (exp_avg, exp_avg_sq, momentum_buffer)
so ``state_dict()`` / ``load_state_dict()`` work, and drives one list per
parameter set (below) and gradient dtype.  A step is:

  * with ``max_norm``: one clip over the joint norm of every gradient of
    every group (mta_clip_norm_joint over one norm list per gradient dtype,
    lists with no state buffers), the norm and coefficient left in device
    tensors (``last_norm``, ``last_coef``);
  * one mta_step per parameter set and gradient dtype with that
    coefficient.  A set is one parameter group, or several groups with
    equal lr, betas, eps and momentum and at most one nonzero weight decay
    among them (the usual decay / no-decay split): they share one list and
    one launch, the tensors of their zero-decay groups flagged to take no
    decay (mta_list_set_no_decay), each updated exactly as its own group's
    step would update it.  The sets are recomputed from the groups'
    hyperparameters every step; a change of the sets (not of the values,
    such as a new lr common to all) rebuilds the plan.

With ``loss_scale`` (an initial scale) the step is loss-scaled on the
device: ``opt.loss_scale`` is a one-element float32 device view of the
current scale (multiply the loss by it before backward), the joint norm
unscales by 1/scale and sets the found-inf flag, every group's update is
skipped on overflow, and the scale then grows or backs off (PyTorch's
GradScaler rule) -- no host synchronization anywhere.  The step counter
lives in ``opt.amp`` (an AmpState), not in ``self.state``; ``state_dict()``
saves that state under "mta_amp" (and each parameter's up-to-date "step"),
and ``load_state_dict()`` restores it.

``capturable=True`` keeps the step counter on the device without loss
scaling (a state whose scale is 1 and never grows: the unscale multiplies by
exactly 1), so ``step()`` can be captured in a HIP graph and replayed; the
one difference from the plain step is that a non-finite gradient skips the
update instead of spreading NaN.  Run one eager step first (it builds the
device tables, which allocates), and keep the gradients' storage across
replays (``zero_grad=True`` zeroes them inside the update launch).  A
replay reuses the captured tables and hyperparameters: after a change that
rebuilds the plan (a moved gradient, a change of the parameter sets) or of
a hyperparameter, run an eager step and capture again.

``master_weights=True`` is for a model kept in bfloat16 or float16: the
optimizer holds a float32 master copy of every 16-bit parameter (``state[p]
["master_weight"]``), the update runs on the masters with the model's 16-bit
gradients, and the same launch writes the 16-bit rounding of each new master
into the parameter itself (the list's weight copies).  The model's forward
and backward then read and produce 16-bit values only, while the weights
accumulate updates in float32.  A parameter the model keeps in float32 (one
whose uses need full precision) is its own master and takes no copy; its
float32 gradient joins the same joint clip.

Every step of the arithmetic runs in libmta.  Parameters are float32 CUDA
tensors (with master_weights, also bfloat16 or float16 ones); gradients are
float32, bfloat16 or float16, a 16-bit parameter's in its own dtype.  The
device tables
are rebuilt whenever a parameter, gradient or state buffer moved.  This
class's ``zero_grad()`` therefore zeroes gradients in place by default
(``set_to_none=False``), so a plain ``backward(); step(); zero_grad()`` loop
keeps one plan; ``zero_grad(set_to_none=True)`` lets PyTorch reallocate
the gradients and costs a rebuild at the next step, and ``zero_grad=True``
in the constructor zeroes them inside the update launch instead.
``tables_built`` counts the device tables built so far.
``load_state_dict`` keeps every state tensor in the dtype it was saved in
(PyTorch's default would cast float32 masters and moments to a 16-bit
parameter's dtype).

Host cost: the checks, the device tables and the step counts form a plan
that a step reuses while every parameter and gradient keeps its address and
dtype, so a step costs two address reads per parameter on the host (0.04 ms
for 110 tensors, 2.9 ms for 10,000) besides its launches.  Tensors are
checked when the plan is built.  The per-parameter ``state[p]["step"]`` is
brought up to date by ``state_dict()`` (and whenever the plan is rebuilt);
in between, the count lives with the plan.
"""
import torch

from . import _binding as B
from .torch_list import MtaList, clip_norm_joint

_KINDS = ("adamw", "adam", "sgd", "momentum")
_GTYPE = {torch.float32: B.MTA_F32, torch.bfloat16: B.MTA_BF16,
          torch.float16: B.MTA_F16}


class MtaOptimizer(torch.optim.Optimizer):
    """kind: "adamw" (decoupled decay), "adam" (coupled decay), "sgd",
    "momentum" (SGD with momentum, no dampening, not Nesterov)."""

    def __init__(self, params, kind="adamw", lr=1e-3, betas=(0.9, 0.999),
                 eps=1e-8, weight_decay=0.0, momentum=0.0, max_norm=None,
                 packed_moments=False, zero_grad=False, loss_scale=None,
                 growth_factor=2.0, backoff_factor=0.5,
                 growth_interval=2000, capturable=False,
                 master_weights=False):
        if kind not in _KINDS:
            raise ValueError(f"kind must be one of {_KINDS}")
        if packed_moments and kind not in ("adamw", "adam"):
            raise ValueError("packed moments are for the Adam family")
        defaults = dict(lr=lr, betas=tuple(betas), eps=eps,
                        weight_decay=weight_decay, momentum=momentum)
        super().__init__(params, defaults)
        self.kind = kind
        self.max_norm = max_norm
        self.packed = bool(packed_moments)
        self.zero_grad_in_step = bool(zero_grad)
        self.master_weights = bool(master_weights)
        self._lists = {}       # (groups, grad dtype) -> (key, MtaList)
        self._norm_cache = {}  # grad dtype -> (pointer key, MtaList)
        self._plan = None      # see step()
        self.tables_built = 0  # device tables built (list handles made)
        self.last_norm = None
        self.last_coef = None
        self.amp = None
        self.loss_scale = None
        if loss_scale is None and capturable:
            # a device step counter without loss scaling: scale 1 that never
            # grows within 2^31 - 1 good steps
            loss_scale, growth_interval = 1.0, 2 ** 31 - 1
        if loss_scale is not None:
            from .torch_list import AmpState
            self.amp = AmpState(float(loss_scale))
            # the scale is the state's first 4 bytes
            self.loss_scale = self.amp.buf.view(torch.float32)[:1]
            self._amp_rule = (float(growth_factor), float(backoff_factor),
                              int(growth_interval))

    def zero_grad(self, set_to_none: bool = False):
        """PyTorch's zero_grad, with set_to_none False by default: every
        gradient keeps its storage and is zeroed in place, so the next step
        finds the gradients at the addresses its plan holds and reuses it.
        With set_to_none=True the next backward allocates new gradients and
        the next step builds new device tables (a device allocation, an
        upload and a wait on the host), as any address change does."""
        super().zero_grad(set_to_none=set_to_none)

    # -- state buffers ----------------------------------------------------
    def master(self, p):
        """The float32 weight the update runs on: p itself (a float32
        parameter), or the master of a 16-bit one."""
        if p.dtype == torch.float32:
            return p
        st = self.state[p]
        if "master_weight" not in st:
            st["master_weight"] = p.detach().float().contiguous()
        return st["master_weight"]

    def _state_buffers(self, p):
        st = self.state[p]
        mdt = torch.bfloat16 if self.packed else torch.float32
        if self.kind in ("adamw", "adam"):
            if "exp_avg" not in st:
                st["exp_avg"] = torch.zeros_like(p, dtype=mdt)
                st["exp_avg_sq"] = torch.zeros_like(p, dtype=mdt)
                st["step"] = 0
            for name in ("exp_avg", "exp_avg_sq"):
                # load_state_dict casts floating state to the parameter's
                # dtype; a bfloat16 moment comes back exactly
                if st[name].dtype != mdt:
                    st[name] = st[name].to(mdt).contiguous()
            return st["exp_avg"], st["exp_avg_sq"]
        if self.kind == "momentum":
            if "momentum_buffer" not in st:
                st["momentum_buffer"] = torch.zeros_like(
                    p, dtype=torch.float32)
                st["step"] = 0
            return st["momentum_buffer"], None
        st.setdefault("step", 0)
        return None, None

    def _check(self, p):
        if self.master_weights:
            if p.dtype not in _GTYPE or not p.is_cuda or \
                    not p.is_contiguous():
                raise TypeError("with master_weights, parameters must be "
                                "contiguous float32, bfloat16 or float16 "
                                "CUDA tensors")
        elif p.dtype != torch.float32 or not p.is_cuda or \
                not p.is_contiguous():
            raise TypeError("parameters must be contiguous float32 CUDA "
                            "tensors (16-bit ones need master_weights=True)")
        g = p.grad
        if g is None or not g.is_cuda or not g.is_contiguous():
            raise ValueError("every parameter needs a contiguous CUDA "
                             "gradient before step()")

    def _group_list(self, k, params, no_decay=None):
        """The update list of these params (all with one gradient dtype;
        k is (group indices, dtype)); no_decay: one flag per param, or
        None."""
        groups, key = [], [tuple(no_decay) if no_decay else None]
        for p in params:
            m, v = self._state_buffers(p)
            w = self.master(p)
            groups.append((w, p.grad, m, v))
            key.append((w.data_ptr(), p.grad.data_ptr(),
                        None if m is None else m.data_ptr(),
                        None if v is None else v.data_ptr(), p.numel(),
                        p.grad.dtype, p.data_ptr()))
        key = tuple(key)
        cached = self._lists.get(k)
        if cached is None or cached[0] != key:
            if cached is not None:
                cached[1].close()
            mk = B.MTA_MOM_BF16X2 if self.packed else B.MTA_MOM_F32
            self.tables_built += 1
            L = MtaList([], entries=[(w.data_ptr(), g.data_ptr(),
                                      None if m is None else m.data_ptr(),
                                      None if v is None else v.data_ptr(),
                                      w.numel()) for w, g, m, v in groups],
                        gtype=_GTYPE[groups[0][1].dtype], mkind=mk, vkind=mk)
            L._keep = groups
            if any(p.dtype != torch.float32 for p in params):
                # 16-bit parameters are the list's weight copies (a float32
                # one among them is its own weight and takes none)
                L.set_weight_copies([None if p.dtype == torch.float32
                                     else p.detach() for p in params])
            if no_decay and any(no_decay):
                L.set_no_decay(no_decay)
            self._lists[k] = (key, L)
        return self._lists[k][1]

    def _merge_sig(self):
        """The parameter sets the current hyperparameters allow: for each
        group, (index of the first group of its set, its weight decay is
        0).  Groups with equal lr, betas, eps and momentum form one set when
        at most one nonzero weight decay appears among them; otherwise each
        of them is a set of its own."""
        keys, nonzero = [], {}
        for g in self.param_groups:
            key = (float(g["lr"]), tuple(float(b) for b in g["betas"]),
                   float(g["eps"]), float(g["momentum"]))
            keys.append(key)
            if float(g["weight_decay"]) != 0.0:
                nonzero.setdefault(key, set()).add(float(g["weight_decay"]))
        first, out = {}, []
        for i, (g, key) in enumerate(zip(self.param_groups, keys)):
            if len(nonzero.get(key, ())) > 1:
                head = i
            else:
                head = first.setdefault(key, i)
            out.append((head, float(g["weight_decay"]) == 0.0))
        return tuple(out)

    def _norm_lists(self, all_params):
        """One norm list per gradient dtype (float32, bfloat16, float16
        order); the clip is over their joint norm."""
        out, keys = [], []
        for dt in _GTYPE:
            ps = [p for p in all_params if p.grad.dtype == dt]
            if not ps:
                continue
            # the norm reads only the gradients; w is the float32 weight
            # the list's validation sizes as 4 bytes per element
            ws = [self.master(p) for p in ps]
            key = tuple((w.data_ptr(), p.grad.data_ptr(), p.numel())
                        for w, p in zip(ws, ps))
            cached = self._norm_cache.get(dt)
            if cached is None or cached[0] != key:
                if cached is not None:
                    cached[1].close()
                self.tables_built += 1
                L = MtaList([], entries=[(w.data_ptr(), p.grad.data_ptr(),
                                          None, None, p.numel())
                                         for w, p in zip(ws, ps)],
                            gtype=_GTYPE[dt], mkind=B.MTA_MOM_F32,
                            vkind=B.MTA_MOM_F32)
                L._keep = [(w, p.grad) for w, p in zip(ws, ps)]
                self._norm_cache[dt] = (key, L)
            out.append(self._norm_cache[dt][1])
            keys.append(dt)
        for dt in [d for d in self._norm_cache if d not in keys]:
            self._norm_cache.pop(dt)[1].close()
        return out

    # -- the step ---------------------------------------------------------
    @torch.no_grad()
    def step(self, closure=None):
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        groups = [[p for p in g["params"] if p.grad is not None]
                  for g in self.param_groups]
        # The plan (checked tensors, device tables, per-list step counts)
        # is rebuilt only when a parameter or gradient moved or changed
        # dtype: two addresses and a dtype per parameter per step, not the
        # checks and the table keys.
        sig = tuple((p.data_ptr(), p.grad.data_ptr(), p.grad.dtype)
                    for ps in groups for p in ps)
        msig = self._merge_sig()
        if self._plan is None or sig != self._plan["sig"] or \
                msig != self._plan["merge_sig"]:
            self._sync_steps()
            self._plan = self._build_plan(groups, sig, msig)
        plan = self._plan
        if not plan["updates"]:
            return loss
        coef = None
        if self.max_norm is not None or self.amp is not None:
            cap = float("inf") if self.max_norm is None else \
                float(self.max_norm)
            clip_norm_joint(plan["norm_lists"], cap, self.last_norm,
                            self.last_coef, amp=self.amp)
            coef = self.last_coef
        for u in plan["updates"]:
            # the set's groups share every value but the weight decay; the
            # flagged (zero-decay) tensors ignore the one given here
            group = self.param_groups[u["group"]]
            b1, b2 = group["betas"]
            wd = next((w for w in (float(self.param_groups[i]
                                         ["weight_decay"])
                                   for i in u["groups"]) if w != 0.0), 0.0)
            rule = dict(kind=self.kind, lr=group["lr"], beta1=b1, beta2=b2,
                        eps=group["eps"], weight_decay=wd,
                        momentum=group["momentum"],
                        zero_grad=self.zero_grad_in_step)
            if self.amp is not None:
                u["list"].amp_step(rule, self.amp, coef)
            else:
                u["t"] += 1
                u["list"].step(rule, u["t"], coef)
        if self.amp is not None:
            self.amp.update(*self._amp_rule)
        return loss

    def _build_plan(self, groups, sig, msig):
        all_params = [p for ps in groups for p in ps]
        for p in all_params:
            self._check(p)
            if p.grad.dtype not in _GTYPE:
                raise TypeError("gradients are float32, bfloat16 or float16")
            if p.dtype != torch.float32 and p.grad.dtype != p.dtype:
                raise TypeError("a 16-bit parameter's gradient has its dtype")
        plan = dict(sig=sig, merge_sig=msig, norm_lists=[], updates=[])
        if not all_params:
            return plan
        dev = all_params[0].device
        if self.last_norm is None or self.last_norm.device != dev:
            self.last_norm = torch.zeros(1, device=dev)
            self.last_coef = torch.zeros(1, device=dev)
        plan["norm_lists"] = self._norm_lists(all_params)
        for p in all_params:
            self._state_buffers(p)
        steps = []
        for k, ps in enumerate(groups):
            st = {int(self.state[p]["step"]) for p in ps}
            if self.amp is None and len(st) > 1:
                raise RuntimeError(
                    "the parameters of one group have taken different "
                    "numbers of steps; one launch applies one t to a group")
            steps.append(max(st) if st else 0)
        # the sets: groups of one merge head, and (the step count is one t
        # per launch) of one step count unless the device counts steps
        sets = {}
        for k, (head, _) in enumerate(msig):
            if groups[k]:
                t = 0 if self.amp is not None else steps[k]
                sets.setdefault((head, t), []).append(k)
        used = set()
        for (head, _), ks in sorted(sets.items(), key=lambda x: x[1][0]):
            flagged = any(not msig[k][1] for k in ks) and \
                any(msig[k][1] for k in ks)
            for dt in _GTYPE:   # one launch per gradient dtype in the set
                ps, nd = [], []
                for k in ks:
                    for p in groups[k]:
                        if p.grad.dtype == dt:
                            ps.append(p)
                            nd.append(flagged and msig[k][1])
                if not ps:
                    continue
                lk = (tuple(ks), dt)
                used.add(lk)
                L = self._group_list(lk, ps, nd if flagged else None)
                plan["updates"].append(dict(
                    group=ks[0], groups=tuple(ks), list=L, params=ps,
                    t=max(steps[k] for k in ks)))
        for lk in [x for x in self._lists if x not in used]:
            self._lists.pop(lk)[1].close()
        return plan

    def _sync_steps(self):
        """Write each list's step count into its parameters' state (the
        step loop keeps one count per list, not per parameter)."""
        if self._plan is None or self.amp is not None:
            return
        for u in self._plan["updates"]:
            for p in u["params"]:
                self.state[p]["step"] = u["t"]

    # -- checkpoints ------------------------------------------------------
    def state_dict(self):
        """As torch.optim.Optimizer.state_dict, with every parameter's
        "step" brought up to date.  With a loss-scale state (loss_scale= or
        capturable=True) the count comes from the device counter, and the
        state itself (scale, found_inf, growth_tracker, step) is saved under
        "mta_amp"; reading it synchronizes the stream."""
        self._sync_steps()
        sd = super().state_dict()
        if self.amp is not None:
            amp = self.amp.read()
            sd["mta_amp"] = amp
            sd["state"] = {k: dict(v, step=amp["step"]) if "step" in v
                           else v for k, v in sd["state"].items()}
        return sd

    def load_state_dict(self, state_dict):
        """As torch.optim.Optimizer.load_state_dict, except that every state
        tensor comes back in the dtype it was saved in (masters and float32
        moments of a 16-bit parameter stay float32).  The state buffers are
        new allocations and the device tables are rebuilt on the next step:
        capture a graph of step() again after loading.

        With a loss-scale state, the saved one ("mta_amp") is written back
        to the device; a checkpoint without one (saved by a plain
        optimizer) sets the device step counter from the parameters'
        common "step" and keeps the current scale.  A plain optimizer
        takes the saved per-parameter counts either way."""
        self._plan = None          # its step counts belong to the old state
        if self.amp is not None:
            amp = state_dict.get("mta_amp")
            if amp is None:
                steps = {int(v["step"]) for v in
                         state_dict["state"].values() if "step" in v}
                if len(steps) > 1:
                    raise ValueError(
                        "a loss-scaled optimizer keeps one step count; the "
                        f"checkpoint's parameters have taken {sorted(steps)}")
                cur = self.amp.read()
                amp = dict(cur, step=steps.pop() if steps else cur["step"],
                           found_inf=0.0)
        super().load_state_dict(state_dict)
        if self.amp is not None:
            self.amp.write(amp["scale"], amp["step"], amp["growth_tracker"],
                           amp["found_inf"])
        ids = [i for g in state_dict["param_groups"] for i in g["params"]]
        params = [p for g in self.param_groups for p in g["params"]]
        saved = state_dict["state"]
        for i, p in zip(ids, params):
            for name, val in saved.get(i, {}).items():
                if torch.is_tensor(val) and name != "step":
                    self.state[p][name] = val.to(
                        device=p.device, dtype=val.dtype,
                        copy=True).contiguous()
        # every table is rebuilt on the next step
        for _, L in self._lists.values():
            L.close()
        self._lists = {}
