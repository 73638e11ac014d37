"""Seeded synthetic workloads: tensor-list shapes and input generators.

This module holds no optimizer arithmetic.  It only says which tensors a
workload has, and fills weights and gradients with seeded normal draws
(torch's generators, on the device the arena lives on; a 16-bit gradient
is torch's own float32 -> bfloat16 / float16 conversion of the drawn value).  Moments
start at zero.  The tests and the benchmark feed the same bytes to the HIP
library and to the CPU oracle.

Workloads (parameter counts are exact):
  tiny       3 tensors [384x384], [384x1536], [1536]: 738,816 params, f32
             w ~ N(0, 0.02), g ~ N(0, 0.01), f32 moments, 10 steps.
  gpt2_124m  GPT-2-small-shaped list, 110 tensors, 124,419,840 params:
             wte 50257x768, wpe 1024x768, 12 x {ln 768x2, c_attn 768x2304 +
             2304, proj 768x768 + 768, fc 768x3072 + 3072, fc2 3072x768 +
             768}; f32 g ~ N(0, 1e-3), f32 moments.
  gpt2_124m_bf16g  the same list with bfloat16 gradients holding
             65536 * N(0, 1e-3), unscaled by 2^-16 before the clip; f32
             moments; 100 steps.
  gpt2_124m_f16amp  the same list with float16 gradients under dynamic loss
             scaling: a device loss-scale state starting at 65536 (growth 2,
             backoff 0.5, interval 2000), gradients holding 65536 *
             N(0, 1e-3); f32 moments.
  gpt2_xl    GPT-2-XL-shaped list (vocab 50257, d 1600, 48 layers, d_ff
             6400), 434 tensors, 1,557,454,400 params; f32 g ~ N(0, 1e-3),
             packed bfloat16 m and v.
  ragged     10,000 tensors of max(1, floor(2^(20u))) elements, u ~ U(0,1),
             plus two 50257x1024 embeddings; bfloat16 g ~ N(0, 1e-2) with 1%
             of the 10,000 all-zero; packed bfloat16 m, f32 v; wd = 0.01.
All use lr 3e-4, betas (0.9, 0.999), eps 1e-8, weight decay 0.1 (ragged:
0.01), clip 1.0, and w ~ N(0, 0.02) unless stated.

<name>_shard<r>of<N> is rank r's share of workload <name> when its flat
element space is cut into N equal ranges (tensors split at the range
edges): one GPU's list under sharded optimizer state, e.g.
gpt2_xl_shard0of8 (194,681,800 params in 35 pieces).
"""
import re
from dataclasses import dataclass, field

import numpy as np

SEED = 20261202

F32, BF16, F16 = 0, 1, 2
MOM_F32, MOM_BF16X2 = 0, 1

# element alignment of every tensor inside an arena: 128 elements is 512 B
# of float32 and 256 B of bfloat16, so all four buffers of a tensor start
# 16-byte aligned and share one element offset
ALIGN_ELEMS = 128


@dataclass
class Workload:
    name: str
    sizes: list
    gtype: int
    mkind: int
    vkind: int
    steps: int
    lr: float = 3e-4
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.1
    max_norm: float = 1.0
    scale: float = 1.0          # deferred unscale factor (1 = none)
    w_sigma: float = 0.02
    g_sigma: float = 1e-3
    g_mult: float = 1.0         # gradient stored as g_mult * N(0, g_sigma)
    zero_grad: frozenset = field(default_factory=frozenset)
    ident: int = 0
    amp: bool = False           # dynamic loss scaling with a device state
    amp_scale: float = 65536.0  # its initial scale
    amp_growth: float = 2.0
    amp_backoff: float = 0.5
    amp_interval: int = 2000

    @property
    def n(self):
        return int(sum(self.sizes))

    @property
    def count(self):
        return len(self.sizes)

    @property
    def hparams(self):
        return dict(lr=self.lr, beta1=self.beta1, beta2=self.beta2,
                    eps=self.eps, weight_decay=self.weight_decay)

    def bytes_per_param(self):
        """Algorithmic HBM bytes per parameter of one step: the norm reads g
        once; the update reads w, g, m, v and writes w, m, v."""
        gb = 4 if self.gtype == F32 else 2
        mb = 2 if self.mkind == MOM_BF16X2 else 4
        vb = 2 if self.vkind == MOM_BF16X2 else 4
        return {"norm": gb, "update": 4 + gb + mb + vb + 4 + mb + vb}


def gpt2_sizes(vocab, d, ctx, layers, d_ff):
    sizes = [vocab * d, ctx * d]
    for _ in range(layers):
        sizes += [d * 2, d * 3 * d, 3 * d, d * d, d, d * d_ff, d_ff,
                  d_ff * d, d]
    return sizes


def ragged_sizes(count=10_000, seed=SEED):
    rng = np.random.default_rng([seed, 5, 0])
    u = rng.random(count)
    sizes = np.maximum(1, np.floor(2.0 ** (20.0 * u))).astype(np.int64)
    zero = rng.permutation(count)[: count // 100]
    return [int(x) for x in sizes] + [50257 * 1024] * 2, frozenset(
        int(i) for i in zero)


def shard_sizes(sizes, rank, world):
    """The pieces of a tensor list that one of `world` equal ranges of its
    flat element space holds (range `rank`): each tensor cut at the range
    edges, empty pieces dropped, in list order.  This is one GPU's share of
    a list whose optimizer state is sharded across `world` GPUs."""
    total = sum(sizes)
    lo, hi = total * rank // world, total * (rank + 1) // world
    out, off = [], 0
    for n in sizes:
        a, b = max(lo, off), min(hi, off + n)
        if b > a:
            out.append(b - a)
        off += n
    return out


def get(name):
    m = re.fullmatch(r"(.+)_shard(\d+)of(\d+)", name)
    if m:
        base = get(m.group(1))
        rank, world = int(m.group(2)), int(m.group(3))
        if not 0 <= rank < world or base.zero_grad:
            raise KeyError(name)
        import dataclasses
        return dataclasses.replace(
            base, name=name, sizes=shard_sizes(base.sizes, rank, world),
            ident=base.ident * 1000 + world * 10 + rank)
    if name == "tiny":
        return Workload("tiny", [384 * 384, 384 * 1536, 1536], F32, MOM_F32,
                        MOM_F32, steps=10, g_sigma=0.01, ident=1)
    if name == "gpt2_124m":
        return Workload("gpt2_124m", gpt2_sizes(50257, 768, 1024, 12, 3072),
                        F32, MOM_F32, MOM_F32, steps=3, ident=2)
    if name == "gpt2_124m_bf16g":
        return Workload("gpt2_124m_bf16g",
                        gpt2_sizes(50257, 768, 1024, 12, 3072), BF16, MOM_F32,
                        MOM_F32, steps=100, g_mult=65536.0,
                        scale=2.0 ** -16, ident=3)
    if name == "gpt2_124m_f16amp":
        return Workload("gpt2_124m_f16amp",
                        gpt2_sizes(50257, 768, 1024, 12, 3072), F16, MOM_F32,
                        MOM_F32, steps=20, g_mult=65536.0, amp=True, ident=6)
    if name == "gpt2_xl":
        return Workload("gpt2_xl", gpt2_sizes(50257, 1600, 1024, 48, 6400),
                        F32, MOM_BF16X2, MOM_BF16X2, steps=2, ident=4)
    if name == "ragged":
        sizes, zero = ragged_sizes()
        return Workload("ragged", sizes, BF16, MOM_BF16X2, MOM_F32, steps=3,
                        g_sigma=1e-2, weight_decay=0.01, zero_grad=zero,
                        ident=5)
    raise KeyError(name)


NAMES = ("tiny", "gpt2_124m", "gpt2_124m_bf16g", "gpt2_124m_f16amp",
         "gpt2_xl", "ragged")


def scaled_down(wl, sizes, name=None, zero_grad=None):
    """The same workload (dtypes, hyperparameters, distributions) over other
    tensor sizes: for parity runs the oracle finishes in seconds."""
    import dataclasses
    return dataclasses.replace(
        wl, name=name or wl.name + "_small", sizes=list(sizes),
        zero_grad=frozenset(zero_grad or ()))


def _seed(wl, buffer, step):
    return (SEED * 1_000_003 + wl.ident * 10_007 + buffer * 101 + step) % (
        2 ** 63)


class Arena:
    """Flat buffers w, g, m, v for a whole list on one device; tensor i
    occupies elements [off[i], off[i] + n[i]) of each (same element offsets
    for every buffer kind; g_shift, 0..ALIGN_ELEMS-1, moves every gradient
    that many elements further, to give g a different alignment from the
    other buffers)."""

    def __init__(self, wl, device, offsets=None, g_shift=0):
        import torch
        if not 0 <= g_shift < ALIGN_ELEMS:
            raise ValueError("g_shift must be in [0, ALIGN_ELEMS)")
        self.g_shift = int(g_shift)
        self.wl = wl
        self.device = torch.device(device)
        if offsets is None:
            offsets, pos = [], 0
            for n in wl.sizes:
                offsets.append(pos)
                pos += -(-n // ALIGN_ELEMS) * ALIGN_ELEMS
            total = pos
        else:
            total = max([o + n for o, n in zip(offsets, wl.sizes)] + [0])
            total = -(-total // ALIGN_ELEMS) * ALIGN_ELEMS
        self.offsets = [int(o) for o in offsets]
        self.total = int(total) + ALIGN_ELEMS   # room for guard elements
        gd = {F32: torch.float32, BF16: torch.bfloat16,
              F16: torch.float16}[wl.gtype]
        md = torch.bfloat16 if wl.mkind == MOM_BF16X2 else torch.float32
        vd = torch.bfloat16 if wl.vkind == MOM_BF16X2 else torch.float32
        self.w = torch.zeros(self.total, dtype=torch.float32,
                             device=self.device)
        self.g = torch.zeros(self.total, dtype=gd, device=self.device)
        self.m = torch.zeros(self.total, dtype=md, device=self.device)
        self.v = torch.zeros(self.total, dtype=vd, device=self.device)

    def view(self, buf, i):
        o, n = self.offsets[i], self.wl.sizes[i]
        if buf == "g":
            o += self.g_shift
        return getattr(self, buf)[o:o + n]

    def entries(self):
        """(w, g, m, v, n) device pointers for mta_list_create."""
        out = []
        for i, n in enumerate(self.wl.sizes):
            o = self.offsets[i]
            out.append((self.w[o:].data_ptr(),
                        self.g[o + self.g_shift:].data_ptr(),
                        self.m[o:].data_ptr(), self.v[o:].data_ptr(), n))
        return out

    def _gen(self, buffer, step):
        import torch
        gen = torch.Generator(device=self.device)
        gen.manual_seed(_seed(self.wl, buffer, step))
        return gen

    def fill_weights(self):
        import torch
        x = torch.randn(self.total, generator=self._gen(0, 0),
                        device=self.device, dtype=torch.float32)
        self.w.copy_(x * self.wl.w_sigma)
        self.m.zero_()
        self.v.zero_()

    def fill_grads(self, step):
        import torch
        x = torch.randn(self.total, generator=self._gen(1, step),
                        device=self.device, dtype=torch.float32)
        x = x * self.wl.g_sigma
        if self.wl.g_mult != 1.0:
            x = x * self.wl.g_mult
        self.g.copy_(x.to(self.g.dtype))
        for i in self.wl.zero_grad:
            self.view("g", i).zero_()
