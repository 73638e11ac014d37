// mta_kernels.hip -- gfx950 kernels of the fused clip + multi-tensor optimizer
// step.
//
// Kernels:
//   k_sumsq       joint sum of squares -> norm and clip coefficient
//                 (ClipGradNorms, "Mica 7.7: a training step on the card, in
//                 every float type", section "The whole model in one call";
//                 the norm and coefficient stay in device memory, section
//                 "Values that stay on the card"); with a loss-scale state it
//                 also reports whether any unscaled gradient is not finite.
//                 Launches over several lists chain through a float64
//                 running total (one threshold over the norm of all).
//   k_adamw       AdamW over every (w, g, m, v) group (AdamWSteps, same
//                 section), with the element arithmetic of "BendTorch
//                 main.bend", section "Optimizers": adam_decay, adam_m, adam_v,
//                 adam_w, and the packed bfloat16 moments of adamh_l /
//                 adamhv_l (ph_of_bits, ph_to); when a tensor has one, it also
//                 writes the bfloat16 or float16 copy of its new weights
//                 (Mica, section "float16 and bfloat16, whole").  With a loss-scale state it
//                 skips a step whose gradients were not finite and takes the
//                 step number from device memory.  The same kernel runs Adam
//                 with coupled decay (adam_grad with dec = false).
//   k_sgd, k_momentum  the SGD and momentum-SGD rules (sgd_l, mom_l), on the
//                 same tile walk.  Every update kernel can also zero the
//                 gradient after reading it, as every step loop there does.
//   k_scale       ScaleTensors in place (same Mica section), by a factor
//                 given by the host or read from device memory (the clip
//                 coefficient a norm left there: the gradients scaled on
//                 the card, section "Values that stay on the card").
//   k_amp_update  the loss-scale update after a step (one thread).
// Each of the first three is one launch over the whole tensor list.
//
// Gradients are float32, bfloat16 or IEEE float16 (Mica: float16 and bfloat16
// stand beside float32; a float16 step unscales before its clip).
//
// Work is cut into tiles of kTileElems elements of one tensor.  The tile
// tables are built once per list on the host: each record holds the tile's
// own buffer addresses, length and alignment, so one scalar load describes a
// tile.  The update kernels and the in-place scale run one workgroup per
// tile; the norm is a persistent grid that walks the tiles with a grid
// stride.  Inside a full
// tile of a 16-byte-aligned tensor every wave instruction reads or writes one
// contiguous run of memory: lane l of group j owns elements j*G + V*l ..
// j*G + V*l + V-1, where V is 4 for k_adamw (a 16-byte access of a float32
// buffer, 8 bytes of a 16-bit one, so all buffers share one element mapping)
// and 16 bytes' worth for the single-buffer kernels.  The tail tile of a
// tensor, the head tile peeled off a tensor whose buffers reach alignment
// only after a few elements, and the tiles of a tensor that never does take
// the element path: one-element accesses with consecutive lanes on
// consecutive elements, loads clamped into the tile and issued before any
// use, stores masked to the tile.  A lane owns whole elements, so a packed
// bfloat16 moment is written with 8-byte or 16-bit stores and no 32-bit word
// is ever shared between lanes (no read-modify-write of a neighbour's half).
//
// Numerics: this file is compiled with -ffp-contract=off.  Every float32
// operation of the AdamW update is rounded on its own, '/' and sqrtf are the
// correctly rounded ones, and denormals are kept.  The only fused multiply-adds
// are the explicit float64 fma of the norm's accumulation and of the
// double-double power, which need to be accurate, not to follow a fixed
// rounding sequence.
#include <mutex>
#include <type_traits>

#include "mta_internal.h"

namespace mta {
namespace {

// Element types of a buffer (template argument D).
constexpr int kF32 = 0;   // float32
constexpr int kBF16 = 1;  // bfloat16 (packed moments are bfloat16 arrays)
constexpr int kF16 = 2;   // IEEE binary16 (gradients only)

// ---------------------------------------------------------------------------
// 16-bit floats <-> float32 ("BendTorch main.bend", Optimizers: ph_to,
// ph_of_bits for bfloat16)
// ---------------------------------------------------------------------------

// bfloat16 bits (low 16 bits of h) -> float32, exact.
__device__ __forceinline__ float from_bf16(uint32_t h) {
  return __uint_as_float(h << 16);
}

// float32 -> bfloat16, round to nearest, ties to even; any NaN -> 0xFFFF.
__device__ __forceinline__ uint32_t to_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? 0xFFFFu : r;
}

// float32 -> the float32 value of its bfloat16 rounding (low half zero).
__device__ __forceinline__ float round_bf16(float x) {
  return from_bf16(to_bf16(x));
}

// binary16 bits (low 16 bits of h) -> float32, exact (the hardware convert).
__device__ __forceinline__ float from_f16(uint32_t h) {
  return static_cast<float>(
      __builtin_bit_cast(_Float16, static_cast<uint16_t>(h & 0xFFFFu)));
}

// float32 -> binary16 bits, round to nearest, ties to even (the hardware
// convert in the default rounding mode); any NaN -> 0xFFFF, as for bfloat16.
// The empty asm pins x in a register as the float32 value it is: without it
// the compiler fuses a producing multiply and this convert into one
// mixed-precision fma with a +0 addend, which turns a -0 product into +0.
__device__ __forceinline__ uint32_t to_f16(float x) {
  __asm__("" : "+v"(x));
  const uint32_t h =
      __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  return (x != x) ? 0xFFFFu : h;
}

template <int D>
__device__ __forceinline__ float decode16(uint32_t h) {
  if constexpr (D == kBF16) return from_bf16(h & 0xFFFFu);
  else return from_f16(h);
}

template <int D>
__device__ __forceinline__ uint32_t encode16(float x) {
  if constexpr (D == kBF16) return to_bf16(x);
  else return to_f16(x);
}

// Two bfloat16-exact float32 values (low halves zero) -> one packed word,
// the even element in the low half.
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}

// ---------------------------------------------------------------------------
// Loads and stores through global-address-space pointers.  The buffers come
// from the tile records, so without the cast the compiler cannot tell them
// from LDS and would emit flat instructions.  Every tile has a uniform base
// pointer (SGPRs) and each lane a 32-bit element offset, which maps to
// global_load/store with an SGPR base and a VGPR offset.  The vector accesses
// carry the nontemporal hint: every byte is touched once per launch, and on
// gfx950 the streaming hint measured faster for these contiguous-per-wave
// patterns (reads and read-modify-write streams alike).
// ---------------------------------------------------------------------------

#define MTA_GLOBAL __attribute__((address_space(1)))
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int D>
using elem_t = typename std::conditional<D == kF32, float, uint16_t>::type;

template <typename T>
__device__ __forceinline__ MTA_GLOBAL T *gp(const void *p, int64_t elem) {
  return (MTA_GLOBAL T *)(p) + elem;
}

// 4 consecutive elements at element offset e (a multiple of 4) of a
// 16-byte-aligned tile base: a 16-byte store for float32, 8 bytes for
// bfloat16 (values already bfloat16-exact; element 2k in the low half).
template <int D>
__device__ __forceinline__ void store4(MTA_GLOBAL elem_t<D> *p, uint32_t e,
                                       const float (&x)[4]) {
  if constexpr (D == kBF16)
    __builtin_nontemporal_store(u32x2{pack2(x[0], x[1]), pack2(x[2], x[3])},
                                (MTA_GLOBAL u32x2 *)(p + e));
  else
    __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]},
                                (MTA_GLOBAL f32x4 *)(p + e));
}

// 16 bytes per lane: 4 float32 or 8 16-bit elements at offset e, as one raw
// vector, unpacked separately: a loop can issue every load of an iteration
// before it unpacks any of them.
template <int D>
constexpr int kWide = D == kF32 ? 4 : 8;

template <int D>
using raw16_t = typename std::conditional<D == kF32, f32x4, u32x4>::type;

template <int D>
__device__ __forceinline__ raw16_t<D> load16b_raw(MTA_GLOBAL const elem_t<D> *p,
                                                 uint32_t e) {
  return __builtin_nontemporal_load((const MTA_GLOBAL raw16_t<D> *)(p + e));
}

// Keep = true: the same load without the streaming hint, so the line is
// allocated in the caches on its way in (the norm's kept tiles, below).
template <int D, bool Keep>
__device__ __forceinline__ raw16_t<D> load16b(MTA_GLOBAL const elem_t<D> *p,
                                             uint32_t e) {
  if constexpr (Keep) return *((const MTA_GLOBAL raw16_t<D> *)(p + e));
  else return load16b_raw<D>(p, e);
}

template <int D>
__device__ __forceinline__ void unpack16b(const raw16_t<D> &a,
                                          float (&x)[kWide<D>]) {
  if constexpr (D == kF32) {
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  } else {
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = decode16<D>(w[k]);
      x[2 * k + 1] = decode16<D>(w[k] >> 16);
    }
  }
}

template <int D>
__device__ __forceinline__ float load1(MTA_GLOBAL const elem_t<D> *p,
                                       uint32_t e) {
  if constexpr (D == kF32) return p[e];
  else return decode16<D>(p[e]);
}

// Writes one element of a float32 or bfloat16 buffer; a bfloat16 value is
// already bfloat16-exact and goes out as a 16-bit store.
template <int D>
__device__ __forceinline__ void store1(MTA_GLOBAL elem_t<D> *p, uint32_t e,
                                       float x) {
  if constexpr (D == kBF16)
    p[e] = static_cast<uint16_t>(__float_as_uint(x) >> 16);
  else
    p[e] = x;
}

// Element e of a tile of `lim` (>= 1) elements, or 0 past its end.  The
// address is clamped to the tile's last element, so the load is always in
// bounds and needs no branch: every such load of a loop issues back to back.
template <int D>
__device__ __forceinline__ float load1_clamped(MTA_GLOBAL const elem_t<D> *p,
                                               uint32_t e, uint32_t lim) {
  const float x = load1<D>(p, e < lim ? e : lim - 1);
  return e < lim ? x : 0.0f;
}

// This lane's element (j, k) of a tile on the element path, for a kernel
// whose full tiles give each lane V consecutive elements per group j:
// consecutive lanes take consecutive elements, so each single-element
// access instruction of a wave covers one contiguous run and fetches each
// line once.  (The full tiles' mapping would give such an instruction a
// V-element stride across the lanes and touch every line V times: the
// element path then moved its bytes at about half the vector path's rate.)
// Every index is below kTileElems: j*(kBlock*V) + k*kBlock + lane.
template <int V>
__device__ __forceinline__ uint32_t elem_of(int j, int k) {
  return static_cast<uint32_t>(j * (kBlock * V) + k * kBlock) + threadIdx.x;
}

// ---------------------------------------------------------------------------
// The tile stream of a workgroup.  Every kernel walks the tile table with a
// grid stride: stream k takes tiles k, k + grid, k + 2*grid, ...  gfx950
// dispatches workgroups to its 8 XCDs round-robin (workgroup b to XCD b % 8),
// so numbering the streams b itself would give each XCD every 8th tile.
// Workgroup b takes stream (b % 8) * (grid / 8) + b / 8 instead: the
// workgroups of one XCD walk neighbouring tiles, and each XCD's L2 and
// address translation see one contiguous window of every buffer at a time.
// Any one-to-one assignment is correct; this one measured 2.5% faster for
// the AdamW update on a 124M-parameter list.  Grids that are not a multiple
// of 8 keep b.
// ---------------------------------------------------------------------------

constexpr uint32_t kXcds = 8;

__device__ __forceinline__ uint32_t stream_of_block() {
  return (gridDim.x % kXcds)
             ? blockIdx.x
             : (blockIdx.x % kXcds) * (gridDim.x / kXcds) + blockIdx.x / kXcds;
}

// The update kernels are not persistent: workgroup b updates one tile, and
// the grid has one workgroup per tile.  The hardware dispatches workgroups
// in order as earlier ones retire, so the tiles in flight always form one
// narrow window that moves through the list front to back.  (A persistent
// grid-stride walk lets its workgroups drift apart over thousands of
// iterations; the window of open rows widens and the update measured 6-12%
// slower on the 1.56B-parameter lists.)  Within each run of 8 * kXcdRun
// workgroups, XCD x (workgroup b goes to XCD b % 8) takes kXcdRun
// consecutive tiles, so every XCD streams contiguous runs of each buffer:
// measured against plain b -> b, +1% to +5% depending on the list, best at
// runs of 16-32 tiles.  The last partial run keeps b -> b.
constexpr uint32_t kXcdRun = 32;

__device__ __forceinline__ uint32_t tile_of_block() {
  const uint32_t b = blockIdx.x;
  const uint32_t full = gridDim.x / (kXcds * kXcdRun) * (kXcds * kXcdRun);
  if (b >= full) return b;
  const uint32_t x = b % kXcds, k = b / kXcds;
  return (k / kXcdRun) * (kXcds * kXcdRun) + x * kXcdRun + k % kXcdRun;
}

// ---------------------------------------------------------------------------
// b^t rounded to the nearest float64, for step counts that live in device
// memory: square-and-multiply in double-double (a float64 pair whose sum
// carries ~106 bits; every product is exact to that width through fma), so
// the result is the float64 nearest the true power unless it lies within
// ~2^-100 (relative) of a rounding boundary.
// ---------------------------------------------------------------------------

struct DoubleDouble {
  double hi, lo;  // |lo| <= ulp(hi)/2
};

__device__ __forceinline__ DoubleDouble dd_mul(DoubleDouble a,
                                               DoubleDouble b) {
  const double p = a.hi * b.hi;
  double e = fma(a.hi, b.hi, -p);  // exact error of p
  e = fma(a.hi, b.lo, e);
  e = fma(a.lo, b.hi, e);
  const double s = p + e;          // |e| << |p|: fast two-sum
  return DoubleDouble{s, e - (s - p)};
}

__device__ double pow_rn(double b, int64_t t) {
  DoubleDouble r{1.0, 0.0}, x{b, 0.0};
  for (uint64_t k = static_cast<uint64_t>(t); k; k >>= 1) {
    if (k & 1u) r = dd_mul(r, x);
    x = dd_mul(x, x);
  }
  return r.hi;  // hi is the sum hi + lo rounded to nearest
}

// The unscale factor of a loss scale: float32(1 / float64(scale)).
__device__ __forceinline__ float inv_scale(float scale) {
  return static_cast<float>(1.0 / static_cast<double>(scale));
}

// ---------------------------------------------------------------------------
// The element step of each update rule ("BendTorch main.bend", Optimizers),
// with the unscale (ScaleTensors) and the clip coefficient (ClipGradNorms)
// applied in registers first.
//   Adam family: adam_grad, adam_decay (AdamW decays w, Adam adds w*wd to the
//   gradient), adam_m, adam_v, adam_w; packed kinds round the new moment to
//   bfloat16 and the weight update reads the rounded value (adamh_l,
//   adamhv_l).
//   SGD: sgd_l.  Momentum: mom_l (float32 buffer in m).
// ---------------------------------------------------------------------------

template <int R>
constexpr bool kUsesM = R != kRuleSgd;
template <int R>
constexpr bool kUsesV = R == kRuleAdamW || R == kRuleAdam;

template <int R, bool MPacked, bool VPacked>
__device__ __forceinline__ void rule_elem(float &w, float g, float &m,
                                          float &v, const StepScalars &sc,
                                          float coef) {
  const float x = g * sc.s;                          // unscale
  float ge = x * coef;                               // clip
  if constexpr (R == kRuleSgd) {
    w = w + (sc.nstep * ge);                         // sgd_l, nstep = -lr
  } else if constexpr (R == kRuleMomentum) {
    const float nb = (m * sc.mu) + ge;               // mom_l
    m = nb;
    w = w + (sc.nstep * nb);
  } else {
    float wd;
    if constexpr (R == kRuleAdam) {
      ge = ge + (w * sc.l2);                         // adam_grad (Adam)
      wd = w;                                        // adam_decay (Adam)
    } else {
      wd = w * sc.dec;                               // adam_decay (AdamW)
    }
    float m1 = m + sc.c1 * (ge - m);                 // adam_m (lerp form)
    float v1 = (v * sc.b2) + ((sc.c2 * ge) * ge);    // adam_v
    if constexpr (MPacked) m1 = round_bf16(m1);
    if constexpr (VPacked) v1 = round_bf16(v1);
    const float denom = (sqrtf(v1) / sc.bc2) + sc.eps; // adam_w
    w = wd + ((sc.nstep * m1) / denom);
    m = m1;
    v = v1;
  }
}

constexpr int kAdamVec = 4;                                   // per access
constexpr int kAdamGroups = kTileElems / (kBlock * kAdamVec); // 4
constexpr uint32_t kAdamStride = kBlock * kAdamVec;           // 1024

// A workgroup issues every load of its tile as raw vectors first, then
// unpacks and computes: no wait falls between a tile's loads.  At most two
// workgroups run on a CU at a time, so each CU has about two tiles' loads
// in flight while it computes.  The register count alone would let three
// to six fit (130-150 VGPRs for the Adam family, fewer for SGD and
// momentum); the launch reserves kUpdateLdsBytes of LDS per workgroup,
// which no kernel touches, so that only two fit in a CU's 160 KiB.  Three
// or four per CU measured 5-7% slower on the 1.56B-parameter and ragged
// lists and 2-3% slower on the 124M ones; two is as fast or faster for
// every rule.
constexpr unsigned kUpdateLdsBytes = 64u << 10;

// raw vectors of one lane's share of a full tile (4 accesses per buffer)
template <int D>
using raw4_t = typename std::conditional<D == kF32, f32x4, u32x2>::type;

template <int D>
__device__ __forceinline__ raw4_t<D> load4_raw(MTA_GLOBAL const elem_t<D> *p,
                                               uint32_t e) {
  return __builtin_nontemporal_load((const MTA_GLOBAL raw4_t<D> *)(p + e));
}

template <int D>
__device__ __forceinline__ void unpack4(const raw4_t<D> &a, float (&x)[4]) {
  if constexpr (D == kF32) {
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  } else {
    x[0] = decode16<D>(a.x);
    x[1] = decode16<D>(a.x >> 16);
    x[2] = decode16<D>(a.y);
    x[3] = decode16<D>(a.y >> 16);
  }
}

// +0 into 4 consecutive gradient elements (16 or 8 bytes; all-zero bits are
// +0 in every gradient type), or into one.
template <int D>
__device__ __forceinline__ void zero4(MTA_GLOBAL elem_t<D> *p, uint32_t e) {
  if constexpr (D == kF32)
    __builtin_nontemporal_store(f32x4{0.0f, 0.0f, 0.0f, 0.0f},
                                (MTA_GLOBAL f32x4 *)(p + e));
  else
    __builtin_nontemporal_store(u32x2{0u, 0u}, (MTA_GLOBAL u32x2 *)(p + e));
}

template <int D>
__device__ __forceinline__ void zero1(MTA_GLOBAL elem_t<D> *p, uint32_t e) {
  p[e] = elem_t<D>(0);
}

template <int R, int G, bool MPacked, bool VPacked>
struct TileRegs {
  static constexpr int M = MPacked ? kBF16 : kF32;
  static constexpr int V = VPacked ? kBF16 : kF32;
  f32x4 w[kAdamGroups];
  raw4_t<G> g[kAdamGroups];
  raw4_t<M> m[kAdamGroups];  // unused (never written) when the rule has no m
  raw4_t<V> v[kAdamGroups];  // likewise for v
};

template <int G, bool MPacked, bool VPacked>
struct TileRef {
  static constexpr int M = MPacked ? kBF16 : kF32;
  static constexpr int V = VPacked ? kBF16 : kF32;
  MTA_GLOBAL float *pw;
  MTA_GLOBAL elem_t<G> *pg;  // read, and written only when zeroing
  MTA_GLOBAL elem_t<M> *pm;
  MTA_GLOBAL elem_t<V> *pv;
  MTA_GLOBAL uint16_t *pw16;  // 16-bit weight copy, or null
  uint32_t lim;
  bool full;
  bool nodecay;  // the tensor's step takes weight_decay = 0
};

template <int G, bool MPacked, bool VPacked>
__device__ __forceinline__ TileRef<G, MPacked, VPacked> tile_ref(
    const StepTile &st) {
  using Ref = TileRef<G, MPacked, VPacked>;
  Ref r;
  r.pw = gp<float>(st.w, 0);
  r.pg = gp<elem_t<G>>(st.g, 0);
  r.pm = gp<elem_t<Ref::M>>(st.m, 0);
  r.pv = gp<elem_t<Ref::V>>(st.v, 0);
  r.pw16 = gp<uint16_t>(st.w16, 0);
  r.lim = st.lim;
  r.full = (st.flags & kTileVec) && st.lim == kTileElems;
  r.nodecay = (st.flags & kTileNoDecay) != 0;
  return r;
}

template <int R, int G, bool MPacked, bool VPacked>
__device__ __forceinline__ void issue_tile(
    TileRegs<R, G, MPacked, VPacked> &X, const TileRef<G, MPacked, VPacked> &T,
    uint32_t e0) {
  using Ref = TileRef<G, MPacked, VPacked>;
#pragma unroll
  for (int j = 0; j < kAdamGroups; ++j) {
    const uint32_t e = e0 + j * kAdamStride;
    X.w[j] = load4_raw<kF32>(T.pw, e);
    X.g[j] = load4_raw<G>(T.pg, e);
    if constexpr (kUsesM<R>) X.m[j] = load4_raw<Ref::M>(T.pm, e);
    if constexpr (kUsesV<R>) X.v[j] = load4_raw<Ref::V>(T.pv, e);
  }
}

// The 16-bit weight copy ("Mica 7.7", section "float16 and bfloat16,
// whole"): bfloat16 or float16 codes of the new float32 weights, nearest-even,
// NaN -> 0xFFFF.  f16 is uniform (a list has one copy format).
__device__ __forceinline__ uint32_t encode_copy(float x, uint32_t f16) {
  return f16 ? to_f16(x) : to_bf16(x);
}

__device__ __forceinline__ void store_copy4(MTA_GLOBAL uint16_t *p,
                                            uint32_t e, const float (&w)[4],
                                            uint32_t f16) {
  uint32_t h[4];
  if (f16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) h[k] = to_f16(w[k]);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) h[k] = to_bf16(w[k]);
  }
  __builtin_nontemporal_store(u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)},
                              (MTA_GLOBAL u32x2 *)(p + e));
}

template <int R, int G, bool MPacked, bool VPacked>
__device__ __forceinline__ void finish_tile(
    const TileRegs<R, G, MPacked, VPacked> &X,
    const TileRef<G, MPacked, VPacked> &T, uint32_t e0, const StepScalars &sc,
    float coef) {
  using Ref = TileRef<G, MPacked, VPacked>;
#pragma unroll
  for (int j = 0; j < kAdamGroups; ++j) {
    float w[4], g[4], m[4] = {}, v[4] = {};
    unpack4<kF32>(X.w[j], w);
    unpack4<G>(X.g[j], g);
    if constexpr (kUsesM<R>) unpack4<Ref::M>(X.m[j], m);
    if constexpr (kUsesV<R>) unpack4<Ref::V>(X.v[j], v);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      rule_elem<R, MPacked, VPacked>(w[k], g[k], m[k], v[k], sc, coef);
    const uint32_t e = e0 + j * kAdamStride;
    store4<kF32>(T.pw, e, w);
    if constexpr (kUsesM<R>) store4<Ref::M>(T.pm, e, m);
    if constexpr (kUsesV<R>) store4<Ref::V>(T.pv, e, v);
    if (sc.zero) zero4<G>(T.pg, e);  // uniform; after this lane's g load
    if (T.pw16) store_copy4(T.pw16, e, w, sc.copy_f16);  // uniform
  }
}

template <int R, int G, bool MPacked, bool VPacked>
__device__ __forceinline__ void partial_tile(
    const TileRef<G, MPacked, VPacked> &T, const StepScalars &sc,
    float coef) {
  using Ref = TileRef<G, MPacked, VPacked>;
  float w[kAdamGroups][kAdamVec], g[kAdamGroups][kAdamVec],
      m[kAdamGroups][kAdamVec] = {}, v[kAdamGroups][kAdamVec] = {};
#pragma unroll
  for (int j = 0; j < kAdamGroups; ++j)
#pragma unroll
    for (int k = 0; k < kAdamVec; ++k) {
      const uint32_t e = elem_of<kAdamVec>(j, k);
      w[j][k] = load1_clamped<kF32>(T.pw, e, T.lim);
      g[j][k] = load1_clamped<G>(T.pg, e, T.lim);
      if constexpr (kUsesM<R>)
        m[j][k] = load1_clamped<Ref::M>(T.pm, e, T.lim);
      if constexpr (kUsesV<R>)
        v[j][k] = load1_clamped<Ref::V>(T.pv, e, T.lim);
    }
#pragma unroll
  for (int j = 0; j < kAdamGroups; ++j)
#pragma unroll
    for (int k = 0; k < kAdamVec; ++k) {
      rule_elem<R, MPacked, VPacked>(w[j][k], g[j][k], m[j][k], v[j][k], sc,
                                     coef);
      const uint32_t e = elem_of<kAdamVec>(j, k);
      if (e < T.lim) {
        T.pw[e] = w[j][k];
        if constexpr (kUsesM<R>) store1<Ref::M>(T.pm, e, m[j][k]);
        if constexpr (kUsesV<R>) store1<Ref::V>(T.pv, e, v[j][k]);
        if (sc.zero) zero1<G>(T.pg, e);
        if (T.pw16) T.pw16[e] = encode_copy(w[j][k], sc.copy_f16);
      }
    }
}

// +0 into every gradient element of one tile: the whole work of a skipped
// loss-scaled step that was asked to zero the gradients.
template <int G>
__device__ __forceinline__ void zero_grad_tile(const StepTile &st,
                                               uint32_t e0) {
  MTA_GLOBAL elem_t<G> *pg = gp<elem_t<G>>(st.g, 0);
  if ((st.flags & kTileVec) && st.lim == kTileElems) {
#pragma unroll
    for (int j = 0; j < kAdamGroups; ++j) zero4<G>(pg, e0 + j * kAdamStride);
  } else {
#pragma unroll
    for (int j = 0; j < kAdamGroups; ++j)
#pragma unroll
      for (int k = 0; k < kAdamVec; ++k) {
        const uint32_t e = elem_of<kAdamVec>(j, k);
        if (e < st.lim) zero1<G>(pg, e);
      }
  }
}

// The body of every update kernel: the one tile of this workgroup.
template <int R, int G, bool MPacked, bool VPacked>
__device__ __forceinline__ void update_tile(
    const StepTile *__restrict__ tiles, uint32_t ntiles, StepScalars sc,
    const float *__restrict__ d_coef, const AmpStep &amp) {
  using Ref = TileRef<G, MPacked, VPacked>;
  const uint32_t t = tile_of_block();
  if (t >= ntiles) return;  // never, with one workgroup per tile
  const uint32_t e0 = threadIdx.x * kAdamVec;
  const StepTile rec = tiles[t];
  // loss-scaled step: skipped when an unscaled gradient was not finite
  // (zeroing the gradients still happens when asked).  The state is read
  // before any of the tile's traffic.
  float lscale = 1.0f;
  int64_t step = 0;
  if (amp.state) {
    if (amp.state->found_inf != 0.0f) {
      if (sc.zero) zero_grad_tile<G>(rec, e0);
      return;
    }
    lscale = amp.state->scale;
    step = amp.state->step + 1;
  }
  // For the Adam family, t and the two t-dependent constants come from the
  // device state, formed in float64 as the host forms them.  Every
  // workgroup of a launch needs the same two constants; the first ones to
  // run form them (a few hundred float64 operations per lane) and leave
  // them in the list's cache, tagged with the hyperparameters' generation
  // and t; later workgroups find them there.  Each cache word carries its
  // own tag, so a word is used only when it holds this step's value, and a
  // word not yet visible here (a store from another XCD, or one still in
  // flight) only means forming the constants again.  The accesses are
  // therefore workgroup-scope atomics (plain loads and stores through this
  // XCD's L2, never torn): agent-scope ones go past the L2 to memory and
  // made every workgroup wait, 9% of the update on the 124M float16 list.
  // The two cache loads are issued before the tile's loads: loads return in
  // order, so waiting for them later does not wait for the tile.
  uint64_t cache_a = 0, cache_b = 0;
  if constexpr (kUsesV<R>) {
    if (amp.state) {
      cache_a = __hip_atomic_load(amp.cache, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_WORKGROUP);
      cache_b = __hip_atomic_load(amp.cache + 1, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  const float coef = d_coef ? *d_coef : 1.0f;
  const Ref cur = tile_ref<G, MPacked, VPacked>(rec);
  TileRegs<R, G, MPacked, VPacked> X;
  if (cur.full) issue_tile(X, cur, e0);
  __builtin_amdgcn_sched_barrier(0);  // every load in flight first
  if (amp.state) {
    // while the tile's loads are in flight
    if constexpr (kUsesV<R>) {
      const uint64_t tag = (uint64_t{amp.gen} << 24) |
                           (static_cast<uint64_t>(step) & 0xFFFFFFu);
      if ((cache_a >> 32) == tag && (cache_b >> 32) == tag) {
        sc.nstep = __uint_as_float(static_cast<uint32_t>(cache_a));
        sc.bc2 = __uint_as_float(static_cast<uint32_t>(cache_b));
      } else {
        const double q1 = 1.0 - pow_rn(amp.beta1, step);
        const double q2 = 1.0 - pow_rn(amp.beta2, step);
        sc.nstep = -static_cast<float>(amp.lr / q1);
        sc.bc2 = static_cast<float>(sqrt(q2));
        if (threadIdx.x == 0) {
          __hip_atomic_store(amp.cache,
                             (tag << 32) | __float_as_uint(sc.nstep),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          __hip_atomic_store(amp.cache + 1,
                             (tag << 32) | __float_as_uint(sc.bc2),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
    }
    sc.s = inv_scale(lscale);
  }
  // a tensor flagged no-decay takes the step's constants for
  // weight_decay = 0: dec = f32(1 - lr*0) = 1 (AdamW), l2 = 0 (Adam)
  if (cur.nodecay) {
    sc.dec = 1.0f;
    sc.l2 = 0.0f;
  }
  if (cur.full)
    finish_tile(X, cur, e0, sc, coef);
  else
    partial_tile<R>(cur, sc, coef);
}

// AdamW (L2 = false) and Adam with coupled decay (L2 = true).
template <int G, bool MPacked, bool VPacked, bool L2>
__global__ void __launch_bounds__(kBlock)
k_adamw(const StepTile *__restrict__ tiles, uint32_t ntiles, StepScalars sc,
        const float *__restrict__ d_coef, AmpStep amp) {
  update_tile<L2 ? kRuleAdam : kRuleAdamW, G, MPacked, VPacked>(
      tiles, ntiles, sc, d_coef, amp);
}

template <int G>
__global__ void __launch_bounds__(kBlock)
k_sgd(const StepTile *__restrict__ tiles, uint32_t ntiles, StepScalars sc,
      const float *__restrict__ d_coef, AmpStep amp) {
  update_tile<kRuleSgd, G, false, false>(tiles, ntiles, sc, d_coef, amp);
}

template <int G>
__global__ void __launch_bounds__(kBlock)
k_momentum(const StepTile *__restrict__ tiles, uint32_t ntiles,
           StepScalars sc, const float *__restrict__ d_coef, AmpStep amp) {
  update_tile<kRuleMomentum, G, false, false>(tiles, ntiles, sc, d_coef,
                                              amp);
}

// ---------------------------------------------------------------------------
// Joint sum of squares, one launch in two stages.
//   Stage 1 (every workgroup): each thread forms x = f32(g*s), squares it in
//   float64 (exact, and free of the float32 overflow above 1.8e19) and
//   accumulates with a float64 fma; the wave then reduces with DPP lane moves,
//   the four waves combine through LDS, and the workgroup writes one float64
//   partial.
//   Stage 2 (the last workgroup to finish, chosen by a two-level atomic
//   ticket): one wave sums the partials in a fixed lane-strided order, takes
//   the square root, forms the clip coefficient and writes both, then
//   re-arms the ticket counters.
// The grid and the tile order are fixed per list, so the result is the same
// bits on every call.  The float64 sum of the squares of float32 values
// cannot overflow, so the total is finite exactly when every x is.
// ---------------------------------------------------------------------------

// DPP controls (gfx9 encoding): quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_ror:4, row_ror:8.
constexpr int kDppQuadXor1 = 0xB1;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;

template <int Ctrl>
__device__ __forceinline__ double dpp_f64(double x) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(x), Ctrl, 0xF,
                                             0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(x), Ctrl, 0xF,
                                             0xF, false);
  return __hiloint2double(hi, lo);
}

__device__ __forceinline__ double readlane_f64(double x, int lane) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(x), lane);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(x), lane);
  return __hiloint2double(hi, lo);
}

// Sum over the 64 lanes of a fully active wave; every lane gets the result.
__device__ __forceinline__ double wave_sum(double x) {
  x += dpp_f64<kDppQuadXor1>(x);  // pairs
  x += dpp_f64<kDppQuadXor2>(x);  // quads
  x += dpp_f64<kDppRowRor4>(x);   // every lane of a row: 2 quads
  x += dpp_f64<kDppRowRor8>(x);   // every lane of a row: the row's 16 lanes
  return (readlane_f64(x, 0) + readlane_f64(x, 16)) +
         (readlane_f64(x, 32) + readlane_f64(x, 48));
}

// An empty partial slot: a negative signalling NaN.  No arithmetic result
// has these bits (a NaN a float64 operation returns is quiet), so a stored
// partial can never be mistaken for it.
constexpr uint64_t kEmptySlot = kNormSlotEmpty;
// Reloads of one slot before the finishing wave gives up on it (the sum then
// carries the NaN of kEmptySlot).  A store made before the storing
// workgroup's ticket is normally visible by the first load.
constexpr uint32_t kSpinLimit = 1u << 16;

// One grid-stride walk of k_sumsq over tile pairs (t0, t0 + gridDim.x),
// from t0 while t0 < end: two tiles per iteration, their records read one
// iteration ahead (clamped to the last tile: always in bounds).  When both
// tiles are full tiles of aligned tensors (the common case) all their loads
// are issued as raw 16-byte vectors before any is unpacked; otherwise each
// tile goes on its own, a tail tile through clamped one-element loads.
// Keep selects the vector loads' cache policy; the kernel runs one walk of
// each kind, one after the other, so each is its own loop (the compiler
// would merge two policies behind one branch into one load and drop the
// streaming hint).
template <int D, bool Keep>
__device__ __forceinline__ void sumsq_walk(
    const GradTile *__restrict__ tiles, uint32_t ntiles, uint32_t end,
    uint32_t &t0, GradTile (&rec)[2],
    double (&acc)[kTileElems / (kBlock * kWide<D>)], float s) {
  constexpr int V = kWide<D>;
  constexpr int G = kTileElems / (kBlock * V);
  constexpr int U = 2;
  const uint32_t last = ntiles ? ntiles - 1 : 0;
  const uint32_t stride = U * gridDim.x;
  const uint32_t e0 = threadIdx.x * V;
  for (; t0 < end; t0 += stride) {
    GradTile cur[U];
    bool valid[U];
    bool all_full = true;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      cur[u] = rec[u];
      valid[u] = t0 + u * gridDim.x < ntiles;
      all_full = all_full && valid[u] && cur[u].vec &&
                 cur[u].lim == kTileElems;
    }
    if (all_full) {
      raw16_t<D> r[U][G];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < G; ++j)
          r[u][j] = load16b<D, Keep>(gp<elem_t<D>>(cur[u].g, j * (kBlock * V)),
                                     e0);
      // the next records only after the vector loads (scalar loads return
      // out of order: an earlier one would be waited for with these)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U; ++u)
        rec[u] = tiles[min(t0 + stride + u * gridDim.x, last)];
      __builtin_amdgcn_sched_barrier(0);  // every load in flight first
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < G; ++j) {
          float x[V];
          unpack16b<D>(r[u][j], x);
#pragma unroll
          for (int k = 0; k < V; ++k) {
            const double xs = static_cast<double>(x[k] * s);
            acc[j] = fma(xs, xs, acc[j]);
          }
        }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u)
        rec[u] = tiles[min(t0 + stride + u * gridDim.x, last)];
      // unrolled: indexing cur[] with a loop variable would move the
      // records out of scalar registers
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (!valid[u]) continue;
        MTA_GLOBAL const elem_t<D> *pg = gp<elem_t<D>>(cur[u].g, 0);
        const uint32_t lim = cur[u].lim;
        float x[G][V];
        if (cur[u].vec && lim == kTileElems) {
#pragma unroll
          for (int j = 0; j < G; ++j)
            unpack16b<D>(load16b<D, Keep>(pg + j * (kBlock * V), e0), x[j]);
        } else {
#pragma unroll
          for (int j = 0; j < G; ++j)
#pragma unroll
            for (int k = 0; k < V; ++k)
              x[j][k] = load1_clamped<D>(pg, elem_of<V>(j, k), lim);
        }
#pragma unroll
        for (int j = 0; j < G; ++j)
#pragma unroll
          for (int k = 0; k < V; ++k) {
            const double xs = static_cast<double>(x[j][k] * s);
            acc[j] = fma(xs, xs, acc[j]);
          }
      }
    }
  }
}

// Tiles from keep_from on are the list's last gradient bytes, up to what
// the device's memory-side cache holds: the norm reads them with allocating
// loads so the update launch that follows, which reads the same gradients
// last, finds them there instead of in HBM.  Earlier tiles stream.
template <int D>
__global__ void __launch_bounds__(kBlock)
k_sumsq(const GradTile *__restrict__ tiles, uint32_t ntiles,
        uint32_t keep_from, float s, float max_norm,
        double *__restrict__ partials, unsigned int *__restrict__ ticket,
        const double *acc_in, double *acc_out, float *__restrict__ d_norm,
        float *__restrict__ d_coef, mta_amp_state *__restrict__ amp) {
  constexpr int V = kWide<D>;
  constexpr int G = kTileElems / (kBlock * V);
  if (amp) s = inv_scale(amp->scale);  // loss-scaled: unscale by 1/scale
  constexpr int U = 2;
  const uint32_t last = ntiles ? ntiles - 1 : 0;
  double acc[G] = {};
  uint32_t t0 = stream_of_block();
  GradTile rec[U];
  if (ntiles) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      rec[u] = tiles[min(t0 + u * gridDim.x, last)];
  }
  // a pair streams when both its tiles lie before keep_from (a tile past
  // the end counts as before it)
  const uint32_t reach = (U - 1) * gridDim.x;
  const uint32_t split = keep_from >= ntiles  ? ntiles
                         : keep_from > reach ? keep_from - reach
                                             : 0;
  sumsq_walk<D, false>(tiles, ntiles, min(split, ntiles), t0, rec, acc, s);
  sumsq_walk<D, true>(tiles, ntiles, ntiles, t0, rec, acc, s);
  double mine = acc[0];
#pragma unroll
  for (int j = 1; j < G; ++j) mine += acc[j];

  __shared__ double wave_part[kBlock / 64];
  __shared__ bool is_last;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const double wsum = wave_sum(mine);
  if (lane == 0) wave_part[wave] = wsum;
  __syncthreads();
  // Each partial slot is its own flag: an agent-scope atomic holding
  // kEmptySlot until this workgroup's partial is stored into it.  No release
  // fence is needed (a fence per workgroup costs ~47 ns, serialized across
  // the grid); the ticket only elects the finishing workgroup.
  uint64_t *const slots = reinterpret_cast<uint64_t *>(partials);
  if (threadIdx.x == 0) {
    const double part = (wave_part[0] + wave_part[1]) +
                        (wave_part[2] + wave_part[3]);
    __hip_atomic_store(slots + blockIdx.x,
                       static_cast<uint64_t>(__double_as_longlong(part)),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // two-level ticket: workgroup b counts in group b % kTicketGroups; the
    // workgroup that completes its group counts at the top, and the one
    // that completes the top finishes.  Eight counters on their own lines
    // take the burst of atomics of workgroups that end together in
    // parallel instead of one after another.
    const uint32_t grp = blockIdx.x % kTicketGroups;
    const uint32_t members =
        (gridDim.x - grp + kTicketGroups - 1) / kTicketGroups;
    bool last = false;
    if (__hip_atomic_fetch_add(ticket + grp * kTicketStride, 1u,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
        members - 1) {
      const uint32_t groups = min(gridDim.x, kTicketGroups);
      last = __hip_atomic_fetch_add(ticket + kTicketGroups * kTicketStride,
                                    1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT) == groups - 1;
    }
    is_last = last;
  }
  __syncthreads();
  if (!is_last) return;

  // Stage 2: the finishing wave.  Every other workgroup has stored its
  // partial (each did so before taking its ticket), but a store may not be
  // visible yet: lane l reads slots l, l+64, ... with atomic loads and
  // reloads a slot that still holds kEmptySlot, at most kSpinLimit times,
  // then sums them in that order and re-arms each slot for the next call.
  // kEmptySlot is a NaN, so a partial that never arrived makes the norm NaN:
  // loud, never silent.
  if (wave != 0) return;
  constexpr int kBatch = 8;
  double a = 0.0;
  for (uint32_t i0 = 0; i0 < gridDim.x; i0 += 64 * kBatch) {
    uint64_t raw[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const uint32_t i = i0 + q * 64 + lane;
      raw[q] = i < gridDim.x
                   ? __hip_atomic_load(slots + i, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT)
                   : 0ull;  // the bits of +0.0
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const uint32_t i = i0 + q * 64 + lane;
      for (uint32_t spin = 0; raw[q] == kEmptySlot && spin < kSpinLimit;
           ++spin)
        raw[q] = __hip_atomic_load(slots + i, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
      a += __longlong_as_double(static_cast<long long>(raw[q]));
      if (i < gridDim.x)
        __hip_atomic_store(slots + i, kEmptySlot, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  double total = wave_sum(a);
  if (lane == 0) {
    // a norm over several lists: the earlier lists' total comes first
    // (acc_in and acc_out may be one address: read, then written)
    if (acc_in) total = *acc_in + total;
    if (acc_out) *acc_out = total;
    const float nrm = static_cast<float>(sqrt(total));
    // PyTorch's clip_grad_norm_: max / (norm + 1e-6), clamped at 1; the
    // comparison lets a NaN through and an infinite norm gives 0.
    const float c = max_norm / (nrm + 1e-6f);
    if (d_norm) *d_norm = nrm;
    *d_coef = (c > 1.0f) ? 1.0f : c;
    if (amp) amp->found_inf = isfinite(total) ? 0.0f : 1.0f;
    // every workgroup has counted by now: re-arm every counter
    for (uint32_t k = 0; k <= kTicketGroups; ++k)
      __hip_atomic_store(ticket + k * kTicketStride, 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------------------
// ScaleTensors in place: g = g * s, a 16-bit gradient rounded back to its
// type (nearest-even; NaN -> 0xFFFF).
// ---------------------------------------------------------------------------

// g = f32(g * s), rounded back to g's type, for one tile of a full,
// aligned tensor whose loads are already in r.
template <int D>
__device__ __forceinline__ void scale_store_tile(
    MTA_GLOBAL elem_t<D> *pg, const raw16_t<D> (&r)[kTileElems /
                                                   (kBlock * kWide<D>)],
    uint32_t e0, float s) {
  constexpr int V = kWide<D>;
  constexpr int G = kTileElems / (kBlock * V);
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float x[V];
    unpack16b<D>(r[j], x);
    MTA_GLOBAL elem_t<D> *q = pg + j * (kBlock * V) + e0;
    if constexpr (D == kF32) {
      __builtin_nontemporal_store(
          f32x4{x[0] * s, x[1] * s, x[2] * s, x[3] * s},
          (MTA_GLOBAL f32x4 *)q);
    } else {
      uint32_t h[V];
#pragma unroll
      for (int k = 0; k < V; ++k) h[k] = encode16<D>(x[k] * s);
      __builtin_nontemporal_store(
          u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16),
                h[4] | (h[5] << 16), h[6] | (h[7] << 16)},
          (MTA_GLOBAL u32x4 *)q);
    }
  }
}

// The same for any tile: clamped element loads (all issued first) and
// masked element stores, or the vector path for a full aligned tile.
template <int D>
__device__ __forceinline__ void scale_any_tile(const GradTile &tl, uint32_t e0,
                                               float s) {
  constexpr int V = kWide<D>;
  constexpr int G = kTileElems / (kBlock * V);
  MTA_GLOBAL elem_t<D> *pg = gp<elem_t<D>>(const_cast<void *>(tl.g), 0);
  const uint32_t lim = tl.lim;
  if (tl.vec && lim == kTileElems) {
    raw16_t<D> r[G];
#pragma unroll
    for (int j = 0; j < G; ++j) r[j] = load16b_raw<D>(pg + j * (kBlock * V), e0);
    scale_store_tile<D>(pg, r, e0, s);
    return;
  }
  float x[G][V];
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int k = 0; k < V; ++k)
      x[j][k] = load1_clamped<D>(pg, elem_of<V>(j, k), lim);
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int k = 0; k < V; ++k) {
      const uint32_t e = elem_of<V>(j, k);
      if (e < lim) {
        const float y = x[j][k] * s;
        if constexpr (D == kF32)
          pg[e] = y;
        else
          pg[e] = static_cast<uint16_t>(encode16<D>(y));
      }
    }
}

// One workgroup per tile, in the update kernels' dispatch order (runs of
// kXcdRun tiles per XCD): the workgroup loads its tile, scales it and
// stores it, and the hardware hands out tiles in order as workgroups
// retire.  The launch reserves kScaleLdsBytes<D> of LDS per workgroup, which
// no code touches, so that two workgroups fit on a CU for float32
// gradients and four for 16-bit ones (half the bytes per tile, so twice the
// workgroups for the same bytes in flight).  Measured against the earlier
// persistent two-tile walk (alternating in one process): 5.94 -> 6.61 TB/s
// on the 124M float32 gradients, 5.32 -> 6.54 on the 1.56B ones, 5.55 ->
// 6.60 on the 124M bfloat16 ones and 5.27 -> 6.63 on the 10,002-tensor
// bfloat16 list; without the cap 6.10, 5.81, 6.50 and 6.46, with 2/CU for
// 16-bit gradients 5.31 and 5.15.
template <int D>
constexpr unsigned kScaleLdsBytes = D == kF32 ? (64u << 10) : (40u << 10);

template <int D>
__global__ void __launch_bounds__(kBlock)
k_scale(const GradTile *__restrict__ tiles, uint32_t ntiles, float s,
        const float *__restrict__ d_s) {
  if (d_s) s = *d_s;  // a factor in device memory, read once per workgroup
  const uint32_t t = tile_of_block();  // grid == ntiles: always a tile
  (void)ntiles;
  const GradTile rec = tiles[t];
  scale_any_tile<D>(rec, threadIdx.x * kWide<D>, s);
}

// ---------------------------------------------------------------------------
// The loss-scale update after a step (reading: PyTorch's GradScaler.update):
// a step with a non-finite unscaled gradient backs the scale off and resets
// the tracker; otherwise the step counts, the tracker grows, and every
// `interval` good steps the scale grows when the grown scale is finite.
// Products in float64, rounded once to float32.  The flag is cleared.
// ---------------------------------------------------------------------------

__global__ void k_amp_update(mta_amp_state *__restrict__ st, double growth,
                             double backoff, int32_t interval) {
  if (blockIdx.x != 0 || threadIdx.x != 0) return;
  if (st->found_inf != 0.0f) {
    st->scale = static_cast<float>(static_cast<double>(st->scale) * backoff);
    st->growth_tracker = 0;
  } else {
    st->step += 1;
    const int32_t good = st->growth_tracker + 1;
    if (good == interval) {
      const float grown =
          static_cast<float>(static_cast<double>(st->scale) * growth);
      if (isfinite(grown)) st->scale = grown;
      st->growth_tracker = 0;
    } else {
      st->growth_tracker = good;
    }
  }
  st->found_inf = 0.0f;
}

template <int G, bool M, bool V, bool L2>
hipError_t launch_adamw_t(const Work &wk, const StepScalars &sc,
                          const float *d_coef, const AmpStep &amp) {
  hipLaunchKernelGGL((k_adamw<G, M, V, L2>), dim3(wk.grid), dim3(kBlock),
                     kUpdateLdsBytes, wk.stream, wk.stiles, wk.ntiles, sc,
                     d_coef, amp);
  return hipGetLastError();
}

template <int G, bool L2>
hipError_t launch_adamw_g(int mkind, int vkind, const Work &wk,
                          const StepScalars &sc, const float *d_coef,
                          const AmpStep &amp) {
  switch ((mkind << 1) | vkind) {
    case 0: return launch_adamw_t<G, false, false, L2>(wk, sc, d_coef, amp);
    case 1: return launch_adamw_t<G, false, true, L2>(wk, sc, d_coef, amp);
    case 2: return launch_adamw_t<G, true, false, L2>(wk, sc, d_coef, amp);
    case 3: return launch_adamw_t<G, true, true, L2>(wk, sc, d_coef, amp);
    default: return hipErrorInvalidValue;
  }
}

template <int G>
hipError_t launch_update_g(int rule, int mkind, int vkind, const Work &wk,
                           const StepScalars &sc, const float *d_coef,
                           const AmpStep &amp) {
  switch (rule) {
    case kRuleAdamW:
      return launch_adamw_g<G, false>(mkind, vkind, wk, sc, d_coef, amp);
    case kRuleAdam:
      return launch_adamw_g<G, true>(mkind, vkind, wk, sc, d_coef, amp);
    case kRuleSgd:
      hipLaunchKernelGGL((k_sgd<G>), dim3(wk.grid), dim3(kBlock),
                         kUpdateLdsBytes, wk.stream, wk.stiles, wk.ntiles, sc,
                         d_coef, amp);
      return hipGetLastError();
    case kRuleMomentum:
      if (mkind != 0) return hipErrorInvalidValue;  // float32 buffer only
      hipLaunchKernelGGL((k_momentum<G>), dim3(wk.grid), dim3(kBlock),
                         kUpdateLdsBytes, wk.stream, wk.stiles, wk.ntiles, sc,
                         d_coef, amp);
      return hipGetLastError();
    default:
      return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t launch_sumsq_t(const Work &wk, float s, float max_norm,
                          NormScratch scr, float *d_norm, float *d_coef,
                          mta_amp_state *amp) {
  hipLaunchKernelGGL((k_sumsq<D>), dim3(wk.grid), dim3(kBlock), 0, wk.stream,
                     wk.gtiles, wk.ntiles, wk.keep_from, s, max_norm,
                     scr.partials, scr.ticket, scr.acc_in, scr.acc_out,
                     d_norm, d_coef, amp);
  return hipGetLastError();
}

template <int D>
hipError_t launch_scale_t(const Work &wk, float s, const float *d_s) {
  // one workgroup per tile (the caller never launches an empty list)
  hipLaunchKernelGGL((k_scale<D>), dim3(wk.ntiles), dim3(kBlock),
                     kScaleLdsBytes<D>, wk.stream, wk.gtiles, wk.ntiles, s,
                     d_s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_update(int rule, int gtype, int mkind, int vkind,
                         const Work &wk, const StepScalars &sc,
                         const float *d_coef, const AmpStep &amp) {
  switch (gtype) {
    case kF32:
      return launch_update_g<kF32>(rule, mkind, vkind, wk, sc, d_coef, amp);
    case kBF16:
      return launch_update_g<kBF16>(rule, mkind, vkind, wk, sc, d_coef, amp);
    case kF16:
      return launch_update_g<kF16>(rule, mkind, vkind, wk, sc, d_coef, amp);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_sumsq(int gtype, const Work &wk, float s, float max_norm,
                        NormScratch scr, float *d_norm, float *d_coef,
                        mta_amp_state *amp) {
  switch (gtype) {
    case kF32: return launch_sumsq_t<kF32>(wk, s, max_norm, scr, d_norm, d_coef, amp);
    case kBF16: return launch_sumsq_t<kBF16>(wk, s, max_norm, scr, d_norm, d_coef, amp);
    case kF16: return launch_sumsq_t<kF16>(wk, s, max_norm, scr, d_norm, d_coef, amp);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_scale(int gtype, const Work &wk, float s,
                        const float *d_s) {
  switch (gtype) {
    case kF32: return launch_scale_t<kF32>(wk, s, d_s);
    case kBF16: return launch_scale_t<kBF16>(wk, s, d_s);
    case kF16: return launch_scale_t<kF16>(wk, s, d_s);
    default: return hipErrorInvalidValue;
  }
}

// The scratch of mta_clip_norm_noalloc, for callers that cannot allocate
// device memory: one copy per device, held until the process ends.  In
// host code `scratch` names a host-side stand-in, not device memory: only
// the address hipGetSymbolAddress returns for the current device is ever
// passed to a kernel or a copy.
namespace {
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(int device, void **out) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void *ptr = nullptr;
    const hipError_t e =
        hipGetSymbolAddress(reinterpret_cast<void **>(&ptr),
                            HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[device] = ptr;
  }
  *out = g_scratch_ptr[device];
  return hipSuccess;
}

hipError_t launch_amp_update(mta_amp_state *st, double growth, double backoff,
                             int32_t interval, hipStream_t stream) {
  hipLaunchKernelGGL(k_amp_update, dim3(1), dim3(64), 0, stream, st, growth,
                     backoff, interval);
  return hipGetLastError();
}

}  // namespace mta
