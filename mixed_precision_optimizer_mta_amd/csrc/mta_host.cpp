// mta_host.cpp -- host runtime and C ABI of libmta (see include/mta.h).
//
// Validation, the per-list device tables (one record per tile),
// the float64 -> float32 scalar preparation of each AdamW step, the launch
// policy, and error reporting.  No C++ exception crosses the ABI.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/mta.h"
#include "mta_internal.h"

struct mta_list {
  std::vector<mta_tensor> tensors;  // the caller's table, kept for rebuilds
  std::vector<void *> w16;          // attached 16-bit weight copies (or null)
  std::vector<uint8_t> no_decay;    // 1: the tensor takes weight_decay = 0
                                    // (empty: none is flagged)
  int device = 0;
  int gtype = 0, mkind = 0, vkind = 0;
  int64_t count = 0;
  int64_t elements = 0;
  uint32_t ntiles = 0;
  uint32_t keep_from = 0;  // first tile the norm reads with allocating loads
  int cus = 1;          // compute units of the device
  int grid_update = 1;  // workgroups of an update launch
  uint32_t max_grid = mta::kMaxTileGrid;  // most tiles in one per-tile
                                          // launch
  int grid_norm = 1;    // workgroups of a norm launch
  int state_buffers = 3;  // bit 0: tensors have m; bit 1: they have v
  bool has_w = true;      // false: a gradient-only list (no w, m, v)
  int vector_tensors = 0;
  void *dev_block = nullptr;  // one allocation: tile tables, norm scratch
  mta::GradTile *d_gtiles = nullptr;
  mta::StepTile *d_stiles = nullptr;
  double *d_partials = nullptr;
  unsigned int *d_ticket = nullptr;
  double *d_acc = nullptr;  // running total of a norm over several lists
  uint64_t *d_amp_cache = nullptr;  // loss-scaled step constants (kernels)
  uint32_t amp_gen = 0;             // generation of amp_hp (1..255)
  double amp_hp[3] = {0, 0, 0};     // lr, beta1, beta2 of the last
                                    // loss-scaled step on this list
  int weight_copies = 0;  // tensors with an attached 16-bit copy
  int no_decay_tensors = 0;  // tensors flagged by mta_list_set_no_decay
  int copy_type = MTA_BF16;  // format of the copies: MTA_BF16 or MTA_F16
  bool deferred = false;  // a MTA_SCALE_DEFER factor is pending
  float deferred_s = 1.0f;
};

// Layouts the ABI fixes (include/mta.h, MTA_ABI_VERSION 2).
static_assert(sizeof(mta_tensor) == 40, "mta_tensor layout");
static_assert(sizeof(mta_list_info_t) == 72, "mta_list_info_t layout");
static_assert(sizeof(mta_opt) == 56, "mta_opt layout");

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return MTA_OK;
}

int env_int(const char *name, int dflt, int lo, int hi) {
  const char *s = std::getenv(name);
  if (!s || !*s) return dflt;
  char *end = nullptr;
  long v = std::strtol(s, &end, 10);
  if (*end != '\0' || v < lo || v > hi) return dflt;
  return static_cast<int>(v);
}

bool debug_sync() {
  static const bool on = env_int("MTA_DEBUG_SYNC", 0, 0, 1) == 1;
  return on;
}

// Launch shapes.  A workgroup is four wave64s.  The update kernels and the
// in-place scale launch one workgroup per tile (the hardware hands tiles
// out in order; see the kernels).  The norm is a persistent grid that walks
// the tile table with a grid stride, two tiles of loads in flight per
// workgroup: one workgroup per CU for float32 gradients, two for 16-bit
// ones (half the bytes per tile, so twice the workgroups for the same bytes
// in flight).  Measured on gfx950 (MI355X).
constexpr int kNormBlocksPerCuF32 = 1;
constexpr int kNormBlocksPerCu16 = 2;

// Gradient bytes, at the end of the list, that the norm reads with
// allocating loads so that the memory-side cache (256 MiB on MI355X) still
// holds them when the update reads them again.  The update's full tiles
// stream past that cache (their accesses carry the nontemporal hint), so the
// kept lines survive however far it walks before reaching them: 1.6 GB on
// the 124M float32 list, 31 GB on the 1.56B one.  What evicts them is the
// update's element path (tail tiles and tensors off 16-byte alignment, read
// and written with plain, allocating accesses): tiles are kept only while
// that traffic before the kept tiles stays under kNormKeepElemMiB, a
// quarter of the cache.  The 10,002-tensor list, with 240 MB of it, loses
// 2.4% when keeping; the GPT-2 lists (under 10 MB) gain 0.4-5%.
// MTA_NORM_KEEP_MIB sets the budget for any list at list creation (0:
// every norm load streams).
constexpr int kNormKeepMiB = 256;
constexpr int64_t kNormKeepElemMiB = 64;

int after_launch(hipError_t e, hipStream_t stream, const char *what) {
  if (e != hipSuccess)
    return fail(MTA_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  if (debug_sync()) {
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess)
      return fail(MTA_EHIP, "%s: kernel failed: %s", what,
                  hipGetErrorString(e));
  }
  return ok();
}

int check_device(const mta_list *L) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(MTA_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev != L->device)
    return fail(MTA_EINVAL,
                "list lives on device %d but device %d is current", L->device,
                dev);
  return MTA_OK;
}

bool aligned(const void *p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// PyTorch's AdamW argument checks, plus t >= 1 (the first step is t = 1).
int check_hparams(const mta_adamw_hparams *hp, int64_t t) {
  if (!hp) return fail(MTA_EINVAL, "hparams is NULL");
  if (!(std::isfinite(hp->lr) && hp->lr >= 0.0))
    return fail(MTA_EINVAL, "lr must be finite and >= 0 (got %g)", hp->lr);
  if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0))
    return fail(MTA_EINVAL, "beta1 must be in [0, 1) (got %g)", hp->beta1);
  if (!(hp->beta2 >= 0.0 && hp->beta2 < 1.0))
    return fail(MTA_EINVAL, "beta2 must be in [0, 1) (got %g)", hp->beta2);
  if (!(std::isfinite(hp->eps) && hp->eps >= 0.0))
    return fail(MTA_EINVAL, "eps must be finite and >= 0 (got %g)", hp->eps);
  if (!(std::isfinite(hp->weight_decay) && hp->weight_decay >= 0.0))
    return fail(MTA_EINVAL, "weight_decay must be finite and >= 0 (got %g)",
                hp->weight_decay);
  if (t < 1) return fail(MTA_EINVAL, "step t must be >= 1 (got %lld)",
                         static_cast<long long>(t));
  return MTA_OK;
}

// The step's float32 constants, each formed in float64 and rounded once:
// bias corrections 1 - beta^t from pow (as Python's beta ** t), the step size
// lr / (1 - beta1^t) and sqrt(1 - beta2^t) ("BendTorch main.bend": Opt type
// comment and Opt.at; Training section for q1, q2), 1 - beta formed in
// float64 (comment on adam_m), and the decoupled decay factor 1 - lr*wd.
void make_scalars(const mta_adamw_hparams &hp, int64_t t, float out[7]) {
  const double td = static_cast<double>(t);
  const double bias1 = 1.0 - std::pow(hp.beta1, td);
  const double bias2 = 1.0 - std::pow(hp.beta2, td);
  out[0] = static_cast<float>(hp.lr / bias1);
  out[1] = static_cast<float>(std::sqrt(bias2));
  out[2] = static_cast<float>(1.0 - hp.beta1);
  out[3] = static_cast<float>(1.0 - hp.beta2);
  out[4] = static_cast<float>(hp.beta2);
  out[5] = static_cast<float>(hp.eps);
  out[6] = static_cast<float>(1.0 - hp.lr * hp.weight_decay);
}

// The kernel's scalar block for step t (t-independent entries are the same
// for every t, so a loss-scaled step replaces only nstep, bc2 and s).
mta::StepScalars step_scalars(const mta_adamw_hparams &hp, int64_t t) {
  float c[7];
  make_scalars(hp, t, c);
  mta::StepScalars sc{};
  sc.nstep = -c[0];
  sc.bc2 = c[1];
  sc.c1 = c[2];
  sc.c2 = c[3];
  sc.b2 = c[4];
  sc.eps = c[5];
  sc.dec = c[6];
  sc.s = 1.0f;
  return sc;
}

struct Span {
  uintptr_t lo, hi;
  int64_t tensor;
  int which;
};

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Sorts the spans and fails on the first two that overlap.
int check_overlaps(std::vector<Span> *spans) {
  std::sort(spans->begin(), spans->end(),
            [](const Span &a, const Span &b) { return a.lo < b.lo; });
  static const char *names[5] = {"w", "g", "m", "v", "w16"};
  for (size_t k = 1; k < spans->size(); ++k) {
    const Span &a = (*spans)[k - 1], &b = (*spans)[k];
    if (b.lo < a.hi)
      return fail(MTA_EINVAL,
                  "buffers overlap: tensor %lld %s and tensor %lld %s",
                  static_cast<long long>(a.tensor), names[a.which],
                  static_cast<long long>(b.tensor), names[b.which]);
  }
  return MTA_OK;
}

// The byte ranges of every buffer of the list's non-empty tensors.
void list_spans(const mta_list *L, std::vector<Span> *spans) {
  const uintptr_t sizes[4] = {4, L->gtype == MTA_F32 ? 4u : 2u,
                              L->mkind == MTA_MOM_BF16X2 ? 2u : 4u,
                              L->vkind == MTA_MOM_BF16X2 ? 2u : 4u};
  for (size_t i = 0; i < L->tensors.size(); ++i) {
    const mta_tensor &x = L->tensors[i];
    if (x.n == 0) continue;
    const void *bufs[4] = {x.w, x.g, x.m, x.v};
    for (int b = 0; b < 4; ++b) {
      if (!bufs[b]) continue;  // a state buffer the list does not have
      const uintptr_t lo = reinterpret_cast<uintptr_t>(bufs[b]);
      spans->push_back(Span{lo, lo + static_cast<uintptr_t>(x.n) * sizes[b],
                            static_cast<int64_t>(i), b});
    }
  }
}

uintptr_t elem_size(int kind_is_16bit) { return kind_is_16bit ? 2 : 4; }

// Elements to take off the front of a tensor so that every buffer it has is
// aligned from there on: the smallest h < 64 that puts all of them on a
// 128-byte cache-line boundary, else the smallest h < 8 that makes all of
// them 16-byte aligned, else -1 (their misalignments disagree).  Elements
// are 2 or 4 bytes and each buffer is aligned to its element size, so a
// buffer's offset mod 128 repeats every 64 elements and mod 16 every 8.
// Line-aligned tiles keep every wave's stores to whole cache lines, as in
// a tensor that starts on one.
int64_t vector_peel(const mta_tensor &x, int gtype, int mkind, int vkind) {
  const void *bufs[4] = {x.w, x.g, x.m, x.v};
  const uintptr_t sizes[4] = {4, elem_size(gtype != MTA_F32),
                              elem_size(mkind == MTA_MOM_BF16X2),
                              elem_size(vkind == MTA_MOM_BF16X2)};
  const auto first = [&](uintptr_t period, uintptr_t align) -> int64_t {
    for (uintptr_t h = 0; h < period; ++h) {
      bool ok = true;
      for (int b = 0; b < 4 && ok; ++b)
        ok = !bufs[b] ||
             (reinterpret_cast<uintptr_t>(bufs[b]) + h * sizes[b]) % align ==
                 0;
      if (ok) return static_cast<int64_t>(h);
    }
    return -1;
  };
  const int64_t line = first(64, 128);
  return line >= 0 ? line : first(8, 16);
}

// Tiles of a tensor of n > 0 elements with vector_peel h: a head tile of h
// elements when 0 < h < n, then whole tiles from there.
uint64_t tiles_of(int64_t n, int64_t h) {
  const uint64_t head = (h > 0) ? static_cast<uint64_t>(h < n ? h : n) : 0;
  const uint64_t rest = static_cast<uint64_t>(n) - head;
  return (head ? 1 : 0) + (rest + mta::kTileElems - 1) / mta::kTileElems;
}

// One StepTile per tile of every non-empty tensor, in list order.  w16 may be
// empty (no copies) or hold one pointer per tensor; no_decay likewise (empty:
// every tensor decays).  The tile cuts depend on w, g, m, v only, so
// attaching copies or flags never changes the tile count; a copy that is not
// 16-byte aligned at the vector tiles' starts sends the tensor down the
// element path.
void build_step_tiles(const std::vector<mta_tensor> &tensors,
                      const std::vector<void *> &w16,
                      const std::vector<uint8_t> &no_decay, int gtype,
                      int mkind, int vkind, std::vector<mta::StepTile> *out) {
  const uintptr_t gsz = elem_size(gtype != MTA_F32);
  const uintptr_t msz = elem_size(mkind == MTA_MOM_BF16X2);
  const uintptr_t vsz = elem_size(vkind == MTA_MOM_BF16X2);
  out->clear();
  for (size_t i = 0; i < tensors.size(); ++i) {
    const mta_tensor &x = tensors[i];
    if (x.n == 0) continue;
    void *copy = w16.empty() ? nullptr : w16[i];
    const uint32_t nd =
        (!no_decay.empty() && no_decay[i]) ? mta::kTileNoDecay : 0u;
    const int64_t peel = vector_peel(x, gtype, mkind, vkind);
    const int64_t head = peel > 0 ? std::min(peel, x.n) : 0;
    const bool vec =
        peel >= 0 &&
        (!copy || (reinterpret_cast<uintptr_t>(copy) + head * 2) % 16 == 0);
    const auto push = [&](int64_t base, int64_t lim, bool v) {
      const uintptr_t b = static_cast<uintptr_t>(base);
      const auto at = [b](const void *p, uintptr_t size) -> void * {
        return p ? reinterpret_cast<char *>(const_cast<void *>(p)) + b * size
                 : nullptr;
      };
      mta::StepTile st;
      st.w = static_cast<float *>(at(x.w, 4));
      st.g = at(x.g, gsz);
      st.m = at(x.m, msz);
      st.v = at(x.v, vsz);
      st.lim = static_cast<uint32_t>(lim);
      st.flags = (v ? mta::kTileVec : 0u) | nd;
      st.w16 = at(copy, 2);
      out->push_back(st);
    };
    if (head > 0) push(0, head, false);
    for (int64_t base = head; base < x.n; base += mta::kTileElems) {
      const int64_t left = x.n - base;
      push(base, left < mta::kTileElems ? left : mta::kTileElems, vec);
    }
  }
}

// Rebuild the list's step tile table with these weight copies and no-decay
// flags and upload it on `stream`, waiting for the copy (the host table dies
// with this call).  Nothing of the handle changes; the caller commits the
// new copies and flags once this succeeds.
int upload_step_tiles(mta_list *L, const std::vector<void *> &w16,
                      const std::vector<uint8_t> &no_decay, void *stream) {
  int rc = check_device(L);
  if (rc) return rc;
  std::vector<mta::StepTile> stiles;
  try {
    build_step_tiles(L->tensors, w16, no_decay, L->gtype, L->mkind, L->vkind,
                     &stiles);
  } catch (const std::bad_alloc &) {
    return fail(MTA_ENOMEM, "host allocation failed");
  }
  if (stiles.size() != L->ntiles)  // the cuts depend on w, g, m, v only
    return fail(MTA_EINVAL, "internal: the tile count changed");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (!stiles.empty())
    e = hipMemcpyAsync(L->d_stiles, stiles.data(),
                       stiles.size() * sizeof(mta::StepTile),
                       hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess)
    return fail(MTA_EHIP, "uploading the tile table: %s", hipGetErrorString(e));
  return MTA_OK;
}

mta::Work work_of(const mta_list *L, int grid, void *stream) {
  mta::Work w;
  w.gtiles = L->d_gtiles;
  w.stiles = L->d_stiles;
  w.ntiles = L->ntiles;
  w.keep_from = L->keep_from;
  w.grid = grid;
  w.stream = static_cast<hipStream_t>(stream);
  w.max_grid = L->max_grid;
  return w;
}

// The per-tile kernels (update, in-place scale) take one workgroup per
// tile, and one launch holds at most max_grid of them: a longer list is
// covered by consecutive launches over stretches of its tile table (every
// tile is independent of the others).  A failing launch stops the rest.
template <typename Launch>
hipError_t per_tile_launches(const mta::Work &wk, Launch &&launch) {
  const uint32_t cap = wk.max_grid ? wk.max_grid : mta::kMaxTileGrid;
  for (uint32_t base = 0; base < wk.ntiles; base += cap) {  // < 2^31 + cap
    mta::Work sub = wk;
    sub.ntiles = std::min(cap, wk.ntiles - base);
    sub.grid = static_cast<int>(sub.ntiles);
    sub.stiles = wk.stiles + base;
    sub.gtiles = wk.gtiles + base;
    const hipError_t e = launch(sub);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Argument checks of a norm over `nlists` lists (one list: mta_clip_norm).
int check_joint(mta_list *const *lists, int64_t nlists, float max_norm,
                const float *d_norm, const float *d_coef) {
  if (!lists || nlists < 1) return fail(MTA_EINVAL, "no lists");
  if (!(max_norm > 0.0f))
    return fail(MTA_EINVAL, "max_norm must be > 0 (got %g)",
                static_cast<double>(max_norm));
  if (!d_coef) return fail(MTA_EINVAL, "d_coef is NULL");
  if (!aligned(d_coef, 4) || (d_norm && !aligned(d_norm, 4)))
    return fail(MTA_EALIGN, "d_norm / d_coef must be 4-byte aligned");
  for (int64_t i = 0; i < nlists; ++i) {
    if (!lists[i])
      return nlists == 1 ? fail(MTA_EINVAL, "list is NULL")
                         : fail(MTA_EINVAL, "list %lld is NULL",
                                static_cast<long long>(i));
    for (int64_t j = 0; j < i; ++j)
      if (lists[j] == lists[i])  // its gradients would count twice
        return fail(MTA_EINVAL, "list %lld appears twice",
                    static_cast<long long>(i));
  }
  for (int64_t i = 0; i < nlists; ++i) {
    const int rc = check_device(lists[i]);
    if (rc) return rc;
  }
  return MTA_OK;
}

// One norm launch per list, in order: each adds the running float64 total
// in lists[0]'s accumulator slot and writes the norm and coefficient of the
// total so far; the last launch's are the joint result.  d_amp set: the
// loss-scaled norm (unscale factor from the state, found_inf).
int joint_norm(mta_list *const *lists, int64_t nlists, float max_norm,
               mta_amp_state *d_amp, float *d_norm, float *d_coef,
               void *stream, const char *what) {
  double *const acc = lists[0]->d_acc;
  for (int64_t i = 0; i < nlists; ++i) {
    mta_list *L = lists[i];
    const mta::Work wk = work_of(L, L->grid_norm, stream);
    const float s = (!d_amp && L->deferred) ? L->deferred_s : 1.0f;
    const mta::NormScratch scr{L->d_partials, L->d_ticket,
                               i > 0 ? acc : nullptr,
                               i + 1 < nlists ? acc : nullptr};
    const hipError_t e = mta::launch_sumsq(L->gtype, wk, s, max_norm, scr,
                                           d_norm, d_coef, d_amp);
    if (e != hipSuccess) return after_launch(e, wk.stream, what);
  }
  return after_launch(hipSuccess, static_cast<hipStream_t>(stream), what);
}

const char *opt_name(int kind) {
  switch (kind) {
    case MTA_OPT_ADAMW: return "MTA_OPT_ADAMW";
    case MTA_OPT_ADAM: return "MTA_OPT_ADAM";
    case MTA_OPT_SGD: return "MTA_OPT_SGD";
    case MTA_OPT_MOMENTUM: return "MTA_OPT_MOMENTUM";
    default: return "?";
  }
}

bool adam_family(int kind) {
  return kind == MTA_OPT_ADAMW || kind == MTA_OPT_ADAM;
}

// Argument checks of one step of `o`'s rule (t is checked by the caller).
int check_opt(const mta_opt *o, int64_t t) {
  if (!o) return fail(MTA_EINVAL, "opt is NULL");
  if (o->kind < MTA_OPT_ADAMW || o->kind > MTA_OPT_MOMENTUM)
    return fail(MTA_EINVAL, "unknown optimizer kind %d", o->kind);
  if (o->flags & ~MTA_STEP_ZERO_GRAD)
    return fail(MTA_EINVAL, "unknown step flags 0x%x",
                static_cast<unsigned>(o->flags));
  if (adam_family(o->kind)) {
    const mta_adamw_hparams hp{o->lr, o->beta1, o->beta2, o->eps,
                               o->weight_decay};
    return check_hparams(&hp, t);
  }
  if (!(std::isfinite(o->lr) && o->lr >= 0.0))
    return fail(MTA_EINVAL, "lr must be finite and >= 0 (got %g)", o->lr);
  if (o->weight_decay != 0.0)
    return fail(MTA_EINVAL,
                "%s has no weight decay: weight_decay must be 0 (got %g)",
                opt_name(o->kind), o->weight_decay);
  if (o->kind == MTA_OPT_MOMENTUM &&
      !(std::isfinite(o->momentum) && o->momentum >= 0.0))
    return fail(MTA_EINVAL, "momentum must be finite and >= 0 (got %g)",
                o->momentum);
  if (t < 1) return fail(MTA_EINVAL, "step t must be >= 1 (got %lld)",
                         static_cast<long long>(t));
  return MTA_OK;
}

// The kernel's scalar block for one step of `o`'s rule at step t.
mta::StepScalars opt_scalars(const mta_opt &o, int64_t t) {
  mta::StepScalars sc{};
  if (adam_family(o.kind)) {
    const mta_adamw_hparams hp{o.lr, o.beta1, o.beta2, o.eps,
                               o.weight_decay};
    sc = step_scalars(hp, t);
    if (o.kind == MTA_OPT_ADAM) {
      sc.dec = 1.0f;  // not read: Adam does not decay w
      sc.l2 = static_cast<float>(o.weight_decay);
    }
  } else {
    // w + (-lr)*g: lr is the float32 value, negated exactly
    sc.nstep = -static_cast<float>(o.lr);
    sc.mu = static_cast<float>(o.momentum);
  }
  sc.s = 1.0f;
  sc.zero = (o.flags & MTA_STEP_ZERO_GRAD) ? 1u : 0u;
  return sc;
}


// One step of any rule, plain (d_amp == nullptr: t and the deferred factor
// from the host) or loss-scaled (t and 1/scale from the device state).
int step_common(mta_list *L, const mta_opt *o, int64_t t, const float *d_coef,
                const mta_amp_state *d_amp, void *stream, const char *what) {
  int rc = check_opt(o, t);
  if (rc) return rc;
  if (!L) return fail(MTA_EINVAL, "list is NULL");
  if (!L->has_w)
    return fail(MTA_ESTATE,
                "a gradient-only list (no w) serves the norm and the scale "
                "calls, not an update");
  const bool needs_m = o->kind != MTA_OPT_SGD;
  const bool needs_v = adam_family(o->kind);
  if ((needs_m && !(L->state_buffers & 1)) ||
      (needs_v && !(L->state_buffers & 2)))
    return fail(MTA_ESTATE, "%s needs the list's %s buffers, which it lacks",
                opt_name(o->kind), needs_v ? "m and v" : "m");
  if (o->kind == MTA_OPT_MOMENTUM && L->mkind != MTA_MOM_F32)
    return fail(MTA_EDTYPE, "the momentum buffer (m) must be float32");
  if (d_coef && !aligned(d_coef, 4))
    return fail(MTA_EALIGN, "d_coef must be 4-byte aligned");
  if (d_amp) {
    if (!aligned(d_amp, 8))
      return fail(MTA_EALIGN, "d_amp must be 8-byte aligned");
    if (L->deferred)
      return fail(MTA_ESTATE,
                  "a host deferred scale factor is pending; a loss-scaled "
                  "step takes its factor from the loss-scale state");
  }
  rc = check_device(L);
  if (rc) return rc;
  mta::StepScalars sc = opt_scalars(*o, t);
  sc.s = (!d_amp && L->deferred) ? L->deferred_s : 1.0f;
  sc.copy_f16 = L->copy_type == MTA_F16 ? 1u : 0u;
  mta::AmpStep amp{};
  if (d_amp) {
    // a new generation whenever the constants' inputs change (the device
    // cache is keyed by it and by t)
    if (L->amp_gen == 0 || L->amp_hp[0] != o->lr ||
        L->amp_hp[1] != o->beta1 || L->amp_hp[2] != o->beta2) {
      L->amp_gen = L->amp_gen % 255 + 1;
      L->amp_hp[0] = o->lr;
      L->amp_hp[1] = o->beta1;
      L->amp_hp[2] = o->beta2;
    }
    amp = mta::AmpStep{d_amp, o->lr, o->beta1, o->beta2, L->d_amp_cache,
                       L->amp_gen};
  }
  if (L->ntiles > 0) {
    const mta::Work wk = work_of(L, L->grid_update, stream);
    const hipError_t e = per_tile_launches(wk, [&](const mta::Work &sub) {
      return mta::launch_update(o->kind, L->gtype, L->mkind, L->vkind, sub,
                                sc, d_coef, amp);
    });
    // a launch refused (with one launch per list, as below 2^24 tiles,
    // nothing was enqueued): a deferred factor stays
    if (e != hipSuccess) return after_launch(e, wk.stream, what);
    if (!d_amp) {
      L->deferred = false;
      L->deferred_s = 1.0f;
    }
    return after_launch(hipSuccess, wk.stream, what);
  }
  if (!d_amp) {
    L->deferred = false;
    L->deferred_s = 1.0f;
  }
  return ok();
}

mta_opt adamw_opt(const mta_adamw_hparams *hp) {
  mta_opt o{};
  o.kind = MTA_OPT_ADAMW;
  if (hp) {
    o.lr = hp->lr;
    o.beta1 = hp->beta1;
    o.beta2 = hp->beta2;
    o.eps = hp->eps;
    o.weight_decay = hp->weight_decay;
  }
  return o;
}

// Everything mta_list_create decides before it touches a device: argument
// checks, overlap checks, the tile tables and the norm's kept tiles.
struct Plan {
  std::vector<mta_tensor> kept;
  std::vector<mta::GradTile> gtiles;
  std::vector<mta::StepTile> stiles;
  int64_t elements = 0;
  int vec_tensors = 0;
  int state = -1;
  uint32_t keep_from = 0;
};

int plan_list(const mta_tensor *tensors, int64_t count, int gtype, int mkind,
              int vkind, Plan *plan) {
  if (count < 0) return fail(MTA_EINVAL, "count must be >= 0");
  if (count > 0 && !tensors) return fail(MTA_EINVAL, "tensors is NULL");
  if (count > static_cast<int64_t>(UINT32_MAX))
    return fail(MTA_EINVAL, "too many tensors");
  if (gtype != MTA_F32 && gtype != MTA_BF16 && gtype != MTA_F16)
    return fail(MTA_EDTYPE, "unknown gradient type %d", gtype);
  if (mkind != MTA_MOM_F32 && mkind != MTA_MOM_BF16X2)
    return fail(MTA_EDTYPE, "unknown m kind %d", mkind);
  if (vkind != MTA_MOM_F32 && vkind != MTA_MOM_BF16X2)
    return fail(MTA_EDTYPE, "unknown v kind %d", vkind);

  const uintptr_t gsz = gtype == MTA_F32 ? 4 : 2;
  const uintptr_t msz = mkind == MTA_MOM_BF16X2 ? 2 : 4;
  const uintptr_t vsz = vkind == MTA_MOM_BF16X2 ? 2 : 4;

  std::vector<mta::GradTile> &gtiles = plan->gtiles;
  std::vector<mta::StepTile> &stiles = plan->stiles;
  std::vector<mta_tensor> &kept = plan->kept;
  std::vector<Span> spans;
  uint32_t &keep_from = plan->keep_from;
  int64_t &elements = plan->elements;
  int &vec_tensors = plan->vec_tensors;
  int &state = plan->state;  // m / v presence of the first non-empty tensor
  int64_t state_from = -1;
  try {
    spans.reserve(static_cast<size_t>(count) * 4);
    uint64_t ntiles = 0;
    for (int64_t i = 0; i < count; ++i) {
      const mta_tensor &x = tensors[i];
      if (x.n < 0)
        return fail(MTA_EINVAL, "tensor %lld: n < 0", static_cast<long long>(i));
      if (x.n > (INT64_MAX / 8))
        return fail(MTA_EINVAL, "tensor %lld: n too large",
                    static_cast<long long>(i));
      if (x.n == 0) continue;
      if (!x.g)
        return fail(MTA_EINVAL, "tensor %lld: g is NULL",
                    static_cast<long long>(i));
      if (!x.w && (x.m || x.v))
        return fail(MTA_EINVAL,
                    "tensor %lld: m or v without w (only a gradient-only "
                    "list, w, m and v all NULL, may leave w out)",
                    static_cast<long long>(i));
      // bit 0: m, bit 1: v, bit 2: w
      const int st = (x.m ? 1 : 0) | (x.v ? 2 : 0) | (x.w ? 4 : 0);
      if (state < 0) {
        state = st;
        state_from = i;
      } else if (st != state) {
        return fail(MTA_EINVAL,
                    "tensor %lld: its w / m / v buffers are not given the "
                    "way tensor %lld's are (a list has the same buffers on "
                    "every tensor)",
                    static_cast<long long>(i),
                    static_cast<long long>(state_from));
      }
      if (!aligned(x.w, 4) || !aligned(x.g, gsz) || !aligned(x.m, msz) ||
          !aligned(x.v, vsz))
        return fail(MTA_EALIGN,
                    "tensor %lld: a buffer is not aligned to its element size",
                    static_cast<long long>(i));
      const int64_t peel = vector_peel(x, gtype, mkind, vkind);
      vec_tensors += (peel >= 0 && peel < x.n) ? 1 : 0;
      const uintptr_t n = static_cast<uintptr_t>(x.n);
      const void *bufs[4] = {x.w, x.g, x.m, x.v};
      const uintptr_t sizes[4] = {4, gsz, msz, vsz};
      for (int b = 0; b < 4; ++b) {
        if (!bufs[b]) continue;
        const uintptr_t lo = reinterpret_cast<uintptr_t>(bufs[b]);
        spans.push_back(Span{lo, lo + n * sizes[b], i, b});
      }
      elements += x.n;
      ntiles += tiles_of(x.n, peel);
      // tile numbers and grid strides stay below 2^32 (no wrap-around)
      if (ntiles > (uint64_t{1} << 31)) return fail(MTA_EINVAL, "list too large");
    }
    int rc = check_overlaps(&spans);
    if (rc) return rc;
    // one record per tile: buffer addresses offset to the tile's first
    // element, its length, and whether the vector path may be taken
    kept.assign(tensors, tensors + count);
    build_step_tiles(kept, {}, {}, gtype, mkind, vkind, &stiles);
    gtiles.reserve(stiles.size());
    for (const mta::StepTile &st : stiles)
      gtiles.push_back(mta::GradTile{st.g, st.lim, aligned(st.g, 16) ? 1u : 0u});
    // the last tiles, up to the keep budget
    const int keep_mib = env_int("MTA_NORM_KEEP_MIB", -1, 0, 1 << 20);
    uint64_t budget =
        static_cast<uint64_t>(keep_mib >= 0 ? keep_mib : kNormKeepMiB) << 20;
    keep_from = static_cast<uint32_t>(gtiles.size());
    while (keep_from > 0) {
      const uint64_t bytes = uint64_t{gtiles[keep_from - 1].lim} * gsz;
      if (bytes > budget) break;
      budget -= bytes;
      --keep_from;
    }
    // the update's bytes per element: w read and written, g, and m and v
    // read and written when the list has them
    const uint64_t upd = 8 + gsz + (state < 0 || (state & 1) ? 2 * msz : 0) +
                         (state < 0 || (state & 2) ? 2 * vsz : 0);
    // elements the update takes on its element path before the kept tiles
    uint64_t elem_path = 0;
    for (uint32_t i = 0; i < keep_from; ++i)
      if (!(stiles[i].flags & mta::kTileVec) ||
          stiles[i].lim != static_cast<uint32_t>(mta::kTileElems))
        elem_path += stiles[i].lim;
    if (keep_mib < 0 &&
        elem_path * upd > static_cast<uint64_t>(kNormKeepElemMiB) << 20)
      keep_from = static_cast<uint32_t>(gtiles.size());
  } catch (const std::bad_alloc &) {
    return fail(MTA_ENOMEM, "host allocation failed");
  }
  return MTA_OK;
}

}  // namespace

extern "C" {

int mta_abi_version(void) { return MTA_ABI_VERSION; }

const char *mta_last_error(void) { return g_err; }

int mta_adamw_scalars(const mta_adamw_hparams *hp, int64_t t, float out[7]) {
  int rc = check_hparams(hp, t);
  if (rc) return rc;
  if (!out) return fail(MTA_EINVAL, "out is NULL");
  make_scalars(*hp, t, out);
  return ok();
}

int mta_list_create(const mta_tensor *tensors, int64_t count, int gtype,
                    int mkind, int vkind, void *stream, mta_list **out) {
  if (!out) return fail(MTA_EINVAL, "out is NULL");
  *out = nullptr;
  Plan plan;
  const int rc = plan_list(tensors, count, gtype, mkind, vkind, &plan);
  if (rc) return rc;
  std::vector<mta::GradTile> &gtiles = plan.gtiles;
  std::vector<mta::StepTile> &stiles = plan.stiles;

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(MTA_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess || cus <= 0)
    return fail(MTA_EHIP, "cannot read the compute-unit count: %s",
                hipGetErrorString(e));

  mta_list *L = new (std::nothrow) mta_list;
  if (!L) return fail(MTA_ENOMEM, "host allocation failed");
  L->tensors = std::move(plan.kept);
  L->device = dev;
  L->gtype = gtype;
  L->mkind = mkind;
  L->vkind = vkind;
  L->count = count;
  L->elements = plan.elements;
  L->ntiles = static_cast<uint32_t>(stiles.size());
  L->keep_from = plan.keep_from;
  L->vector_tensors = plan.vec_tensors;
  L->cus = cus;
  // no element: any rule
  L->state_buffers = plan.state < 0 ? 3 : (plan.state & 3);
  L->has_w = plan.state < 0 || (plan.state & 4);
  const int bpc_n = env_int(
      "MTA_NORM_BLOCKS_PER_CU",
      gtype == MTA_F32 ? kNormBlocksPerCuF32 : kNormBlocksPerCu16, 1, 64);
  const int64_t tiles_or_one = std::max<int64_t>(1, L->ntiles);
  // one workgroup per tile, in launches of at most max_grid tiles
  // (MTA_MAX_TILE_GRID lowers the cap, to exercise several launches)
  L->max_grid = static_cast<uint32_t>(env_int(
      "MTA_MAX_TILE_GRID", static_cast<int>(mta::kMaxTileGrid), 1,
      static_cast<int>(mta::kMaxTileGrid)));
  L->grid_update = static_cast<int>(
      std::min<int64_t>(tiles_or_one, static_cast<int64_t>(L->max_grid)));
  L->grid_norm = static_cast<int>(
      std::min<int64_t>(tiles_or_one, static_cast<int64_t>(cus) * bpc_n));

  const size_t off_gt = 0;
  const size_t off_st =
      round_up(off_gt + gtiles.size() * sizeof(mta::GradTile), 256);
  const size_t off_part =
      round_up(off_st + stiles.size() * sizeof(mta::StepTile), 256);
  const size_t off_ticket =
      round_up(off_part + static_cast<size_t>(L->grid_norm) * sizeof(double),
               256);
  const size_t total = off_ticket + mta::kTicketBytes;

  e = hipMalloc(&L->dev_block, total);
  if (e != hipSuccess) {
    delete L;
    return fail(MTA_ENOMEM, "hipMalloc(%zu): %s", total, hipGetErrorString(e));
  }
  char *base = static_cast<char *>(L->dev_block);
  L->d_gtiles = reinterpret_cast<mta::GradTile *>(base + off_gt);
  L->d_stiles = reinterpret_cast<mta::StepTile *>(base + off_st);
  L->d_partials = reinterpret_cast<double *>(base + off_part);
  L->d_ticket = reinterpret_cast<unsigned int *>(base + off_ticket);
  L->d_acc = reinterpret_cast<double *>(base + off_ticket + mta::kAccOffset);
  L->d_amp_cache =
      reinterpret_cast<uint64_t *>(base + off_ticket + mta::kAmpCacheOffset);

  hipStream_t s = static_cast<hipStream_t>(stream);
  e = hipSuccess;
  if (!gtiles.empty())
    e = hipMemcpyAsync(L->d_gtiles, gtiles.data(),
                       gtiles.size() * sizeof(mta::GradTile),
                       hipMemcpyHostToDevice, s);
  if (e == hipSuccess && !stiles.empty())
    e = hipMemcpyAsync(L->d_stiles, stiles.data(),
                       stiles.size() * sizeof(mta::StepTile),
                       hipMemcpyHostToDevice, s);
  // every norm partial slot starts empty (the norm kernel re-arms them)
  std::vector<uint64_t> empty_slots;
  try {
    empty_slots.assign(static_cast<size_t>(L->grid_norm), mta::kNormSlotEmpty);
  } catch (const std::bad_alloc &) {
    (void)hipFree(L->dev_block);
    delete L;
    return fail(MTA_ENOMEM, "host allocation failed");
  }
  if (e == hipSuccess)
    e = hipMemcpyAsync(L->d_partials, empty_slots.data(),
                       empty_slots.size() * sizeof(uint64_t),
                       hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = hipMemsetAsync(L->d_ticket, 0, mta::kTicketBytes, s);
  // the host vectors die with this call: wait for the copies
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    (void)hipFree(L->dev_block);
    delete L;
    return fail(MTA_EHIP, "uploading the list table: %s", hipGetErrorString(e));
  }
  *out = L;
  return ok();
}

int mta_list_destroy(mta_list *L) {
  if (!L) return ok();
  hipError_t e = hipFree(L->dev_block);
  delete L;
  if (e != hipSuccess)
    return fail(MTA_EHIP, "hipFree: %s", hipGetErrorString(e));
  return ok();
}

int mta_list_set_weight_copies(mta_list *L, void *const *w16, void *stream) {
  return mta_list_set_weight_copies_as(L, w16, MTA_BF16, stream);
}

int mta_list_set_weight_copies_as(mta_list *L, void *const *w16,
                                  int32_t copy_type, void *stream) {
  if (!L) return fail(MTA_EINVAL, "list is NULL");
  if (copy_type != MTA_BF16 && copy_type != MTA_F16)
    return fail(MTA_EDTYPE, "a weight copy is bfloat16 or float16, not %d",
                static_cast<int>(copy_type));
  if (w16 && !L->has_w)
    return fail(MTA_ESTATE, "a gradient-only list has no weights to copy");
  std::vector<void *> copies;
  int attached = 0;
  try {
    if (w16) {
      std::vector<Span> spans;
      list_spans(L, &spans);
      copies.assign(w16, w16 + L->tensors.size());
      for (size_t i = 0; i < copies.size(); ++i) {
        const int64_t n = L->tensors[i].n;
        if (!copies[i] || n == 0) {
          copies[i] = nullptr;
          continue;
        }
        if (!aligned(copies[i], 2))
          return fail(MTA_EALIGN, "tensor %lld: weight copy not 2-byte aligned",
                      static_cast<long long>(i));
        const uintptr_t lo = reinterpret_cast<uintptr_t>(copies[i]);
        spans.push_back(Span{lo, lo + static_cast<uintptr_t>(n) * 2,
                             static_cast<int64_t>(i), 4});
        ++attached;
      }
      int rc = check_overlaps(&spans);
      if (rc) return rc;
      if (attached == 0) copies.clear();
    }
  } catch (const std::bad_alloc &) {
    return fail(MTA_ENOMEM, "host allocation failed");
  }
  const int rc = upload_step_tiles(L, copies, L->no_decay, stream);
  if (rc) return rc;
  L->w16 = std::move(copies);
  L->weight_copies = attached;
  L->copy_type = copy_type;
  return ok();
}

int mta_list_set_no_decay(mta_list *L, const uint8_t *no_decay,
                          void *stream) {
  if (!L) return fail(MTA_EINVAL, "list is NULL");
  std::vector<uint8_t> flags;
  int flagged = 0;
  try {
    if (no_decay) {
      flags.assign(L->tensors.size(), 0);
      for (size_t i = 0; i < flags.size(); ++i) {
        flags[i] = no_decay[i] ? 1 : 0;
        flagged += flags[i];
      }
      if (flagged == 0) flags.clear();
    }
  } catch (const std::bad_alloc &) {
    return fail(MTA_ENOMEM, "host allocation failed");
  }
  const int rc = upload_step_tiles(L, L->w16, flags, stream);
  if (rc) return rc;
  L->no_decay = std::move(flags);
  L->no_decay_tensors = flagged;
  return ok();
}

int mta_list_plan(const mta_tensor *tensors, int64_t count, int gtype,
                  int mkind, int vkind, mta_list_info_t *out) {
  if (!out) return fail(MTA_EINVAL, "out is NULL");
  Plan plan;
  try {
    const int rc = plan_list(tensors, count, gtype, mkind, vkind, &plan);
    if (rc) return rc;
  } catch (const std::bad_alloc &) {
    return fail(MTA_ENOMEM, "host allocation failed");
  }
  *out = mta_list_info_t{};
  out->count = count;
  out->elements = plan.elements;
  out->tiles = static_cast<int64_t>(plan.stiles.size());
  out->tile_elems = mta::kTileElems;
  out->device = -1;  // no device: grid_update and grid_norm stay 0
  out->vector_tensors = plan.vec_tensors;
  out->gtype = gtype;
  out->mkind = mkind;
  out->vkind = vkind;
  out->state_buffers = plan.state < 0 ? 3 : (plan.state & 3);
  out->weight_copy_type = MTA_BF16;
  out->norm_kept_tiles =
      static_cast<int32_t>(plan.stiles.size() - plan.keep_from);
  return ok();
}

int mta_list_info(const mta_list *L, mta_list_info_t *out) {
  if (!L || !out) return fail(MTA_EINVAL, "NULL argument");
  out->count = L->count;
  out->elements = L->elements;
  out->tiles = L->ntiles;
  out->tile_elems = mta::kTileElems;
  out->grid_update = L->grid_update;
  out->grid_norm = L->grid_norm;
  out->device = L->device;
  out->vector_tensors = L->vector_tensors;
  out->gtype = L->gtype;
  out->mkind = L->mkind;
  out->vkind = L->vkind;
  out->weight_copies = L->weight_copies;
  out->state_buffers = L->state_buffers;
  out->weight_copy_type = L->copy_type;
  out->norm_kept_tiles = static_cast<int32_t>(L->ntiles - L->keep_from);
  return ok();
}

int mta_scale(mta_list *L, float factor, int flags, void *stream) {
  if (!L) return fail(MTA_EINVAL, "list is NULL");
  if (!std::isfinite(factor))
    return fail(MTA_EINVAL, "scale factor must be finite");
  if (flags == MTA_SCALE_DEFER) {
    if (L->deferred)
      return fail(MTA_ESTATE,
                  "a deferred scale factor is already pending; run "
                  "mta_adamw_step first");
    L->deferred = true;
    L->deferred_s = factor;
    return ok();
  }
  if (flags != MTA_SCALE_INPLACE)
    return fail(MTA_EINVAL, "flags must be MTA_SCALE_INPLACE or MTA_SCALE_DEFER");
  int rc = check_device(L);
  if (rc) return rc;
  if (L->ntiles == 0) return ok();
  // one workgroup per gradient tile
  const mta::Work wk = work_of(L, L->grid_update, stream);
  return after_launch(per_tile_launches(wk, [&](const mta::Work &sub) {
                        return mta::launch_scale(L->gtype, sub, factor,
                                                 nullptr);
                      }),
                      wk.stream, "mta_scale");
}

int mta_scale_device(mta_list *L, const float *d_factor, void *stream) {
  if (!L) return fail(MTA_EINVAL, "list is NULL");
  if (!d_factor) return fail(MTA_EINVAL, "d_factor is NULL");
  if (!aligned(d_factor, 4))
    return fail(MTA_EALIGN, "d_factor must be 4-byte aligned");
  int rc = check_device(L);
  if (rc) return rc;
  if (L->ntiles == 0) return ok();
  const mta::Work wk = work_of(L, L->grid_update, stream);
  return after_launch(per_tile_launches(wk, [&](const mta::Work &sub) {
                        return mta::launch_scale(L->gtype, sub, 1.0f,
                                                 d_factor);
                      }),
                      wk.stream, "mta_scale_device");
}

int mta_clip_norm(mta_list *L, float max_norm, float *d_norm, float *d_coef,
                  void *stream) {
  return mta_clip_norm_joint(&L, 1, max_norm, d_norm, d_coef, stream);
}

int mta_clip_norm_joint(mta_list *const *lists, int64_t nlists,
                        float max_norm, float *d_norm, float *d_coef,
                        void *stream) {
  int rc = check_joint(lists, nlists, max_norm, d_norm, d_coef);
  if (rc) return rc;
  return joint_norm(lists, nlists, max_norm, nullptr, d_norm, d_coef, stream,
                    nlists == 1 ? "mta_clip_norm" : "mta_clip_norm_joint");
}

int mta_adamw_step(mta_list *L, const mta_adamw_hparams *hp, int64_t t,
                   const float *d_coef, void *stream) {
  if (!hp) return fail(MTA_EINVAL, "hparams is NULL");
  const mta_opt o = adamw_opt(hp);
  return step_common(L, &o, t, d_coef, nullptr, stream, "mta_adamw_step");
}

int mta_step(mta_list *L, const mta_opt *opt, int64_t t, const float *d_coef,
             void *stream) {
  return step_common(L, opt, t, d_coef, nullptr, stream, "mta_step");
}

int mta_clip_norm_noalloc(const mta_tensor *tensors, int64_t count,
                          int gtype, float scale, float max_norm,
                          float *d_norm, float *d_coef, void *stream) {
  // the checks of mta_clip_norm, on a tensor array instead of a list
  if (!(max_norm > 0.0f))
    return fail(MTA_EINVAL, "max_norm must be > 0 (got %g)",
                static_cast<double>(max_norm));
  if (!std::isfinite(scale))
    return fail(MTA_EINVAL, "scale factor must be finite");
  if (!d_coef) return fail(MTA_EINVAL, "d_coef is NULL");
  if (!aligned(d_coef, 4) || (d_norm && !aligned(d_norm, 4)))
    return fail(MTA_EALIGN, "d_norm / d_coef must be 4-byte aligned");
  Plan plan;
  try {
    const int rc = plan_list(tensors, count, gtype, MTA_MOM_F32, MTA_MOM_F32,
                             &plan);
    if (rc) return rc;
  } catch (const std::bad_alloc &) {
    return fail(MTA_ENOMEM, "host allocation failed");
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(MTA_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess || cus <= 0)
    return fail(MTA_EHIP, "cannot read the compute-unit count: %s",
                hipGetErrorString(e));
  // the launch shape of mta_clip_norm on the same tensors
  const int64_t ntiles = static_cast<int64_t>(plan.gtiles.size());
  const int bpc_n = env_int(
      "MTA_NORM_BLOCKS_PER_CU",
      gtype == MTA_F32 ? kNormBlocksPerCuF32 : kNormBlocksPerCu16, 1, 64);
  const int grid = static_cast<int>(std::min<int64_t>(
      std::max<int64_t>(1, ntiles), static_cast<int64_t>(cus) * bpc_n));
  // scratch layout: ticket region, partial slots, gradient tile table
  const size_t off_part = mta::kTicketBytes;
  const size_t off_gt = round_up(off_part + sizeof(double) * grid, 256);
  const size_t need = off_gt + sizeof(mta::GradTile) * plan.gtiles.size();
  if (need > mta::kNoAllocScratchBytes)
    return fail(MTA_EINVAL,
                "the list needs %zu bytes of scratch; the allocation-free "
                "norm has %zu (%lld tiles of %d elements here, at most %zu)",
                need, mta::kNoAllocScratchBytes,
                static_cast<long long>(ntiles), mta::kTileElems,
                (mta::kNoAllocScratchBytes - off_gt) /
                    sizeof(mta::GradTile));
  void *base = nullptr;
  e = mta::noalloc_scratch(dev, &base);
  if (e != hipSuccess)
    return fail(MTA_EHIP, "the scratch's device address: %s",
                hipGetErrorString(e));
  std::vector<uint64_t> slots;
  try {
    slots.assign(static_cast<size_t>(grid), mta::kNormSlotEmpty);
  } catch (const std::bad_alloc &) {
    return fail(MTA_ENOMEM, "host allocation failed");
  }
  char *const b = static_cast<char *>(base);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // one call at a time per process: the scratch is shared by every call on
  // a device, and each call waits for its own work before it returns
  static std::mutex mu;
  std::lock_guard<std::mutex> lock(mu);
  // the ticket counters and the running total start at zero, every partial
  // slot empty (the array keeps whatever the last call left)
  e = hipMemsetAsync(b, 0, mta::kTicketBytes, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(b + off_part, slots.data(),
                       slots.size() * sizeof(uint64_t),
                       hipMemcpyHostToDevice, s);
  if (e == hipSuccess && !plan.gtiles.empty())
    e = hipMemcpyAsync(b + off_gt, plan.gtiles.data(),
                       plan.gtiles.size() * sizeof(mta::GradTile),
                       hipMemcpyHostToDevice, s);
  if (e != hipSuccess) {
    // a copy queued before the failing call still reads the host vectors
    (void)hipStreamSynchronize(s);
    return fail(MTA_EHIP, "mta_clip_norm_noalloc: staging: %s",
                hipGetErrorString(e));
  }
  mta::Work wk{};
  wk.gtiles = reinterpret_cast<const mta::GradTile *>(b + off_gt);
  wk.stiles = nullptr;
  wk.ntiles = static_cast<uint32_t>(ntiles);
  wk.keep_from = plan.keep_from;
  wk.grid = grid;
  wk.stream = s;
  const mta::NormScratch scr{reinterpret_cast<double *>(b + off_part),
                             reinterpret_cast<unsigned int *>(b), nullptr,
                             nullptr};
  e = mta::launch_sumsq(gtype, wk, scale, max_norm, scr, d_norm, d_coef,
                        nullptr);
  if (e != hipSuccess) {
    (void)hipStreamSynchronize(s);  // the copies still read the host vectors
    return fail(MTA_EHIP, "mta_clip_norm_noalloc: launch failed: %s",
                hipGetErrorString(e));
  }
  // the staging vectors die with this call, and the next call reuses the
  // scratch: wait for this one's copies and kernel
  e = hipStreamSynchronize(s);
  if (e != hipSuccess)
    return fail(MTA_EHIP, "mta_clip_norm_noalloc: kernel failed: %s",
                hipGetErrorString(e));
  return ok();
}

int mta_amp_clip_norm(mta_list *L, float max_norm, mta_amp_state *d_amp,
                      float *d_norm, float *d_coef, void *stream) {
  return mta_amp_clip_norm_joint(&L, 1, max_norm, d_amp, d_norm, d_coef,
                                 stream);
}

int mta_amp_clip_norm_joint(mta_list *const *lists, int64_t nlists,
                            float max_norm, mta_amp_state *d_amp,
                            float *d_norm, float *d_coef, void *stream) {
  if (!d_amp) return fail(MTA_EINVAL, "d_amp is NULL");
  if (!aligned(d_amp, 8))
    return fail(MTA_EALIGN, "d_amp must be 8-byte aligned");
  int rc = check_joint(lists, nlists, max_norm, d_norm, d_coef);
  if (rc) return rc;
  for (int64_t i = 0; i < nlists; ++i)
    if (lists[i]->deferred)
      return fail(MTA_ESTATE,
                  "list %lld: a host deferred scale factor is pending; a "
                  "loss-scaled norm takes its factor from the loss-scale "
                  "state",
                  static_cast<long long>(i));
  return joint_norm(lists, nlists, max_norm, d_amp, d_norm, d_coef, stream,
                    nlists == 1 ? "mta_amp_clip_norm"
                                : "mta_amp_clip_norm_joint");
}

int mta_amp_adamw_step(mta_list *L, const mta_adamw_hparams *hp,
                       const mta_amp_state *d_amp, const float *d_coef,
                       void *stream) {
  if (!hp) return fail(MTA_EINVAL, "hparams is NULL");
  if (!d_amp) return fail(MTA_EINVAL, "d_amp is NULL");
  const mta_opt o = adamw_opt(hp);
  return step_common(L, &o, 1, d_coef, d_amp, stream, "mta_amp_adamw_step");
}

int mta_amp_step(mta_list *L, const mta_opt *opt, const mta_amp_state *d_amp,
                 const float *d_coef, void *stream) {
  if (!d_amp) return fail(MTA_EINVAL, "d_amp is NULL");
  return step_common(L, opt, 1, d_coef, d_amp, stream, "mta_amp_step");
}

int mta_amp_update(mta_amp_state *d_amp, double growth_factor,
                   double backoff_factor, int32_t growth_interval,
                   void *stream) {
  if (!d_amp) return fail(MTA_EINVAL, "d_amp is NULL");
  if (!aligned(d_amp, 8))
    return fail(MTA_EALIGN, "d_amp must be 8-byte aligned");
  if (!(std::isfinite(growth_factor) && growth_factor > 1.0))
    return fail(MTA_EINVAL, "growth_factor must be finite and > 1 (got %g)",
                growth_factor);
  if (!(backoff_factor > 0.0 && backoff_factor < 1.0))
    return fail(MTA_EINVAL, "backoff_factor must be in (0, 1) (got %g)",
                backoff_factor);
  if (growth_interval < 1)
    return fail(MTA_EINVAL, "growth_interval must be >= 1 (got %d)",
                static_cast<int>(growth_interval));
  hipStream_t s = static_cast<hipStream_t>(stream);
  return after_launch(mta::launch_amp_update(d_amp, growth_factor,
                                             backoff_factor, growth_interval,
                                             s),
                      s, "mta_amp_update");
}

}  // extern "C"
