// mta_internal.h -- types shared by the host runtime and the gfx950 kernels
// of libmta.  Not part of the public C ABI (that is include/mta.h).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/mta.h"

namespace mta {

// A tile is the work of one workgroup iteration: up to kTileElems consecutive
// elements of one tensor.  Tiles never straddle tensors, so every vector
// access inside a tile stays in one buffer.  A tensor's tiles start at
// multiples of kTileElems, or, when its buffers reach alignment together only
// after its first h (1..63) elements, at 0 (a head tile of h elements) and
// then at h + multiples of kTileElems.
constexpr int kBlock = 256;       // threads per workgroup (4 wave64s)
constexpr int kTileElems = 4096;  // 16 elements per thread

// The kernels read one self-contained record per tile, built once per list:
// its buffers' addresses already offset to the tile's first element, the
// number of elements in it, and whether all of them are 16-byte aligned.  One
// scalar load of the record is all a workgroup needs before it can issue the
// tile's vector loads (no second, dependent lookup of a per-tensor record).

// k_sumsq and k_scale read only the gradient.
struct GradTile {
  const void *g;
  uint32_t lim;  // elements in this tile, 1..kTileElems
  uint32_t vec;  // 1: the gradient buffer is 16-byte aligned
};
static_assert(sizeof(GradTile) == 16, "gradient tile layout");

// The update kernels read and write the buffers their rule uses (w and g
// always; m for momentum and the Adam family; v for the Adam family), and
// write the 16-bit weight copy when one is attached.  Unused buffers are
// null.
struct StepTile {
  float *w;
  const void *g;
  void *m;
  void *v;
  uint32_t lim;    // elements in this tile, 1..kTileElems
  uint32_t flags;  // kTileVec | kTileNoDecay
  void *w16;       // 16-bit copy of w at this tile, or nullptr
};
static_assert(sizeof(StepTile) == 48, "step tile layout");

// StepTile flags.
constexpr uint32_t kTileVec = 1;      // all buffers (w16 too, when present)
                                      // 16-byte aligned: the vector path
constexpr uint32_t kTileNoDecay = 2;  // the tensor's step takes
                                      // weight_decay = 0

// Update rules, numbered as mta_opt_kind.
constexpr int kRuleAdamW = MTA_OPT_ADAMW;
constexpr int kRuleAdam = MTA_OPT_ADAM;
constexpr int kRuleSgd = MTA_OPT_SGD;
constexpr int kRuleMomentum = MTA_OPT_MOMENTUM;

// Per-call float32 constants of a step (formed on the host in float64,
// rounded once).  Adam family: nstep = -step (negation is exact, so
// (-step)*m is unchanged), bc2, c1, c2, b2, eps; dec is AdamW's decay
// factor, l2 Adam's coupled decay.  SGD and momentum: nstep = -lr, mu.
struct StepScalars {
  float nstep, bc2, c1, c2, b2, eps, dec;
  float s;        // deferred unscale factor (1 when none)
  float l2;       // Adam: g' = g + w*l2
  float mu;       // momentum
  uint32_t zero;  // 1: write +0 into every gradient element after reading it
  uint32_t copy_f16;  // weight copies are float16 (else bfloat16)
};

// Per-tile launches (the update kernels, the in-place scale) give every
// tile its own workgroup.  The dispatch packet counts a grid's work-items
// in 32 bits, so one launch of kBlock-thread workgroups holds fewer than
// 2^24 of them; a list with more tiles is covered by consecutive launches
// over stretches of its tile table, each at most kMaxTileGrid tiles (whole
// runs of 256 workgroups).
constexpr uint32_t kMaxTileGrid = (1u << 24) - 256;

struct Work {
  const GradTile *gtiles;
  const StepTile *stiles;
  uint32_t ntiles;
  uint32_t keep_from;  // k_sumsq: first tile read with allocating loads
  int grid;
  hipStream_t stream;
  uint32_t max_grid;   // per-tile launches: most tiles in one launch
                       // (0: kMaxTileGrid)
};

// Norm scratch: one float64 partial slot per norm workgroup, then the
// ticket.  A slot holds kNormSlotEmpty (the host fills them at list
// creation) except between the storing workgroup and the finishing wave of
// one launch, which re-arms it.
constexpr uint64_t kNormSlotEmpty = 0xFFF0DEADBEEF0001ull;
// The ticket region: kTicketGroups group counters and one top counter,
// kTicketStride words (128 bytes) apart, then the float64 running total of
// a norm over several lists.
constexpr uint32_t kTicketGroups = 8;
constexpr uint32_t kTicketStride = 32;
constexpr size_t kTicketBytes = 2048;
constexpr size_t kAccOffset = (kTicketGroups + 1) * kTicketStride * 4;
static_assert(kAccOffset + 8 <= kTicketBytes, "ticket region layout");

struct NormScratch {
  double *partials;
  unsigned int *ticket;  // the ticket region
  // A norm over several lists launches one norm per list: each adds the
  // float64 total the previous one left in *acc_in (null for the first)
  // and leaves its own in *acc_out (null when there is no later list).
  const double *acc_in;
  double *acc_out;
};

// Loss-scaled step: with `state` set, the kernel skips the update when
// state->found_inf is set (it still zeroes the gradients when asked), and
// otherwise takes the unscale factor 1/state->scale and, for the Adam
// family, t = state->step + 1 from device memory, forming the t-dependent
// constants itself from these float64 hyperparameters.
static_assert(sizeof(mta_amp_state) == 24, "loss-scale state layout");

struct AmpStep {
  const mta_amp_state *state;  // nullptr: constants come from the host
  double lr, beta1, beta2;
  // The list's cache of the last step's t-dependent constants: two 64-bit
  // words, each (tag << 32) | float32 bits, for nstep and bc2; the tag is
  // (gen << 24) | (t mod 2^24).  gen (1..255, never 0) is the list's
  // generation of (lr, beta1, beta2), bumped on the host whenever they
  // change, so a tag names one set of constants and a word that starts
  // zeroed never matches.
  uint64_t *cache;
  uint32_t gen;
};

// Where a list's amp constant cache sits in its ticket region.
constexpr size_t kAmpCacheOffset = 1536;
static_assert(kAmpCacheOffset >= kAccOffset + 8 &&
                  kAmpCacheOffset + 16 <= kTicketBytes,
              "amp cache inside the ticket region, clear of the rest");

hipError_t launch_update(int rule, int gtype, int mkind, int vkind,
                         const Work &work, const StepScalars &sc,
                         const float *d_coef, const AmpStep &amp);
hipError_t launch_sumsq(int gtype, const Work &work, float s, float max_norm,
                        NormScratch scratch, float *d_norm, float *d_coef,
                        mta_amp_state *amp);
// d_s: null, or a device float that replaces s (read by the kernel).
hipError_t launch_scale(int gtype, const Work &work, float s,
                        const float *d_s);
hipError_t launch_amp_update(mta_amp_state *state, double growth,
                             double backoff, int32_t interval,
                             hipStream_t stream);

// The allocation-free norm's scratch: a file-scope device array in
// mta_kernels.hip of this many bytes (its ticket region, its partial
// slots, then its gradient tile table).
constexpr size_t kNoAllocScratchBytes = size_t{32} << 20;
// The device address of that array on the current device (taken with
// hipGetSymbolAddress on the first call on each device, kept per device).
hipError_t noalloc_scratch(int device, void **out);

}  // namespace mta
