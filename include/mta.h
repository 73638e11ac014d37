/*
 * mta.h -- fused mixed-precision gradient clip + multi-tensor AdamW step for
 * AMD Instinct MI355X (gfx950).  C ABI: plain pointers and sizes only.
 *
 * The operations and their sources (by page title and section):
 *
 *   mta_scale       ScaleTensors -- "Mica 7.7: a training step on the card, in
 *                   every float type", section "The whole model in one call":
 *                   one factor applied to every element of many tensors;
 *                   there it is how a float16 step removes its loss scale
 *                   ahead of the clip.
 *   mta_scale_device  ScaleTensors by a factor held in device memory: with
 *                   the coefficient mta_clip_norm left there, the clipped
 *                   gradients themselves, the scaling done on the device
 *                   as well (section "Values that stay on the card").
 *   mta_clip_norm   ClipGradNorms -- same page and section: a single clip
 *                   threshold over the L2 norm of all gradients taken
 *                   together; section "Values that stay on the card": the
 *                   norm and the factor are both formed on the device and
 *                   stay there until the host reads them.
 *   mta_adamw_step  AdamWSteps -- same page and section: a single launch
 *                   whatever the number of tensors, leaving every group as
 *                   the single-group AdamWStep would.  The element arithmetic is that
 *                   of "BendTorch main.bend", section "Optimizers" (adam_decay,
 *                   adam_m, adam_v, adam_w in PyTorch's order; packed
 *                   bfloat16 moments as in adamh_l / adamhv_l; bias
 *                   correction step = lr/(1-b1^t), bc2 = sqrt(1-b2^t) as in
 *                   Opt.at and the Training section, t = 1 on the first step).
 *   mta_step        any update rule of that "Optimizers" section (the Opt
 *                   type): AdamW, Adam with coupled decay (adam_grad), SGD
 *                   (sgd_l), momentum SGD (mom_l); optionally zeroing the
 *                   gradient as every step loop there does.
 *   mta_amp_*       the same steps under a dynamic loss scale kept in device
 *                   memory (Mica, same section: a float16 step divides its
 *                   loss scale out before the clip; section "Values that
 *                   stay on the card": the loss is scaled on the device),
 *                   with PyTorch's GradScaler rule for skipping and
 *                   rescaling.
 *   mta_list_set_weight_copies  bfloat16 (or, by mta_list_set_weight_copies_as,
 *                   float16) copies of the new weights (Mica, section
 *                   "float16 and bfloat16, whole").
 *   mta_list_set_no_decay  tensors that take no weight decay, in the same
 *                   launch as those that do.
 *   mta_list_create, mta_list_destroy  the list handle: the tensors of a
 *                   step described once, on the device, so that each call
 *                   above is a single launch over all of them (same page,
 *                   section "The whole model in one call").
 *
 * Memory and ownership.  Every w, g, m, v pointer is device memory owned by
 * the caller (for example a PyTorch tensor's data pointer).  The library never
 * allocates, frees or resizes caller memory.  A list handle owns small device
 * tables (one record per tile of up to 4096 elements: its buffer addresses,
 * length and alignment) and the scratch of the norm reduction; it is created
 * once and reused every step, so the caller's buffers must stay at the same
 * addresses for the handle's life.
 *
 * Layouts.
 *   w            float32, n elements; NULL for every tensor of a
 *                gradient-only list (norm and scale calls only).
 *   g            float32, bfloat16 or IEEE float16 (MTA_F32 / MTA_BF16 /
 *                MTA_F16, whole list), n elements.
 *   m, v         the optimizer state.  Either may be NULL for every tensor of
 *                a list (the choice is the same for all non-empty tensors):
 *                a list for SGD needs neither, one for momentum SGD needs m
 *                (float32), the Adam family needs both.
 *                MTA_MOM_F32: float32, n elements.
 *                MTA_MOM_BF16X2: packed bfloat16, two per 32-bit word, element
 *                2k in the low half of word k ("BendTorch main.bend", PTree
 *                comment).  On this little-endian device that is byte for
 *                byte a bfloat16 array of n elements, so a torch.bfloat16
 *                tensor's data pointer can be passed.  For odd n the last
 *                word's high half is never read or written; the buffer only
 *                needs 2n bytes.
 *   Alignment    float32 buffers 4 bytes, bfloat16 buffers 2 bytes.  A tensor
 *                whose buffers are all 16-byte aligned takes the 16-byte
 *                vector path.  One whose buffers all become aligned together
 *                after its first h elements (tensors at the same element
 *                offset of flat buffers, for instance) has those h elements
 *                processed one by one and the rest on the vector path: h < 64
 *                where that reaches a 128-byte boundary in every buffer, else
 *                h < 8 to 16 bytes.  Any other tensor is processed element by
 *                element.
 *   Buffers of one list must not overlap (checked at create).
 *
 * Streams.  Every device call enqueues its work on the caller's hipStream_t
 * (passed as void*, NULL = the null stream) and returns without waiting.  A
 * list is used on one stream at a time: the norm scratch is shared by all
 * calls on the list, so calls on one list that overlap in time race.  A list
 * handle also holds host state (a pending deferred scale factor, attached
 * weight copies), so one list is driven by one host thread at a time;
 * different lists are independent on every count.
 *
 * Errors.  Functions return MTA_OK (0) or a negative mta_status.  On failure
 * nothing has been enqueued and mta_last_error() (per host thread) says why.
 * Arguments are checked before any device work, so a request the library
 * cannot serve is turned away before anything runs (the reading taken of
 * "Mica 7.7", section "The card a program uses", where an invalid card
 * number stops the program at its start).  A fault inside a kernel is
 * asynchronous: work is queued on the caller's stream, and a failure of a
 * queued kernel is reported when the caller next synchronizes with that
 * stream (section "Upgrading": in an optimizing build such a failure
 * surfaces when the program next waits on the device).  With the environment variable MTA_DEBUG_SYNC=1 every call
 * that launches work waits for it before returning, so a kernel failure is
 * reported, as MTA_EHIP, by the call that launched it (section "Kernels
 * ready at the start": the debug tier waits for each kernel so the failure
 * is named where it happened).  MTA_DEBUG_SYNC is read once per process.
 */
#ifndef MTA_H
#define MTA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 2: mta_list_info_t gained weight_copy_type and norm_kept_tiles (72 bytes;
 *    a caller built against version 1 passes a 64-byte struct, so check
 *    mta_abi_version() before calling mta_list_info or mta_list_plan).
 * 3: mta_list_set_no_decay.
 * 4: mta_scale_device.
 * 5: mta_clip_norm_noalloc. */
#define MTA_ABI_VERSION 5

typedef struct mta_list mta_list; /* opaque */

typedef enum { MTA_F32 = 0, MTA_BF16 = 1, MTA_F16 = 2 } mta_gtype;
typedef enum { MTA_MOM_F32 = 0, MTA_MOM_BF16X2 = 1 } mta_mkind;

typedef enum {
  MTA_OK = 0,
  MTA_EINVAL = -1, /* bad argument value (null, negative size, bad hparam) */
  MTA_EALIGN = -2, /* pointer not aligned to its element size */
  MTA_EDTYPE = -3, /* unknown gradient type or moment kind */
  MTA_ENOMEM = -4, /* device or host allocation failed (create only) */
  MTA_EHIP = -5,   /* the HIP runtime reported an error */
  MTA_ESTATE = -6  /* call not allowed in the handle's current state */
} mta_status;

/* One parameter group: the caller's device buffers and the element count.
 * A gradient-only list gives g alone (w, m and v NULL for every tensor): it
 * serves mta_clip_norm, mta_clip_norm_joint, mta_scale and mta_scale_device,
 * and refuses every update and weight copies with MTA_ESTATE. */
typedef struct {
  float *w;  /* master weights, float32 [n]               (read, written) */
  void *g;   /* gradient, list's gradient type [n]        (read; written only by MTA_SCALE_INPLACE) */
  void *m;   /* first moment, list's m kind               (read, written) */
  void *v;   /* second moment, list's v kind              (read, written) */
  int64_t n; /* elements; 0 is allowed and skipped */
} mta_tensor;

/* AdamW hyperparameters as the caller states them (float64).  The kernel's
 * float32 constants are formed from these in float64 and rounded once:
 * step = lr/(1-beta1^t), bc2 = sqrt(1-beta2^t), c1 = 1-beta1, c2 = 1-beta2,
 * b2 = beta2, eps, dec = 1 - lr*weight_decay (decoupled decay). */
typedef struct {
  double lr, beta1, beta2, eps, weight_decay;
} mta_adamw_hparams;

/* Loss-scale state for float16 (or bfloat16) training with dynamic loss
 * scaling, kept by the caller in DEVICE memory (24 bytes, 8-byte aligned) and
 * read and written only by the device, so no step needs a host sync.  The
 * gradients hold scale * (true gradient).  "Mica 7.7", section "The whole
 * model in one call", has a float16 step divide its loss scale out of the
 * gradients before the clip; the reading taken for how the scale itself
 * moves is PyTorch's GradScaler, whose numerics the pages promise.  Initialise scale (e.g. 65536), the other fields to 0. */
typedef struct {
  float scale;            /* loss scale */
  float found_inf;        /* 1 when the last norm saw a non-finite unscaled
                             gradient, else 0 (set by mta_amp_clip_norm,
                             cleared by mta_amp_update) */
  int32_t growth_tracker; /* good steps since the scale last changed */
  int32_t reserved;
  int64_t step;           /* AdamW steps taken; the next one is step + 1 */
} mta_amp_state;

/* Shape of a list handle, for callers and tests that want to see it. */
typedef struct {
  int64_t count;       /* tensors in the list */
  int64_t elements;    /* sum of n */
  int64_t tiles;       /* work tiles (each covers up to tile_elems of one tensor) */
  int32_t tile_elems;  /* elements per tile */
  int32_t grid_update; /* workgroups of an update or in-place scale
                          launch: one per tile, at most 16,776,960 per
                          launch (a longer list takes several launches) */
  int32_t grid_norm;   /* workgroups of a norm launch (= norm partials) */
  int32_t device;      /* HIP device the list lives on */
  int32_t vector_tensors; /* tensors that take the 16-byte vector path
                             (after a head of under 64 elements) */
  int32_t gtype, mkind, vkind;
  int32_t weight_copies;  /* tensors with an attached 16-bit weight copy */
  int32_t state_buffers;  /* bit 0: the list has m; bit 1: it has v */
  int32_t weight_copy_type; /* MTA_BF16 or MTA_F16: the copies' format */
  int32_t norm_kept_tiles;  /* the list's last tiles, whose gradients the
                               norm reads with cache-allocating loads so
                               that the update finds them in the device's
                               memory-side cache (a cache policy only) */
} mta_list_info_t;

/* The update rules of "BendTorch main.bend", section "Optimizers" (the Opt
 * type and its comment; adam_grad, adam_decay, sgd_l, mom_l). */
typedef enum {
  MTA_OPT_ADAMW = 0,   /* decoupled decay: w' = w*(1 - lr*wd) */
  MTA_OPT_ADAM = 1,    /* coupled decay (dec = false): g' = g + f32(w*wd) */
  MTA_OPT_SGD = 2,     /* w = w + (-lr)*g */
  MTA_OPT_MOMENTUM = 3 /* buf = buf*mu + g; w = w + (-lr)*buf (PyTorch's
                          SGD momentum: no dampening, not Nesterov) */
} mta_opt_kind;

/* Flags of mta_opt. */
#define MTA_STEP_ZERO_GRAD 1 /* write +0 into every gradient element after the
                                step reads it, as every step loop of the
                                Optimizers section does */

/* One optimizer step's configuration.  Fields a rule does not use are
 * ignored, except weight_decay, which must be 0 for SGD and momentum (their
 * rules have no decay). */
typedef struct {
  int32_t kind;        /* mta_opt_kind */
  int32_t flags;       /* MTA_STEP_ZERO_GRAD or 0 */
  double lr;           /* all rules; finite, >= 0 */
  double beta1, beta2; /* Adam family: 0 <= beta < 1 */
  double eps;          /* Adam family: finite, >= 0 */
  double weight_decay; /* Adam family: finite, >= 0 */
  double momentum;     /* MTA_OPT_MOMENTUM: mu, finite, >= 0 */
} mta_opt;

/* Flags of mta_scale. */
#define MTA_SCALE_INPLACE 1 /* launch now: g = g * factor, rounded to g's type */
#define MTA_SCALE_DEFER 2   /* no launch: the next mta_clip_norm and
                               mta_adamw_step read f32(g * factor) in registers */

/* Create a list handle over `count` (>= 0) tensors described by the host array
 * `tensors` ("Mica 7.7", section "The whole model in one call": the calls
 * take every tensor of the model at once, one launch each; the handle is
 * that set of tensors, described once, so that no call re-describes it).
 * Validates every entry (null or misaligned buffers, negative sizes,
 * overlapping buffers, unknown types: MTA_EINVAL, MTA_EALIGN, MTA_EDTYPE,
 * before any device work), builds the tile tables and copies them to the
 * current device on `stream`, then waits for that copy.  Allocates device
 * memory (MTA_ENOMEM when that fails).  On success *out owns the handle;
 * release it with mta_list_destroy.  On failure *out is NULL and nothing
 * is allocated. */
int mta_list_create(const mta_tensor *tensors, int64_t count, int gtype,
                    int mkind, int vkind, void *stream, mta_list **out);

/* Free a handle: its device tables and norm scratch (the counterpart of
 * mta_list_create, same passage).  The caller must have synchronized every
 * stream that used it: a kernel still running on the handle's tables would
 * read freed memory.  NULL is accepted and ignored.  MTA_EHIP when the HIP
 * runtime refuses the free (the handle is released on the host either
 * way). */
int mta_list_destroy(mta_list *list);

/* ScaleTensors over the list's gradients.  MTA_SCALE_INPLACE launches one
 * kernel that writes g = g*factor (bfloat16 gradients are rounded back to
 * nearest-even).  MTA_SCALE_DEFER records the factor in the handle without a
 * launch; it applies to the next mta_clip_norm calls and to the next
 * mta_adamw_step, which clears it.  A second MTA_SCALE_DEFER before that step
 * returns MTA_ESTATE.  factor must be finite. */
int mta_scale(mta_list *list, float factor, int flags, void *stream);

/* ScaleTensors in place by a factor in DEVICE memory: one launch, the
 * kernel reads *d_factor (4-byte aligned float32) and writes
 * g = f32(g * factor), a 16-bit gradient rounded back to its type
 * (nearest-even, NaN -> 0xFFFF) -- MTA_SCALE_INPLACE with a factor the host
 * never sees, so no synchronization.  With the d_coef of mta_clip_norm this
 * clips the gradients themselves, as PyTorch's clip_grad_norm_ does (for a
 * caller that reads them or updates with another optimizer; the fused step
 * applies the coefficient in mta_adamw_step instead and needs no such pass).
 * Whatever the device holds is applied: a NaN factor makes every gradient
 * NaN.  A pending MTA_SCALE_DEFER factor is untouched and still applies to
 * the next reads.  d_factor NULL: MTA_EINVAL. */
int mta_scale_device(mta_list *list, const float *d_factor, void *stream);

/* ClipGradNorms: one launch.  Computes the joint L2 norm of f32(g*s) over
 * every gradient of the list (s = the deferred scale factor, else 1), and
 * coef = min(1, max_norm / (norm + 1e-6)) in float32 (a NaN norm gives a NaN
 * coef, an infinite norm gives 0).  Writes the float32 norm to *d_norm (device
 * pointer, may be NULL) and coef to *d_coef (device pointer, required).
 * The gradients are not modified: the coefficient is applied by
 * mta_adamw_step.  max_norm must be > 0 (infinity allowed, NaN not). */
int mta_clip_norm(mta_list *list, float max_norm, float *d_norm, float *d_coef,
                  void *stream);

/* mta_clip_norm for callers that cannot allocate device memory (code that
 * must not call hipMalloc: tight serving loops, harnesses that forbid it).
 * No list handle: the gradients are described by the host array `tensors`
 * (count >= 0 entries, checked as mta_list_create checks them; only g is
 * read, and w, m, v may all be NULL), `scale` is the unscale factor s of
 * mta_clip_norm (1 for none; finite), and the result is the norm and
 * coefficient mta_clip_norm writes for the same gradients, bit for bit
 * (same kernel, same launch shape).  The call allocates no device memory:
 * its tile table and reduction scratch live in one device array of the
 * library, 32 MiB, which each device the library runs on holds until the
 * process ends; it holds the table of up to about 2.09 million tiles of
 * 4096 elements (about 8.6e9 gradient elements in whole tiles), and a
 * larger list returns MTA_EINVAL before any device work.  The call stages
 * the table with copies on `stream`, launches the norm there and waits for
 * all of it before returning (it is not for graph capture).  The array is
 * shared by every call on a device and keeps the last call's contents:
 * each call re-initializes what it reads, and the library serializes its
 * calls within a process; calls from different processes use their own
 * copies. */
int mta_clip_norm_noalloc(const mta_tensor *tensors, int64_t count,
                          int gtype, float scale, float max_norm,
                          float *d_norm, float *d_coef, void *stream);

/* ClipGradNorms over several lists: a single clip threshold applied to the
 * L2 norm taken jointly over every gradient of every list ("Mica 7.7",
 * section "The whole model in one call"), each list keeping its own gradient type and its own pending
 * deferred factor (a bfloat16 program whose high-numerics parameters keep
 * float32 gradients: "Precision and numerics", Parameters).  One launch per
 * list, in order on `stream`; each adds its float64 sum of squares to the
 * running total (kept in lists[0]'s handle, so a list's total is never
 * rounded to float32 on the way) and writes the norm and coef of the total
 * so far, so the last launch leaves the joint ones in *d_norm and *d_coef.
 * nlists >= 1; no list may appear twice (MTA_EINVAL); all on the current
 * device.  nlists == 1 is mta_clip_norm.  Every list's mta_adamw_step (or
 * mta_step) then takes the same d_coef.  Like every call on a list, not
 * concurrent with other work on these lists. */
int mta_clip_norm_joint(mta_list *const *lists, int64_t nlists,
                        float max_norm, float *d_norm, float *d_coef,
                        void *stream);

/* AdamWSteps: one launch over every tensor of the list, step number t >= 1.
 * Per element, in float32 with every operation rounded on its own:
 *   ge = f32(f32(g*s) * coef)        (coef = *d_coef, or 1 when d_coef is NULL)
 *   w' = w*dec;  m = m + c1*(ge - m);  v = (v*b2) + ((c2*ge)*ge)
 *   packed kinds: m, v rounded to bfloat16 (nearest-even, NaN -> 0xFFFF),
 *   stored, and the rounded values used below
 *   w  = w' + ((-step*m) / ((sqrt(v)/bc2) + eps))
 * Hyperparameters follow PyTorch's AdamW checks: 0 <= beta1, beta2 < 1,
 * lr >= 0, eps >= 0, weight_decay >= 0, all finite.  Clears a deferred scale
 * factor. */
int mta_adamw_step(mta_list *list, const mta_adamw_hparams *hp, int64_t t,
                   const float *d_coef, void *stream);

/* One step of any rule of mta_opt_kind: one launch over every tensor.
 * Per element, ge = f32(f32(g*s) * coef) as in mta_adamw_step, then
 *   MTA_OPT_ADAMW     the update of mta_adamw_step;
 *   MTA_OPT_ADAM      ge' = ge + f32(w*wd) feeds m and v, and w is not
 *                     decayed (w' = w); otherwise as AdamW;
 *   MTA_OPT_SGD       w = w + f32(-lr)*ge;
 *   MTA_OPT_MOMENTUM  m = (m*mu) + ge; w = w + f32(-lr)*m   (m float32);
 * each operation rounded on its own; with MTA_STEP_ZERO_GRAD the gradient
 * element is then set to +0.  Requires the state buffers of the rule
 * (MTA_ESTATE when the list lacks them; MTA_EDTYPE for a packed momentum
 * buffer).  t >= 1 (read by the Adam family only).  Clears a deferred scale
 * factor, and writes the attached weight copies, as mta_adamw_step. */
int mta_step(mta_list *list, const mta_opt *opt, int64_t t,
             const float *d_coef, void *stream);

/* Attach bfloat16 copies of the weights: every later mta_adamw_step also
 * writes w16[i][k] = bfloat16(w_new[k]) (nearest-even, NaN -> 0xFFFF) for
 * each tensor i that has one, in the same launch ("Mica 7.7: a training step
 * on the card, in every float type", section "float16 and bfloat16, whole":
 * the weights stay float32 and a product reads them as bfloat16; "Precision
 * and numerics", section "bf16 regions": nearest-even is the one cast).
 * w16 is a host array of `count` device pointers in list order, each NULL (no
 * copy for that tensor) or the caller-owned address of n bfloat16 elements,
 * 2-byte aligned, overlapping no buffer of the list and no other copy.
 * w16 == NULL detaches every copy.  Rewrites the device tile table on
 * `stream` and waits for that upload; must not overlap a running step of
 * this list.  On failure the previous copies stay attached. */
int mta_list_set_weight_copies(mta_list *list, void *const *w16,
                               void *stream);

/* As mta_list_set_weight_copies, with the copies' format: copy_type MTA_BF16
 * (the same call) or MTA_F16, IEEE binary16 (Mica, section "float16 and
 * bfloat16, whole": the two 16-bit types stand side by side, and a float16
 * step reads its weights as float16).  A float16 copy is the nearest-even
 * binary16 value, +-Inf beyond its range (|w| >= 65520), with NaN -> 0xFFFF.
 * One format per list; the call sets it for every attached copy.
 * MTA_EDTYPE for any other copy_type (nothing changes then). */
int mta_list_set_weight_copies_as(mta_list *list, void *const *w16,
                                  int32_t copy_type, void *stream);

/* Flag tensors that take no weight decay (biases and normalization gains,
 * as a model usually keeps them), so that one list, and one launch per step,
 * covers a decay group and a no-decay group whose other hyperparameters are
 * equal.  Each flagged tensor is updated exactly as the same call with
 * weight_decay = 0 would update it alone ("Mica 7.7", section "The whole model
 * in one call": a multi-tensor step leaves each group as the single-group
 * step would):
 * MTA_OPT_ADAMW takes dec = 1 (w' = w*1), MTA_OPT_ADAM takes
 * ge' = ge + f32(w*0); SGD and momentum have no decay, so the flag changes
 * nothing there.  Applies to mta_adamw_step, mta_step, mta_amp_adamw_step and
 * mta_amp_step.  no_decay is a host array of `count` bytes in list order
 * (nonzero = no decay); NULL clears every flag.  Rewrites the device tile
 * table on `stream` and waits for that upload, like
 * mta_list_set_weight_copies (the two settings are independent and both
 * kept); must not overlap a running step of this list.  On failure the
 * previous flags stay. */
int mta_list_set_no_decay(mta_list *list, const uint8_t *no_decay,
                          void *stream);

/* Loss-scaled ClipGradNorms: as mta_clip_norm with the unscale factor
 * s = float32(1 / float64(d_amp->scale)) read on the device, and one more
 * output: d_amp->found_inf = 1 when the norm (of f32(g*s)) is not finite,
 * that is when some unscaled gradient is Inf or NaN, else 0.  d_amp is a
 * device pointer.  Not allowed while a host MTA_SCALE_DEFER factor is pending
 * (MTA_ESTATE). */
int mta_amp_clip_norm(mta_list *list, float max_norm, mta_amp_state *d_amp,
                      float *d_norm, float *d_coef, void *stream);

/* Loss-scaled ClipGradNorms over several lists: mta_clip_norm_joint with
 * the factor and the found-inf flag of mta_amp_clip_norm (found_inf = 1
 * when the joint norm is not finite).  No list may have a host
 * MTA_SCALE_DEFER factor pending (MTA_ESTATE). */
int mta_amp_clip_norm_joint(mta_list *const *lists, int64_t nlists,
                            float max_norm, mta_amp_state *d_amp,
                            float *d_norm, float *d_coef, void *stream);

/* Loss-scaled AdamWSteps: one launch that does nothing when
 * d_amp->found_inf is set; otherwise the step of mta_adamw_step with
 * t = d_amp->step + 1 and the unscale factor float32(1/float64(scale)), both
 * read on the device.  The device forms step = lr/(1-b1^t) and
 * bc2 = sqrt(1-b2^t) in float64 with b^t rounded once to the nearest float64
 * (the host form rounds b^t through libm's pow; the two agree except where
 * pow is not correctly rounded).  d_amp is not modified: the step counter
 * advances in mta_amp_update.  Same hyperparameter checks as
 * mta_adamw_step. */
int mta_amp_adamw_step(mta_list *list, const mta_adamw_hparams *hp,
                       const mta_amp_state *d_amp, const float *d_coef,
                       void *stream);

/* Loss-scaled mta_step: one launch.  When d_amp->found_inf is set the
 * update is skipped (w and the state untouched), but MTA_STEP_ZERO_GRAD
 * still zeroes every gradient (a caller that zeroes every iteration expects
 * it).  Otherwise the step of mta_step with the unscale factor
 * float32(1/float64(scale)) and, for the Adam family, t = d_amp->step + 1,
 * both read on the device as in mta_amp_adamw_step. */
int mta_amp_step(mta_list *list, const mta_opt *opt,
                 const mta_amp_state *d_amp, const float *d_coef,
                 void *stream);

/* After each loss-scaled step (PyTorch's GradScaler.update): one launch of
 * one thread.  If found_inf: scale *= backoff_factor, growth_tracker = 0.
 * Otherwise step += 1 and growth_tracker += 1; when it reaches
 * growth_interval, scale *= growth_factor (kept only if finite) and
 * growth_tracker = 0.  Products are formed in float64 and rounded to float32.
 * found_inf is cleared.  Requires growth_factor > 1, 0 < backoff_factor < 1,
 * growth_interval >= 1.  Needs no list. */
int mta_amp_update(mta_amp_state *d_amp, double growth_factor,
                   double backoff_factor, int32_t growth_interval,
                   void *stream);

/* Host only, no device work: the seven float32 constants the AdamW kernel
 * receives for step t, in the order {step, bc2, c1, c2, b2, eps, dec}
 * ("BendTorch main.bend", section "Optimizers": the Opt type's comment and
 * Opt.at for step and bc2, the adam_m comment for 1 - beta formed in
 * float64; section "Training": 1 - b^t with t = 1 first). */
int mta_adamw_scalars(const mta_adamw_hparams *hp, int64_t t, float out[7]);

/* Host only: describe a handle -- its tensors, tiles and launch grids (the
 * list of "Mica 7.7", section "The whole model in one call", as the device
 * sees it; section "The card a program uses": the device it lives on). */
int mta_list_info(const mta_list *list, mta_list_info_t *out);

/* Host only: the shape mta_list_create would give a list of these tensors,
 * without creating one.  The same argument, alignment and overlap checks
 * and the same errors as mta_list_create; on success *out holds count,
 * elements, tiles, tile_elems, vector_tensors, gtype, mkind, vkind,
 * state_buffers and norm_kept_tiles as the list would have them (weight
 * copies none, weight_copy_type MTA_BF16).  The device-dependent fields
 * are not set: grid_update = grid_norm = 0, device = -1.  The pointers are
 * compared, never dereferenced; no HIP call is made, so it also runs on a
 * host with no GPU (a caller can check how a flat-buffer layout cuts into
 * vector tiles before allocating it). */
int mta_list_plan(const mta_tensor *tensors, int64_t count, int gtype,
                  int mkind, int vkind, mta_list_info_t *out);

/* Message for the last failure on the calling host thread ("" if none),
 * naming the call and the argument or HIP error: a failure named where it
 * happened ("Mica 7.7", sections "Kernels ready at the start" and
 * "Upgrading").  The pointer stays valid until the thread's next call
 * into the library; a successful call clears it. */
const char *mta_last_error(void);

/* MTA_ABI_VERSION of the built library.  A binding compares it with the
 * version it was written for when it loads the library and refuses a
 * mismatch before any work ("Mica 7.7", section "The card a program uses":
 * a request that cannot be met is refused at the start). */
int mta_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MTA_H */
