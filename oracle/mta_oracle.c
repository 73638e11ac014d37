/*
 * mta_oracle.c -- plain, slow CPU oracle for the fused mixed-precision
 * clip + multi-tensor AdamW step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path
 * (the HIP library and its Python binding) never calls it, and it shares
 * no source, header, table or helper with that path.
 *
 * Every step below is the plain definition the pages give, one element at a
 * time, in the pages' order of operations.  Each float32 operation is its own
 * IEEE-754 round-to-nearest-even operation: the file must be compiled with
 * -ffp-contract=off and without -ffast-math (no fused multiply-add, no
 * reassociation), and sqrtf and '/' are the correctly rounded ones.
 *
 * Sources (cited by page title and section):
 *   [Mica]  "Mica 7.7: a training step on the card, in every float type",
 *           sections "The whole model in one call" (ClipGradNorms,
 *           AdamWSteps, ScaleTensors) and "Values that stay on the card".
 *   [Bend]  "BendTorch main.bend" (bendtorch@1.1.0.0), section "Optimizers:
 *           one pass over a parameter, its gradient and the two moment
 *           buffers": adam_decay, adam_m, adam_v, adam_w, ph_of_bits, ph_to,
 *           ph_half, ph_put, adamh_l, adamhv_l, Opt.at; the comment on the
 *           Opt type; the comment on the PTree type (packed layout); section
 *           "Training" (Train, ts4: q1 = 1 - b1^t, q2 = 1 - b2^t).
 *
 * Readings taken where the pages leave a step open (each is also listed with
 * its reasoning in the design notes of the repository):
 *   - Scalars are formed in float64 and rounded once to float32 (the Opt type
 *     comment says "as PyTorch computes them"; the comment on adam_m says
 *     PyTorch forms 1 - beta in float64).
 *   - The clip is PyTorch's clip_grad_norm_: coef = max / (norm + 1e-6) in
 *     float32, clamped to 1 with NaN passing through.  The norm itself is the
 *     joint L2 norm of the unscaled gradients, summed here in float64 with
 *     Neumaier compensation (effectively exact); the caller rounds it once.
 *   - Unscale and clip act in float32 registers: x = f32(g * s), then
 *     ge = f32(x * coef); gradients are not rewritten by the step.
 *   - The step does not zero the gradient unless asked to (PyTorch's step
 *     does not; every step loop of BendTorch's Optimizers section does, so
 *     zeroing is an option of the step).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define MTO_F32 0
#define MTO_BF16 1
#define MTO_F16 2
#define MTO_MOM_F32 0
#define MTO_MOM_BF16X2 1

/* ---------------------------------------------------------------------- */
/* bit casts                                                               */
/* ---------------------------------------------------------------------- */

static uint32_t bits_of(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  return u;
}

static float float_of(uint32_t u) {
  float x;
  memcpy(&x, &u, sizeof x);
  return x;
}

/* ---------------------------------------------------------------------- */
/* bfloat16 (BendTorch, Optimizers: ph_of_bits, ph_to)                    */
/* ---------------------------------------------------------------------- */

/* float32 bits -> bfloat16 bits, round to nearest, ties to even: add 0x7FFF
 * plus the lowest kept bit and keep the top half.  Any NaN becomes 0xFFFF. */
uint32_t mto_bf16_of_bits(uint32_t u) {
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0xFFFFu;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

/* bfloat16 bits -> float32: the bits move to the top half, exactly. */
float mto_f32_of_bf16(uint32_t h) { return float_of((h & 0xFFFFu) << 16); }

void mto_bf16_of_bits_array(int64_t n, const uint32_t *in, uint16_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint16_t)mto_bf16_of_bits(in[i]);
}

/* ---------------------------------------------------------------------- */
/* packed moments (BendTorch, PTree comment; ph_half, ph_put)             */
/* Element k lives in word k >> 1: even k in the low half, odd k in the   */
/* high half.  Reads and writes go through the 32-bit words themselves.   */
/* ---------------------------------------------------------------------- */

static uint32_t packed_get(const uint32_t *words, int64_t k) {
  uint32_t w = words[k >> 1];
  return (k & 1) ? (w >> 16) : (w & 0xFFFFu);
}

static void packed_put(uint32_t *words, int64_t k, uint32_t h) {
  uint32_t w = words[k >> 1];
  if (k & 1)
    w = (w & 0x0000FFFFu) | (h << 16);
  else
    w = (w & 0xFFFF0000u) | (h & 0xFFFFu);
  words[k >> 1] = w;
}

/* ---------------------------------------------------------------------- */
/* IEEE binary16 ("Mica 7.7": float16 stands beside float32 everywhere a  */
/* float goes, and a float16 step needs its gradients unscaled)           */
/* ---------------------------------------------------------------------- */

/* float16 bits -> float32, exact: sign, 5-bit exponent (bias 15), 10-bit
 * fraction; exponent 0 is zero or subnormal (fraction * 2^-24), 31 is Inf
 * or NaN (the fraction moves into the top of the float32 fraction). */
float mto_f32_of_f16(uint32_t h) {
  const uint32_t sign = (h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1Fu, f = h & 0x3FFu;
  if (e == 0) {
    const float mag = ldexpf((float)f, -24); /* exact: f < 2^10 */
    return sign ? -mag : mag;
  }
  if (e == 31) return float_of(sign | 0x7F800000u | (f << 13));
  return float_of(sign | ((e + 112u) << 23) | (f << 13));
}

/* float32 -> float16 bits, round to nearest, ties to even; overflow goes to
 * Inf; any NaN becomes 0xFFFF (all ones, read by analogy with the
 * bfloat16 rule). */
uint32_t mto_f16_of_f32(float x) {
  const uint32_t u = bits_of(x);
  const uint32_t sign = (u >> 16) & 0x8000u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0xFFFFu;
  if (a >= 0x477FF000u) return sign | 0x7C00u; /* |x| >= 65520 rounds up */
  if (a < 0x38800000u) {                        /* below 2^-14: subnormal */
    /* the subnormal step is 2^-24; |x| * 2^24 is exact in double and
     * rint() rounds it to nearest, ties to even */
    const double q = rint(ldexp((double)float_of(a), 24));
    return sign | (uint32_t)q; /* q == 1024 is the smallest normal */
  }
  uint32_t h = ((a >> 23) - 112u) << 10 | ((a >> 13) & 0x3FFu);
  const uint32_t rest = a & 0x1FFFu;
  if (rest > 0x1000u || (rest == 0x1000u && (h & 1u))) h += 1u;
  return sign | h;
}

void mto_f16_of_f32_array(int64_t n, const float *in, uint16_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint16_t)mto_f16_of_f32(in[i]);
}

void mto_f32_of_f16_array(int64_t n, const uint16_t *in, float *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = mto_f32_of_f16(in[i]);
}

/* gradient element k as float32 (bfloat16 and float16 convert exactly) */
static float grad_at(const void *g, int gtype, int64_t k) {
  if (gtype == MTO_BF16) return mto_f32_of_bf16(((const uint16_t *)g)[k]);
  if (gtype == MTO_F16) return mto_f32_of_f16(((const uint16_t *)g)[k]);
  return ((const float *)g)[k];
}

/* ---------------------------------------------------------------------- */
/* scalars (BendTorch: Opt type comment, Opt.at, comment on adam_m,       */
/* Training/ts4 for q1 and q2; t = 1 on the first step)                   */
/* out = {step, bc2, c1, c2, b2, eps, dec}                                 */
/* ---------------------------------------------------------------------- */

void mto_scalars(double lr, double b1, double b2, double eps, double wd,
                 int64_t t, float out[7]) {
  double q1 = 1.0 - pow(b1, (double)t);
  double q2 = 1.0 - pow(b2, (double)t);
  out[0] = (float)(lr / q1);       /* step = lr / (1 - b1^t) */
  out[1] = (float)sqrt(q2);        /* bc2  = sqrt(1 - b2^t)  */
  out[2] = (float)(1.0 - b1);      /* c1 */
  out[3] = (float)(1.0 - b2);      /* c2 */
  out[4] = (float)b2;              /* b2 as the multiplier of v */
  out[5] = (float)eps;             /* eps */
  out[6] = (float)(1.0 - lr * wd); /* AdamW's decay factor, w *= 1 - lr*wd */
}

/* ---------------------------------------------------------------------- */
/* ScaleTensors, in place (Mica, "The whole model in one call")           */
/* every cell times one factor; a bfloat16 cell is rounded back to bf16   */
/* ---------------------------------------------------------------------- */

void mto_scale_tensor(int64_t n, void *g, int gtype, float s) {
  for (int64_t k = 0; k < n; ++k) {
    if (gtype == MTO_BF16) {
      uint16_t *h = (uint16_t *)g;
      float x = mto_f32_of_bf16(h[k]) * s;
      h[k] = (uint16_t)mto_bf16_of_bits(bits_of(x));
    } else if (gtype == MTO_F16) {
      uint16_t *h = (uint16_t *)g;
      float x = mto_f32_of_f16(h[k]) * s;
      h[k] = (uint16_t)mto_f16_of_f32(x);
    } else {
      float *f = (float *)g;
      f[k] = f[k] * s;
    }
  }
}

/* ---------------------------------------------------------------------- */
/* joint sum of squares (Mica: ClipGradNorms, a single clip threshold    */
/* over the norm of all gradients).  x = f32(g * s) is the unscaled       */
/* gradient; x*x is exact in                                               */
/* float64, and the running sum carries a Neumaier compensation term, so  */
/* the result is the exact sum up to a few float64 roundings.             */
/* state[0] = running sum, state[1] = compensation; call once per tensor  */
/* in list order, then take state[0] + state[1].                          */
/* ---------------------------------------------------------------------- */

void mto_sumsq_accumulate(int64_t n, const void *g, int gtype, float s,
                          double state[2]) {
  double sum = state[0], comp = state[1];
  for (int64_t k = 0; k < n; ++k) {
    float x = grad_at(g, gtype, k) * s;
    double q = (double)x * (double)x;
    double t = sum + q;
    if (isfinite(t)) { /* an Inf or NaN sum stays what it is */
      if (fabs(sum) >= fabs(q))
        comp += (sum - t) + q;
      else
        comp += (q - t) + sum;
    }
    sum = t;
  }
  state[0] = sum;
  state[1] = comp;
}

/* ---------------------------------------------------------------------- */
/* clip coefficient (reading: PyTorch's clip_grad_norm_)                   */
/* coef = max / (norm + 1e-6) in float32; a coef above 1 becomes 1; the   */
/* comparison lets a NaN through and an infinite norm gives 0.            */
/* ---------------------------------------------------------------------- */

float mto_clip_coef(float max_norm, float norm) {
  float d = norm + 1e-6f;
  float c = max_norm / d;
  return (c > 1.0f) ? 1.0f : c;
}

/* ---------------------------------------------------------------------- */
/* AdamW over one tensor (BendTorch: adam_decay, adam_m, adam_v, adam_w;  */
/* adamh_l for packed m and v, adamhv_l for packed m with float32 v;       */
/* Mica: the multi-tensor step leaves each group as AdamWStep would).    */
/* sc = {step, bc2, c1, c2, b2, eps, dec} from mto_scalars.                */
/* A packed moment is rounded to bfloat16 and the weight update reads the  */
/* stored, rounded value.  The gradient is read, never written.            */
/* ---------------------------------------------------------------------- */

/* gradient element k set to +0 (every step loop of BendTorch's Optimizers
   section writes 0.0 into the gradient after reading it) */
static void grad_zero(void *g, int gtype, int64_t k) {
  if (gtype == MTO_F32)
    ((float *)g)[k] = 0.0f;
  else
    ((uint16_t *)g)[k] = 0; /* +0 in bfloat16 and in float16 */
}

/* The Adam family (BendTorch: adam_grad, adam_decay, adam_m, adam_v,
   adam_w; the comment on the Opt type: `dec` picks AdamW's decoupled decay,
   w *= 1 - lr*wd, over Adam's g += wd*w).
   coupled = 0 (AdamW): the gradient is used as it is and w is decayed by
   sc[6].  coupled = 1 (Adam): g' = ge + f32(w * l2) feeds both moments and w
   is not decayed (sc[6] is not read).  zero != 0: the gradient element is
   set to +0 after it is read. */
void mto_adam_tensor(int64_t n, float *w, void *g, int gtype, void *m,
                     int mkind, void *v, int vkind, float s, float coef,
                     const float sc[7], int coupled, float l2, int zero) {
  const float step = sc[0], bc2 = sc[1], c1 = sc[2], c2 = sc[3];
  const float b2 = sc[4], eps = sc[5], dec = sc[6];
  for (int64_t k = 0; k < n; ++k) {
    float x = grad_at(g, gtype, k) * s; /* unscale */
    float ge = x * coef;                /* clip    */
    if (zero) grad_zero(g, gtype, k);

    float wd;
    if (coupled) {
      ge = ge + (w[k] * l2); /* adam_grad (Adam) */
      wd = w[k];             /* adam_decay (Adam): no decay */
    } else {
      wd = w[k] * dec;       /* adam_decay (AdamW) */
    }

    float m0 = (mkind == MTO_MOM_BF16X2)
                   ? mto_f32_of_bf16(packed_get((const uint32_t *)m, k))
                   : ((float *)m)[k];
    float v0 = (vkind == MTO_MOM_BF16X2)
                   ? mto_f32_of_bf16(packed_get((const uint32_t *)v, k))
                   : ((float *)v)[k];

    float m1 = m0 + c1 * (ge - m0);        /* adam_m: lerp form */
    float v1 = (v0 * b2) + ((c2 * ge) * ge); /* adam_v */

    if (mkind == MTO_MOM_BF16X2) {
      uint32_t h = mto_bf16_of_bits(bits_of(m1));
      packed_put((uint32_t *)m, k, h);
      m1 = mto_f32_of_bf16(h);
    } else {
      ((float *)m)[k] = m1;
    }
    if (vkind == MTO_MOM_BF16X2) {
      uint32_t h = mto_bf16_of_bits(bits_of(v1));
      packed_put((uint32_t *)v, k, h);
      v1 = mto_f32_of_bf16(h);
    } else {
      ((float *)v)[k] = v1;
    }

    float denom = (sqrtf(v1) / bc2) + eps; /* adam_w */
    w[k] = wd + ((-step * m1) / denom);
  }
}

/* AdamW with the gradient only read (the hot path's own form) */
void mto_adamw_tensor(int64_t n, float *w, const void *g, int gtype, void *m,
                      int mkind, void *v, int vkind, float s, float coef,
                      const float sc[7]) {
  mto_adam_tensor(n, w, (void *)g, gtype, m, mkind, v, vkind, s, coef, sc, 0,
                  0.0f, 0);
}

/* ---------------------------------------------------------------------- */
/* SGD (BendTorch sgd_l: w <- w + (-lr)*g, as PyTorch's p.add_(g,         */
/* alpha=-lr)) on the unscaled, clipped gradient; lr is the float32 value. */
/* ---------------------------------------------------------------------- */

void mto_sgd_tensor(int64_t n, float *w, void *g, int gtype, float s,
                    float coef, float lr, int zero) {
  const float nlr = -lr;
  for (int64_t k = 0; k < n; ++k) {
    float x = grad_at(g, gtype, k) * s;
    float ge = x * coef;
    if (zero) grad_zero(g, gtype, k);
    w[k] = w[k] + (nlr * ge);
  }
}

/* ---------------------------------------------------------------------- */
/* SGD with momentum (BendTorch mom_l: buf <- buf*mu + g; w <- w +        */
/* (-lr)*buf, as PyTorch's SGD with momentum, no dampening, not Nesterov; */
/* the buffer starts at zero).  buf is float32.                            */
/* ---------------------------------------------------------------------- */

void mto_momentum_tensor(int64_t n, float *w, void *g, int gtype, float *buf,
                         float s, float coef, float lr, float mu, int zero) {
  const float nlr = -lr;
  for (int64_t k = 0; k < n; ++k) {
    float x = grad_at(g, gtype, k) * s;
    float ge = x * coef;
    if (zero) grad_zero(g, gtype, k);
    float nb = (buf[k] * mu) + ge;
    buf[k] = nb;
    w[k] = w[k] + (nlr * nb);
  }
}

/* ---------------------------------------------------------------------- */
/* bfloat16 copy of the updated weights ("Mica 7.7", section "float16 and */
/* bfloat16, whole": weights stay float32 and a product reads them as     */
/* bfloat16; "Precision and numerics": nearest-even is the one cast).     */
/* out[k] = bfloat16(w[k]) by the same nearest-even rule as the moments.  */
/* ---------------------------------------------------------------------- */

void mto_weight_copy(int64_t n, const float *w, uint16_t *out) {
  for (int64_t k = 0; k < n; ++k)
    out[k] = (uint16_t)mto_bf16_of_bits(bits_of(w[k]));
}

/* ---------------------------------------------------------------------- */
/* Dynamic loss scaling on the device (the AMP state a caller keeps in    */
/* device memory).  Reading: PyTorch's GradScaler, as [Mica] promises     */
/* PyTorch's numerics.                                                     */
/* ---------------------------------------------------------------------- */

/* b^t rounded once to the nearest float64: square-and-multiply in
 * __float128 (113-bit significand; the error of ~2*63 roundings stays near
 * 2^-106 relative), then one rounding to double. */
double mto_pow_rn(double b, int64_t t) {
  __float128 r = 1, x = b;
  uint64_t e = (uint64_t)t;
  while (e) {
    if (e & 1u) r *= x;
    x *= x;
    e >>= 1;
  }
  return (double)r;
}

/* The step constants from the device step counter: as mto_scalars, with
 * 1 - b^t formed from the correctly rounded power. */
void mto_scalars_rn(double lr, double b1, double b2, double eps, double wd,
                    int64_t t, float out[7]) {
  const double q1 = 1.0 - mto_pow_rn(b1, t);
  const double q2 = 1.0 - mto_pow_rn(b2, t);
  out[0] = (float)(lr / q1);
  out[1] = (float)sqrt(q2);
  out[2] = (float)(1.0 - b1);
  out[3] = (float)(1.0 - b2);
  out[4] = (float)b2;
  out[5] = (float)eps;
  out[6] = (float)(1.0 - lr * wd);
}

/* The unscale factor of a loss scale S: float32(1 / float64(S)). */
float mto_inv_scale(float scale) { return (float)(1.0 / (double)scale); }

/* After a step: a step with a non-finite unscaled gradient backs the scale
 * off and resets the tracker; otherwise the step counts, the tracker grows,
 * and every `interval` good steps the scale grows (when the grown scale is
 * finite).  The found-inf flag is cleared for the next step.  Products are
 * formed in float64 and rounded once to float32. */
void mto_amp_update(float *scale, int32_t *tracker, float *found_inf,
                    int64_t *step, double growth, double backoff,
                    int32_t interval) {
  if (*found_inf != 0.0f) {
    *scale = (float)((double)*scale * backoff);
    *tracker = 0;
  } else {
    *step += 1;
    const int32_t good = *tracker + 1;
    if (good == interval) {
      const float grown = (float)((double)*scale * growth);
      if (isfinite(grown)) *scale = grown;
      *tracker = 0;
    } else {
      *tracker = good;
    }
  }
  *found_inf = 0.0f;
}
