/* san_oracle.c -- drives every function of oracle/mta_oracle.c over edge
 * sizes and every type combination, on heap buffers of exactly the size each
 * function's contract names (packed moments: ceil(n/2) 32-bit words), so that
 * AddressSanitizer and UndefinedBehaviorSanitizer builds report any access
 * outside them or any undefined operation.  Test infrastructure: built and
 * run by tests/test_sanitizers.py on the CPU.  Exit status 0 = clean. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* the oracle's exported functions (oracle/mta_oracle.c) */
uint32_t mto_bf16_of_bits(uint32_t u);
float mto_f32_of_bf16(uint32_t h);
void mto_bf16_of_bits_array(int64_t n, const uint32_t *in, uint16_t *out);
float mto_f32_of_f16(uint32_t h);
uint32_t mto_f16_of_f32(float x);
void mto_f16_of_f32_array(int64_t n, const float *in, uint16_t *out);
void mto_f32_of_f16_array(int64_t n, const uint16_t *in, float *out);
void mto_scalars(double lr, double b1, double b2, double eps, double wd,
                 int64_t t, float out[7]);
void mto_scalars_rn(double lr, double b1, double b2, double eps, double wd,
                    int64_t t, float out[7]);
double mto_pow_rn(double b, int64_t t);
void mto_scale_tensor(int64_t n, void *g, int gtype, float s);
void mto_sumsq_accumulate(int64_t n, const void *g, int gtype, float s,
                          double state[2]);
float mto_clip_coef(float max_norm, float norm);
void mto_adam_tensor(int64_t n, float *w, void *g, int gtype, void *m,
                     int mkind, void *v, int vkind, float s, float coef,
                     const float sc[7], int coupled, float l2, int zero);
void mto_adamw_tensor(int64_t n, float *w, const void *g, int gtype, void *m,
                      int mkind, void *v, int vkind, float s, float coef,
                      const float sc[7]);
void mto_sgd_tensor(int64_t n, float *w, void *g, int gtype, float s,
                    float coef, float lr, int zero);
void mto_momentum_tensor(int64_t n, float *w, void *g, int gtype, float *buf,
                         float s, float coef, float lr, float mu, int zero);
void mto_weight_copy(int64_t n, const float *w, uint16_t *out);
float mto_inv_scale(float scale);
void mto_amp_update(float *scale, int32_t *tracker, float *found_inf,
                    int64_t *step, double growth, double backoff,
                    int32_t interval);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next32(void) { /* splitmix64, high half */
  uint64_t z = (rng += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return (uint32_t)((z ^ (z >> 31)) >> 32);
}
/* a float of any bit pattern one time in eight (NaN, Inf, subnormal
   included), else a moderate value */
static float any_float(void) {
  uint32_t u = next32();
  if ((u & 7u) == 0) {
    uint32_t b = next32();
    float f;
    memcpy(&f, &b, 4);
    return f;
  }
  return ((float)(int32_t)next32()) * 1e-11f;
}

static void *xmalloc(size_t bytes) {
  void *p = malloc(bytes ? bytes : 1);
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(2);
  }
  return p;
}

/* a gradient buffer of n elements of type gtype with random contents */
static void *grad_buf(int64_t n, int gtype) {
  size_t es = gtype == 0 ? 4 : 2;
  unsigned char *g = xmalloc((size_t)n * es);
  for (int64_t k = 0; k < n; ++k) {
    if (gtype == 0) {
      float f = any_float();
      memcpy(g + 4 * k, &f, 4);
    } else {
      uint16_t h = (uint16_t)next32();
      memcpy(g + 2 * k, &h, 2);
    }
  }
  return g;
}

/* a moment buffer: n float32, or ceil(n/2) packed words */
static void *mom_buf(int64_t n, int kind) {
  size_t bytes = kind == 0 ? (size_t)n * 4 : (size_t)((n + 1) / 2) * 4;
  uint32_t *m = xmalloc(bytes);
  for (size_t k = 0; k < bytes / 4; ++k) {
    float f = any_float();
    memcpy(&m[k], &f, 4);
    if (kind == 1) m[k] = next32();
  }
  return m;
}

static float *f32_buf(int64_t n) {
  float *w = xmalloc((size_t)n * 4);
  for (int64_t k = 0; k < n; ++k) w[k] = any_float();
  return w;
}

int main(void) {
  static const int64_t sizes[] = {0, 1, 2, 3, 7, 8, 9, 15, 17, 63, 64, 65,
                                  4095, 4096, 4097};
  const int nsizes = (int)(sizeof sizes / sizeof sizes[0]);
  long calls = 0;

  /* conversions over every 16-bit pattern and many 32-bit ones */
  for (uint32_t h = 0; h < 65536; ++h) {
    float f = mto_f32_of_bf16(h);
    float e = mto_f32_of_f16(h);
    uint32_t u;
    memcpy(&u, &f, 4);
    (void)mto_bf16_of_bits(u);
    (void)mto_f16_of_f32(e);
    (void)mto_f16_of_f32(f);
  }
  for (int i = 0; i < 1 << 20; ++i) {
    uint32_t u = next32();
    float f;
    memcpy(&f, &u, 4);
    (void)mto_bf16_of_bits(u);
    (void)mto_f16_of_f32(f);
  }
  calls += 2;

  for (int si = 0; si < nsizes; ++si) {
    const int64_t n = sizes[si];
    /* array conversions */
    {
      uint32_t *in = xmalloc((size_t)n * 4);
      uint16_t *out = xmalloc((size_t)n * 2);
      float *f = f32_buf(n);
      for (int64_t k = 0; k < n; ++k) in[k] = next32();
      mto_bf16_of_bits_array(n, in, out);
      mto_f16_of_f32_array(n, f, out);
      mto_f32_of_f16_array(n, out, f);
      mto_weight_copy(n, f, out);
      free(in);
      free(out);
      free(f);
      calls += 4;
    }
    for (int gtype = 0; gtype < 3; ++gtype) {
      /* scale, norm */
      void *g = grad_buf(n, gtype);
      double st[2] = {0.0, 0.0};
      mto_sumsq_accumulate(n, g, gtype, 0.5f, st);
      mto_scale_tensor(n, g, gtype, 0.25f);
      mto_scale_tensor(n, g, gtype, any_float());
      (void)mto_clip_coef(1.0f, (float)sqrt(st[0] + st[1]));
      calls += 4;
      /* the Adam family, every moment kind, coupled or not, zeroing or not */
      for (int mk = 0; mk < 2; ++mk)
        for (int vk = 0; vk < 2; ++vk)
          for (int coupled = 0; coupled < 2; ++coupled)
            for (int zero = 0; zero < 2; ++zero) {
              float *w = f32_buf(n);
              void *m = mom_buf(n, mk), *v = mom_buf(n, vk);
              float sc[7];
              mto_scalars(3e-4, 0.9, 0.999, 1e-8, 0.1,
                          1 + (int64_t)(next32() % 1000), sc);
              mto_adam_tensor(n, w, g, gtype, m, mk, v, vk, 1.0f / 65536,
                              0.37f, sc, coupled, 0.1f, zero);
              mto_adamw_tensor(n, w, g, gtype, m, mk, v, vk, 1.0f, 1.0f, sc);
              free(w);
              free(m);
              free(v);
              calls += 2;
            }
      /* SGD and momentum */
      for (int zero = 0; zero < 2; ++zero) {
        float *w = f32_buf(n), *buf = f32_buf(n);
        mto_sgd_tensor(n, w, g, gtype, 0.5f, 0.9f, 0.05f, zero);
        mto_momentum_tensor(n, w, g, gtype, buf, 2.0f, 1.0f, 0.05f, 0.9f,
                            zero);
        free(w);
        free(buf);
        calls += 2;
      }
      free(g);
    }
  }

  /* scalars and the correctly rounded power over wide ranges of t */
  for (int64_t t = 1; t < (int64_t)1 << 40; t = t * 3 + 1) {
    float sc[7];
    mto_scalars(1e-3, 0.9, 0.999, 1e-8, 0.01, t, sc);
    mto_scalars_rn(1e-3, 0.9, 0.999, 1e-8, 0.01, t, sc);
    (void)mto_pow_rn(0.999, t);
    (void)mto_pow_rn(0.0, t);
    calls += 4;
  }
  /* loss-scale updates: growth to overflow, backoff to underflow, and the
     largest growth interval */
  {
    float scale = 65536.0f, found = 0.0f;
    int32_t tracker = 0;
    int64_t step = 0;
    for (int i = 0; i < 400; ++i) {
      mto_amp_update(&scale, &tracker, &found, &step, 2.0, 0.5, 1);
      (void)mto_inv_scale(scale);
    }
    for (int i = 0; i < 400; ++i) {
      found = 1.0f;
      mto_amp_update(&scale, &tracker, &found, &step, 2.0, 0.5, 2000);
      (void)mto_inv_scale(scale);
    }
    tracker = 2147483645;
    for (int i = 0; i < 4; ++i)
      mto_amp_update(&scale, &tracker, &found, &step, 2.0, 0.5, 2147483647);
    calls += 804;
  }
  printf("san_oracle: %ld calls clean\n", calls);
  return 0;
}
