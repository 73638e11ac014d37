/*
 * abi_demo.c -- a plain C program that drives libmta through include/mta.h
 * alone (no Python, no torch): three steps of deferred unscale, joint-norm
 * clip and AdamW over a three-tensor list, on the null stream.  It prints
 * the device norm and clip coefficient of every step and the final w, m and
 * v as float32 bit patterns; tests/test_gpu_c_abi.py rebuilds the same
 * inputs and checks every line against the CPU oracle.
 *
 * Inputs are exact dyadic values (k / 1024 and k / 2048 for small integers
 * k), so both sides form them without rounding.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mta.h"

#define NT 3
#define CHECK_HIP(x)                                                     \
  do {                                                                   \
    hipError_t e_ = (x);                                                 \
    if (e_ != hipSuccess) {                                              \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));            \
      return 2;                                                          \
    }                                                                    \
  } while (0)
#define CHECK_MTA(x)                                                     \
  do {                                                                   \
    int r_ = (x);                                                        \
    if (r_ != MTA_OK) {                                                  \
      fprintf(stderr, "%s: %d %s\n", #x, r_, mta_last_error());          \
      return 3;                                                          \
    }                                                                    \
  } while (0)

/* element i of the whole list (tensors concatenated in list order) */
static float w_init(int64_t i) {
  return (float)((i * 37) % 101 - 50) / 1024.0f;
}
static float g_at(int64_t i, int t) {
  return (float)((i * 53 + t * 11) % 97 - 48) / 2048.0f;
}

static uint32_t bits(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  return u;
}

int main(void) {
  const int64_t n[NT] = {4096 * 2 + 5, 777, 1};
  int64_t base[NT], total = 0;
  for (int k = 0; k < NT; ++k) {
    base[k] = total;
    total += n[k];
  }
  float *host = (float *)malloc((size_t)total * sizeof(float));
  if (!host) return 4;
  float *dw[NT], *dg[NT], *dm[NT], *dv[NT];
  mta_tensor ts[NT];
  for (int k = 0; k < NT; ++k) {
    const size_t bytes = (size_t)n[k] * sizeof(float);
    CHECK_HIP(hipMalloc((void **)&dw[k], bytes));
    CHECK_HIP(hipMalloc((void **)&dg[k], bytes));
    CHECK_HIP(hipMalloc((void **)&dm[k], bytes));
    CHECK_HIP(hipMalloc((void **)&dv[k], bytes));
    CHECK_HIP(hipMemset(dm[k], 0, bytes));
    CHECK_HIP(hipMemset(dv[k], 0, bytes));
    for (int64_t i = 0; i < n[k]; ++i) host[i] = w_init(base[k] + i);
    CHECK_HIP(hipMemcpy(dw[k], host, bytes, hipMemcpyHostToDevice));
    ts[k].w = dw[k];
    ts[k].g = dg[k];
    ts[k].m = dm[k];
    ts[k].v = dv[k];
    ts[k].n = n[k];
  }
  mta_list *L = NULL;
  CHECK_MTA(mta_list_create(ts, NT, MTA_F32, MTA_MOM_F32, MTA_MOM_F32, NULL,
                            &L));
  float *d_out;
  CHECK_HIP(hipMalloc((void **)&d_out, 2 * sizeof(float)));
  const mta_adamw_hparams hp = {1e-3, 0.9, 0.999, 1e-8, 0.1};
  for (int t = 1; t <= 3; ++t) {
    for (int k = 0; k < NT; ++k) {
      for (int64_t i = 0; i < n[k]; ++i) host[i] = g_at(base[k] + i, t);
      CHECK_HIP(hipMemcpy(dg[k], host, (size_t)n[k] * sizeof(float),
                          hipMemcpyHostToDevice));
    }
    CHECK_MTA(mta_scale(L, 0.5f, MTA_SCALE_DEFER, NULL));
    CHECK_MTA(mta_clip_norm(L, 0.05f, d_out, d_out + 1, NULL));
    CHECK_MTA(mta_adamw_step(L, &hp, t, d_out + 1, NULL));
    float out[2];
    CHECK_HIP(hipMemcpy(out, d_out, sizeof out, hipMemcpyDeviceToHost));
    printf("step %d norm %08x coef %08x\n", t, bits(out[0]), bits(out[1]));
  }
  const char *names[3] = {"w", "m", "v"};
  for (int k = 0; k < NT; ++k) {
    float *bufs[3] = {dw[k], dm[k], dv[k]};
    for (int b = 0; b < 3; ++b) {
      CHECK_HIP(hipMemcpy(host, bufs[b], (size_t)n[k] * sizeof(float),
                          hipMemcpyDeviceToHost));
      printf("%s %d", names[b], k);
      for (int64_t i = 0; i < n[k]; ++i) printf(" %08x", bits(host[i]));
      printf("\n");
    }
  }
  CHECK_MTA(mta_list_destroy(L));
  for (int k = 0; k < NT; ++k) {
    CHECK_HIP(hipFree(dw[k]));
    CHECK_HIP(hipFree(dg[k]));
    CHECK_HIP(hipFree(dm[k]));
    CHECK_HIP(hipFree(dv[k]));
  }
  CHECK_HIP(hipFree(d_out));
  free(host);
  return 0;
}
