/* san_host.c -- drives the host logic of libmta (validation, tile planning,
 * overlap checks, scalar preparation, error reporting) through the C ABI of
 * include/mta.h with no device: mta_list_plan over random tensor tables whose
 * addresses are never dereferenced, mta_adamw_scalars over valid and invalid
 * hyperparameters, and every call's refusal of a NULL list or bad argument
 * (refused before any device work).  Built by tests/test_sanitizers.py with
 * AddressSanitizer and UndefinedBehaviorSanitizer, against a build of
 * mta_host.cpp whose kernel launchers are stubs that are never reached.
 * Exit status 0 = clean. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mta.h"

static uint64_t rng = 0xD1B54A32D192ED03ull;
static uint64_t next64(void) { /* splitmix64 */
  uint64_t z = (rng += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static int failures = 0;
#define CHECK(cond, ...)                      \
  do {                                        \
    if (!(cond)) {                            \
      fprintf(stderr, "FAIL line %d: ", __LINE__); \
      fprintf(stderr, __VA_ARGS__);           \
      fprintf(stderr, "\n");                  \
      ++failures;                             \
    }                                         \
  } while (0)

/* a fake device address: a base in a realistic range plus an offset */
static void *addr(uint64_t base, uint64_t off) {
  return (void *)(uintptr_t)(base + off);
}

int main(void) {
  CHECK(mta_abi_version() == MTA_ABI_VERSION, "abi %d", mta_abi_version());

  /* scalars: valid over many t; every invalid hyperparameter refused */
  float sc[7];
  for (int64_t t = 1; t < (int64_t)1 << 40; t = t * 5 + 1) {
    mta_adamw_hparams hp = {3e-4, 0.9, 0.999, 1e-8, 0.1};
    CHECK(mta_adamw_scalars(&hp, t, sc) == MTA_OK, "t=%lld",
          (long long)t);
  }
  {
    const mta_adamw_hparams bad[] = {
        {-1e-3, 0.9, 0.999, 1e-8, 0.1}, {1e-3, 1.0, 0.999, 1e-8, 0.1},
        {1e-3, 0.9, 1.0, 1e-8, 0.1},    {1e-3, -0.1, 0.999, 1e-8, 0.1},
        {1e-3, 0.9, 0.999, -1.0, 0.1},  {1e-3, 0.9, 0.999, 1e-8, -0.1},
        {1.0 / 0.0, 0.9, 0.999, 1e-8, 0.1}};
    for (size_t i = 0; i < sizeof bad / sizeof bad[0]; ++i) {
      CHECK(mta_adamw_scalars(&bad[i], 1, sc) == MTA_EINVAL, "bad hp %zu", i);
      CHECK(strlen(mta_last_error()) > 0, "no message for bad hp %zu", i);
    }
    mta_adamw_hparams hp = {3e-4, 0.9, 0.999, 1e-8, 0.1};
    CHECK(mta_adamw_scalars(&hp, 0, sc) == MTA_EINVAL, "t=0");
    CHECK(mta_adamw_scalars(NULL, 1, sc) == MTA_EINVAL, "NULL hp");
    CHECK(mta_adamw_scalars(&hp, 1, NULL) == MTA_EINVAL, "NULL out");
  }

  /* every device call refuses a NULL list (or NULL state) before any work */
  {
    mta_adamw_hparams hp = {3e-4, 0.9, 0.999, 1e-8, 0.1};
    mta_opt o;
    memset(&o, 0, sizeof o);
    o.kind = MTA_OPT_ADAMW;
    o.lr = 1e-3;
    o.beta1 = 0.9;
    o.beta2 = 0.999;
    o.eps = 1e-8;
    float *fake = (float *)addr(0x7f0000000000ull, 0);
    uint8_t flags[2] = {1, 0};
    CHECK(mta_scale(NULL, 2.0f, MTA_SCALE_DEFER, NULL) == MTA_EINVAL, "scale");
    CHECK(mta_clip_norm(NULL, 1.0f, fake, fake + 1, NULL) == MTA_EINVAL,
          "clip");
    CHECK(mta_clip_norm_joint(NULL, 1, 1.0f, fake, fake + 1, NULL) ==
              MTA_EINVAL, "joint");
    {
      /* the allocation-free norm refuses before any HIP call */
      mta_tensor bad = {NULL, addr(0x7f1000000000ull, 1), NULL, NULL, 64};
      CHECK(mta_clip_norm_noalloc(&bad, 1, MTA_F32, 1.0f, 0.0f, fake,
                                  fake + 1, NULL) == MTA_EINVAL,
            "noalloc max_norm");
      CHECK(mta_clip_norm_noalloc(&bad, 1, MTA_F32, 1.0f, 1.0f, fake, NULL,
                                  NULL) == MTA_EINVAL, "noalloc coef");
      CHECK(mta_clip_norm_noalloc(&bad, 1, MTA_F32, 1.0f, 1.0f, fake,
                                  fake + 1, NULL) == MTA_EALIGN,
            "noalloc g align");
      CHECK(mta_clip_norm_noalloc(NULL, 1, MTA_F32, 1.0f, 1.0f, fake,
                                  fake + 1, NULL) == MTA_EINVAL,
            "noalloc NULL table");
      CHECK(mta_clip_norm_noalloc(&bad, 1, 7, 1.0f, 1.0f, fake, fake + 1,
                                  NULL) == MTA_EDTYPE, "noalloc gtype");
    }
    CHECK(mta_adamw_step(NULL, &hp, 1, NULL, NULL) == MTA_EINVAL, "adamw");
    CHECK(mta_step(NULL, &o, 1, NULL, NULL) == MTA_EINVAL, "step");
    CHECK(mta_list_set_weight_copies(NULL, NULL, NULL) == MTA_EINVAL,
          "copies");
    CHECK(mta_list_set_no_decay(NULL, flags, NULL) == MTA_EINVAL, "no decay");
    CHECK(mta_amp_update(NULL, 2.0, 0.5, 2000, NULL) == MTA_EINVAL, "amp");
    CHECK(mta_amp_update((mta_amp_state *)fake, 1.0, 0.5, 2000, NULL) ==
              MTA_EINVAL, "growth 1");
    CHECK(mta_amp_adamw_step(NULL, &hp, NULL, NULL, NULL) == MTA_EINVAL,
          "amp adamw");
    CHECK(mta_list_destroy(NULL) == MTA_OK, "destroy NULL");
    mta_list_info_t info;
    CHECK(mta_list_info(NULL, &info) == MTA_EINVAL, "info");
    CHECK(mta_list_plan(NULL, 1, MTA_F32, 0, 0, &info) == MTA_EINVAL,
          "plan NULL table");
    CHECK(mta_list_plan(NULL, -1, MTA_F32, 0, 0, &info) == MTA_EINVAL,
          "plan count<0");
    CHECK(mta_list_plan(NULL, 0, MTA_F32, 0, 0, NULL) == MTA_EINVAL,
          "plan NULL out");
    CHECK(mta_list_plan(NULL, 0, 7, 0, 0, &info) == MTA_EDTYPE, "gtype");
    CHECK(mta_scale_device(NULL, fake, NULL) == MTA_EINVAL, "scale dev");
    /* a gradient-only table is a list; m without w is not */
    mta_tensor go[2] = {{NULL, addr(0x7f2000000000ull, 0), NULL, NULL, 100},
                        {NULL, addr(0x7f2000000000ull, 512), NULL, NULL, 9}};
    CHECK(mta_list_plan(go, 2, MTA_F32, 0, 0, &info) == MTA_OK &&
              info.state_buffers == 0 && info.elements == 109,
          "gradient-only plan");
    go[1].m = addr(0x7f3000000000ull, 0);
    CHECK(mta_list_plan(go, 2, MTA_F32, 0, 0, &info) == MTA_EINVAL,
          "m without w");
  }

  /* random tables through the planner: sizes 0..2^20 with a few huge ones,
     buffers at random alignments in disjoint or overlapping ranges, m and v
     present or not; the result is OK or a refusal, and an accepted plan's
     counts are consistent */
  long plans = 0, accepted = 0;
  for (int trial = 0; trial < 600; ++trial) {
    const int64_t count = (int64_t)(next64() % 120);
    const int gtype = (int)(next64() % 3);
    const int mkind = (int)(next64() % 2), vkind = (int)(next64() % 2);
    const int state = (int)(next64() % 4); /* bit 0: m, bit 1: v */
    const int overlap = next64() % 10 == 0;
    const int odd_align = next64() % 4 == 0;
    mta_tensor *tab = malloc(sizeof(mta_tensor) * (count ? count : 1));
    if (!tab) return 2;
    const uint64_t bases[4] = {0x7f1000000000ull, 0x7f5000000000ull,
                               0x7f9000000000ull, 0x7fd000000000ull};
    uint64_t off[4] = {0, 0, 0, 0};
    int64_t elements = 0;
    for (int64_t i = 0; i < count; ++i) {
      int64_t n;
      const uint64_t r = next64();
      if (r % 50 == 0)
        n = 0;
      else if (r % 997 == 0)
        n = (int64_t)1 << 33; /* 8 Gi elements */
      else
        n = (int64_t)(next64() % ((uint64_t)1 << (1 + next64() % 20)));
      const uint64_t sizes[4] = {4, gtype == MTA_F32 ? 4u : 2u,
                                 mkind ? 2u : 4u, vkind ? 2u : 4u};
      for (int b = 0; b < 4; ++b) {
        uint64_t pad = odd_align ? (next64() % 8) * (sizes[b] / 2 ? 2 : 1) : 0;
        off[b] += pad;
        if (overlap && b == 1 && i > 0 && next64() % 3 == 0)
          off[b] -= 2; /* overlap the previous gradient */
      }
      tab[i].w = (float *)addr(bases[0], off[0]);
      tab[i].g = addr(bases[1], off[1]);
      tab[i].m = (state & 1) ? addr(bases[2], off[2]) : NULL;
      tab[i].v = (state & 2) ? addr(bases[3], off[3]) : NULL;
      tab[i].n = n;
      for (int b = 0; b < 4; ++b) off[b] += (uint64_t)n * sizes[b];
      elements += n;
    }
    mta_list_info_t info;
    memset(&info, 0, sizeof info);
    const int rc = mta_list_plan(tab, count, gtype, mkind, vkind, &info);
    ++plans;
    CHECK(rc == MTA_OK || rc == MTA_EINVAL || rc == MTA_EALIGN,
          "trial %d: rc %d", trial, rc);
    if (rc == MTA_OK) {
      ++accepted;
      CHECK(info.count == count && info.elements == elements,
            "trial %d: counts", trial);
      CHECK(info.tiles >= (elements + 4095) / 4096, "trial %d: tiles", trial);
      CHECK(info.norm_kept_tiles >= 0 && info.norm_kept_tiles <= info.tiles,
            "trial %d: kept", trial);
      CHECK(info.vector_tensors >= 0 && info.vector_tensors <= count,
            "trial %d: vector tensors", trial);
    } else {
      CHECK(strlen(mta_last_error()) > 0, "trial %d: no message", trial);
    }
    free(tab);
  }
  CHECK(accepted > 0 && accepted < plans, "accepted %ld of %ld", accepted,
        plans);
  if (failures) {
    fprintf(stderr, "san_host: %d failures\n", failures);
    return 1;
  }
  printf("san_host: %ld plans (%ld accepted) and every refusal clean\n",
         plans, accepted);
  return 0;
}
