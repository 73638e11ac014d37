// mta_internal.h -- types shared by the host runtime and the gfx950 kernels
// of libmta.  Not part of the public C ABI (that is include/mta.h).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace mta {

// A tile is the work of one workgroup iteration: up to kTileElems consecutive
// elements of one tensor, starting at a multiple of kTileElems.  Tiles never
// straddle tensors, so every vector access inside a tile stays in one buffer.
constexpr int kBlock = 256;       // threads per workgroup (4 wave64s)
constexpr int kTileElems = 4096;  // 16 elements per thread

// One tensor of the list as the kernels see it (device-resident table).
struct TensorDesc {
  float *w;
  const void *g;
  void *m;
  void *v;
  int64_t n;
  uint32_t vec;  // 1: all four buffers 16-byte aligned -> vector path
  uint32_t pad;
};
static_assert(sizeof(TensorDesc) == 48, "descriptor layout");

struct Tile {
  uint32_t tensor;  // index into the descriptor table
  uint32_t index;   // tile number inside the tensor: first element = index * kTileElems
};
static_assert(sizeof(Tile) == 8, "tile layout");

// Per-call float32 constants of the AdamW step (formed on the host in float64,
// rounded once).  nstep = -step: negation is exact, so (-step)*m is unchanged.
struct StepScalars {
  float nstep, bc2, c1, c2, b2, eps, dec;
  float s;  // deferred unscale factor (1 when none)
};

struct Work {
  const TensorDesc *td;
  const Tile *tiles;
  uint32_t ntiles;
  int grid;
  hipStream_t stream;
};

// Norm scratch: one float64 partial per norm workgroup, then the ticket.
struct NormScratch {
  double *partials;
  unsigned int *ticket;
};

hipError_t launch_adamw(int gtype, int mkind, int vkind, const Work &work,
                        const StepScalars &sc, const float *d_coef);
hipError_t launch_sumsq(int gtype, const Work &work, float s, float max_norm,
                        NormScratch scratch, float *d_norm, float *d_coef);
hipError_t launch_scale(int gtype, const Work &work, float s);

}  // namespace mta
