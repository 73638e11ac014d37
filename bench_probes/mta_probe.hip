// mta_probe.hip -- HBM ceiling probes for the update's traffic mix.
//
// Measurement instruments, not part of the optimizer: bench.py --probes
// times them to show what a kernel with the same bytes as an update launch
// can reach on this device when it does (almost) no arithmetic.  Each probe
// streams whole 4096-element tiles with the same contiguous lane mapping as
// the update kernels (4 elements per lane per access: 16 bytes of a float32
// buffer, 8 of a 16-bit one), nontemporal loads and stores, and a
// grid-stride loop over tiles with two tiles of loads in flight (the
// write-only probe has no loads).  n must be
// a multiple of 4096 (the caller sizes the buffers); every index is below n.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

#define PG __attribute__((address_space(1)))
typedef float pf4 __attribute__((ext_vector_type(4)));
typedef uint32_t pu2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kTile = 4096;
constexpr int kGroups = kTile / (kThreads * 4);  // 4 accesses per buffer

template <int B>  // element bytes: 4 or 2
using raw_t = typename std::conditional<B == 4, pf4, pu2>::type;

template <int B>
__device__ __forceinline__ raw_t<B> ld(const void *p, uint64_t e) {
  return __builtin_nontemporal_load((const PG raw_t<B> *)p + e / 4);
}
template <int B>
__device__ __forceinline__ void st(void *p, uint64_t e, raw_t<B> x) {
  __builtin_nontemporal_store(x, (PG raw_t<B> *)p + e / 4);
}
__device__ __forceinline__ pf4 mix(pf4 a, pf4 b) { return a + b; }
__device__ __forceinline__ pu2 mix(pu2 a, pf4 b) {
  return a + pu2{__float_as_uint(b.x), __float_as_uint(b.y)};
}
__device__ __forceinline__ pf4 mix(pf4 a, pu2 b) {
  return a + pf4{__uint_as_float(b.x), __uint_as_float(b.y), 0.0f, 0.0f};
}

// read w, g, m, v; write w, m, v (the update's bytes), two tiles per trip
template <int GB, int MB, int VB>
__global__ void __launch_bounds__(kThreads)
k_probe_mix(void *w, const void *g, void *m, void *v, uint64_t ntiles) {
  const uint64_t l4 = threadIdx.x * 4;
  for (uint64_t t = blockIdx.x * 2ull; t < ntiles; t += gridDim.x * 2ull) {
    pf4 W[2][kGroups];
    raw_t<GB> Gr[2][kGroups];
    raw_t<MB> M[2][kGroups];
    raw_t<VB> V[2][kGroups];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint64_t tt = t + u < ntiles ? t + u : ntiles - 1;
#pragma unroll
      for (int j = 0; j < kGroups; ++j) {
        const uint64_t e = tt * kTile + j * (kThreads * 4) + l4;
        W[u][j] = ld<4>(w, e);
        Gr[u][j] = ld<GB>(g, e);
        M[u][j] = ld<MB>(m, e);
        V[u][j] = ld<VB>(v, e);
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (t + u >= ntiles) continue;
#pragma unroll
      for (int j = 0; j < kGroups; ++j) {
        const uint64_t e = (t + u) * kTile + j * (kThreads * 4) + l4;
        st<4>(w, e, mix(W[u][j], Gr[u][j]));
        st<MB>(m, e, mix(M[u][j], W[u][j]));
        st<VB>(v, e, mix(V[u][j], W[u][j]));
      }
    }
  }
}

// read only: 16 bytes per lane; the sum is stored only if it equals a value
// it never takes, so the loads are kept and nothing is written
__global__ void __launch_bounds__(kThreads)
k_probe_read(const void *a, uint64_t ntiles, float *sink) {
  const uint64_t l4 = threadIdx.x * 4;
  pf4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (uint64_t t = blockIdx.x * 2ull; t < ntiles; t += gridDim.x * 2ull) {
    pf4 x[2][kGroups];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint64_t tt = t + u < ntiles ? t + u : ntiles - 1;
#pragma unroll
      for (int j = 0; j < kGroups; ++j)
        x[u][j] = ld<4>(a, tt * kTile + j * (kThreads * 4) + l4);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int j = 0; j < kGroups; ++j) acc += x[u][j];
  }
  if (acc.x + acc.y + acc.z + acc.w == -1234.5f) sink[threadIdx.x] = acc.x;
}

// write only: 16 bytes per lane of a fixed value, one tile per trip
__global__ void __launch_bounds__(kThreads)
k_probe_write(void *b, uint64_t ntiles) {
  const uint64_t l4 = threadIdx.x * 4;
  const pf4 x = {1.0f, 1.0f, 1.0f, 1.0f};
  for (uint64_t t = blockIdx.x; t < ntiles; t += gridDim.x)
#pragma unroll
    for (int j = 0; j < kGroups; ++j)
      st<4>(b, t * kTile + j * (kThreads * 4) + l4, x);
}

// copy: 16 bytes per lane read and written
__global__ void __launch_bounds__(kThreads)
k_probe_copy(const void *a, void *b, uint64_t ntiles) {
  const uint64_t l4 = threadIdx.x * 4;
  for (uint64_t t = blockIdx.x * 2ull; t < ntiles; t += gridDim.x * 2ull) {
    pf4 x[2][kGroups];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint64_t tt = t + u < ntiles ? t + u : ntiles - 1;
#pragma unroll
      for (int j = 0; j < kGroups; ++j)
        x[u][j] = ld<4>(a, tt * kTile + j * (kThreads * 4) + l4);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (t + u >= ntiles) continue;
#pragma unroll
      for (int j = 0; j < kGroups; ++j)
        st<4>(b, (t + u) * kTile + j * (kThreads * 4) + l4, x[u][j]);
    }
  }
}

template <int GB, int MB>
hipError_t mix_v(int vb, void *w, const void *g, void *m, void *v,
                 uint64_t nt, int grid, hipStream_t s) {
  if (vb == 4)
    hipLaunchKernelGGL((k_probe_mix<GB, MB, 4>), dim3(grid), dim3(kThreads),
                       0, s, w, g, m, v, nt);
  else
    hipLaunchKernelGGL((k_probe_mix<GB, MB, 2>), dim3(grid), dim3(kThreads),
                       0, s, w, g, m, v, nt);
  return hipGetLastError();
}

}  // namespace

extern "C" {

// n elements (a multiple of 4096) of w (f32), g, m, v with the given element
// bytes (4 or 2).  Returns a hipError_t value (0 = launched).
int mta_probe_mix(void *w, const void *g, void *m, void *v, int64_t n,
                  int gbytes, int mbytes, int vbytes, int grid, void *stream) {
  if (n <= 0 || n % kTile || grid < 1) return hipErrorInvalidValue;
  const uint64_t nt = static_cast<uint64_t>(n) / kTile;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int key = (gbytes == 4 ? 4 : 0) | (mbytes == 4 ? 2 : 0);
  switch (key) {
    case 6: return mix_v<4, 4>(vbytes, w, g, m, v, nt, grid, s);
    case 4: return mix_v<4, 2>(vbytes, w, g, m, v, nt, grid, s);
    case 2: return mix_v<2, 4>(vbytes, w, g, m, v, nt, grid, s);
    default: return mix_v<2, 2>(vbytes, w, g, m, v, nt, grid, s);
  }
}

int mta_probe_read(const void *a, int64_t n, float *sink, int grid,
                   void *stream) {
  if (n <= 0 || n % kTile || grid < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_probe_read, dim3(grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), a,
                     static_cast<uint64_t>(n) / kTile, sink);
  return hipGetLastError();
}

int mta_probe_write(void *b, int64_t n, int grid, void *stream) {
  if (n <= 0 || n % kTile || grid < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_probe_write, dim3(grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), b,
                     static_cast<uint64_t>(n) / kTile);
  return hipGetLastError();
}

int mta_probe_copy(const void *a, void *b, int64_t n, int grid,
                   void *stream) {
  if (n <= 0 || n % kTile || grid < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_probe_copy, dim3(grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), a, b,
                     static_cast<uint64_t>(n) / kTile);
  return hipGetLastError();
}

}  // extern "C"
