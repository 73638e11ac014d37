// san_stubs.cpp -- the kernel launchers of libmta, replaced for the host-only
// sanitizer build of mta_host.cpp (tests/test_sanitizers.py).  The driver
// (san_host.c) exercises only paths that refuse before any device work or
// make no HIP call; reaching a launcher is a failure of the test.
#include <cstdio>
#include <cstdlib>

#include "../../mixed_precision_optimizer_mta_amd/csrc/mta_internal.h"

namespace mta {

[[noreturn]] static void reached(const char *what) {
  std::fprintf(stderr, "san_stubs: %s reached in a host-only test\n", what);
  std::exit(3);
}

hipError_t launch_update(int, int, int, int, const Work &, const StepScalars &,
                         const float *, const AmpStep &) {
  reached("launch_update");
}
hipError_t launch_sumsq(int, const Work &, float, float, NormScratch, float *,
                        float *, mta_amp_state *) {
  reached("launch_sumsq");
}
hipError_t launch_scale(int, const Work &, float, const float *) {
  reached("launch_scale");
}
hipError_t launch_amp_update(mta_amp_state *, double, double, int32_t,
                             hipStream_t) {
  reached("launch_amp_update");
}
hipError_t noalloc_scratch(int, void **) { reached("noalloc_scratch"); }

}  // namespace mta
