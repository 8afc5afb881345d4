// Launchers that abort when reached: the host-side sanitizer run links the C ABI against these,
// so any call that gets past the host checks (and would enqueue device work) stops the run.
#include <stdio.h>
#include <stdlib.h>

#include "kernels.h"

namespace moelora {

[[noreturn]] static void reached(const char* what) {
  fprintf(stderr, "device launcher reached: %s\n", what);
  abort();
}

hipError_t launch_route(const float*, int, int, int, int*, float*, int*, hipStream_t) {
  reached("route");
}
hipError_t launch_align(const AlignArgs&, size_t, hipStream_t) { reached("align"); }
hipError_t launch_router_logits(const uint16_t*, const uint16_t*, int, int, int, float*,
                                hipStream_t) {
  reached("router_logits");
}
hipError_t launch_shrink(bool, const ShrinkArgs&, int, hipStream_t) { reached("shrink"); }
hipError_t launch_shrink_tiled(bool, const ShrinkArgs&, int, hipStream_t) {
  reached("shrink_tiled");
}
hipError_t launch_zfinal(const float*, int, int64_t, int, const int*, int, int64_t, uint16_t*,
                         hipStream_t) {
  reached("zfinal");
}
hipError_t launch_skinny(const SkinnyConfig&, bool, const GemmArgs&, int, hipStream_t, bool) {
  reached("skinny");
}
hipError_t launch_tiled(const TiledConfig&, bool, const GemmArgs&, hipStream_t, bool) {
  reached("tiled");
}
hipError_t launch_sgmv_expand(const SgmvArgs&, int, hipStream_t) { reached("sgmv_expand"); }
hipError_t launch_combine(const CombineArgs&, hipStream_t) { reached("combine"); }
hipError_t launch_sgmv_sort(const SgmvSortArgs&, hipStream_t) { reached("sgmv_sort"); }
hipError_t launch_shrink_seg(bool, const ShrinkArgs&, int, hipStream_t) { reached("shrink_seg"); }

}  // namespace moelora
