// Host-only stand-ins for the kernel-side functions of launch.h, so the
// C-ABI layer (gqa_decode_api.cpp) can be built with host sanitizers and
// no device code. Nothing here is reached on a machine without a GPU: the
// argument checks and the device query come first.
#include <stdlib.h>

#include "launch.h"

namespace gqa {

int resident_workgroups_per_cu() { return 2; }

long long grid_for(int, int, int, const SplitConfig& cfg) { return cfg.pieces; }

size_t partial_bytes_for_grid(long long grid, int group) {
  return (size_t)(2 * grid) * group * 130 * sizeof(float);
}

size_t segment_bytes_for_batch(int batch, int kv_heads) {
  return ((size_t)batch * kv_heads * 8 + 255) & ~(size_t)255;
}

hipError_t scratch_area(int, void** ptr) {
  *ptr = nullptr;
  return hipErrorNoDevice;   // never reached without a device
}

hipError_t launch_decode(const void*, const void*, const int32_t*, void*, ElemType, const Layout&,
                         float, float, int, int, const SplitConfig&, long long, void*, int*,
                         hipStream_t, hipEvent_t*) {
  abort();   // never reached without a device
}

}  // namespace gqa
