// Host-only stand-ins for the kernel launchers, linked with the C-ABI layer
// (zha_api.cpp) into the sanitizer build that runs the CPU ABI tests: every
// check those tests reach runs on the host before any launch, so no stub
// is ever called by them; if one is, it reports a HIP error.
#include "../../tree_indexed_sparse_zha_amd/csrc/zha_internal.h"

namespace zha {

hipError_t launch_build(const BuildArgs&, int, Prof&) { return hipErrorNotSupported; }
hipError_t launch_route_init(uint32_t*, int64_t, Prof&) { return hipErrorNotSupported; }
hipError_t launch_route_level(const ScoreArgs&, const SelectArgs&, int, int, int, Prof&) {
  return hipErrorNotSupported;
}
hipError_t launch_attend(const AttendArgs&, int, int, Prof&) { return hipErrorNotSupported; }
hipError_t launch_probe(int, const void*, void*, int64_t, Prof&) { return hipErrorNotSupported; }
hipError_t launch_selected_chunks(const uint32_t*, int64_t, int64_t, int64_t, int32_t*, int32_t*, int64_t,
                                  hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace zha
