// Host-only stand-ins for the kernel launch interface (kernels.h), for the
// sanitizer build of the host library (tree, planner, C ABI) that runs the
// CPU test suite under AddressSanitizer and UndefinedBehaviorSanitizer.
// Every launch reports that no device is present; the product library links
// the real launches from attn.hip instead.
#include "kernels.h"

namespace pkvt {

hipError_t launch_attn(const AttnArgs&, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_units(const AttnArgs&, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_prefill(const AttnArgs&, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_scatter_inline(const ScatterArgs&, const InlineSlots&, int, int, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_copy_words(const int32_t*, int32_t*, int64_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_merge(const MergeArgs&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_scatter(const ScatterArgs&, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_move(const MoveArgs&, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t noalloc_scratch(void**) { return hipErrorNoDevice; }

}  // namespace pkvt
