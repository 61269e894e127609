// Instantiations of the decode kernel (decode_fused_kernel.h) for one token,
// mode kDown.
#include "decode_fused_kernel.h"

namespace moe {
namespace fused {
moe_status launch_t1_down(const FusedParams& p, int grid, hipStream_t s) {
    return launch_shape<1, kDown>(p, grid, s);
}
}  // namespace fused
}  // namespace moe
