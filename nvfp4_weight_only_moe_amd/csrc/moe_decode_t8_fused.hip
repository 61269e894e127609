// Instantiations of the decode kernel (decode_fused_kernel.h) for 2-8 tokens,
// mode kFused.
#include "decode_fused_kernel.h"

namespace moe {
namespace fused {
moe_status launch_t8_fused(const FusedParams& p, int grid, hipStream_t s) {
    return launch_shape<8, kFused>(p, grid, s);
}
}  // namespace fused
}  // namespace moe
