// Backward pass kernels (gfx950). Placeholder until the kernels land.
#include "gqa_launch.h"

namespace gqa {

hipError_t launch_bwd(const BwdArgs &a, int H, hipStream_t stream) {
    (void)a;
    (void)H;
    (void)stream;
    return hipErrorNotSupported;
}

}  // namespace gqa
