// Instantiations of the MFMA forward kernel (mfma_fwd.h) at D = 256.
#include "mfma_fwd.h"

namespace triattn {

hipError_t launch_mfma_d256(const Params& p, int32_t dtype, bool exact, hipStream_t stream) {
    if (dtype == TRIATTN_BF16) return launch_d<__bf16, 256>(p, exact, stream);
    return launch_d<_Float16, 256>(p, exact, stream);
}

}  // namespace triattn
