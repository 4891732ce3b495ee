// Instantiations of the MFMA forward kernel (mfma_fwd.h) at D = 32.
#include "mfma_fwd.h"

namespace triattn {

hipError_t launch_mfma_d32(const Params& p, int32_t dtype, bool exact, hipStream_t stream) {
    if (dtype == TRIATTN_BF16) return launch_d<__bf16, 32>(p, exact, stream);
    return launch_d<_Float16, 32>(p, exact, stream);
}

}  // namespace triattn
