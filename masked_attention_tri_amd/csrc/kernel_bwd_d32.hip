// The MFMA backward kernels (mfma_bwd.h) at D = 32.
#include "mfma_bwd.h"

namespace triattn {

hipError_t launch_bwd_mfma_d32(const Params& p, const BwdParams& g, int32_t dtype, float* ws,
                               size_t ws_bytes, hipStream_t stream) {
    const bool exact = tile::scale_is_exact(p.scale);
    if (dtype == TRIATTN_BF16) return launch_bwd_d<__bf16, 32>(p, g, exact, ws, ws_bytes, stream);
    return launch_bwd_d<_Float16, 32>(p, g, exact, ws, ws_bytes, stream);
}

}  // namespace triattn
