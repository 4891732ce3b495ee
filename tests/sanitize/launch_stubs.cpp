// Launchers of libtriattn replaced for the host-validation driver: every
// call it makes is rejected or has no work, so reaching a launch is an error.
#include <stdio.h>
#include <stdlib.h>

#include "../../masked_attention_tri_amd/csrc/triattn_internal.h"

[[noreturn]] static void reached(const char* what) {
    fprintf(stderr, "abi driver: %s reached a launch\n", what);
    abort();
}

namespace triattn {
hipError_t launch_generic(const Params&, int32_t, hipStream_t) { reached("launch_generic"); }
hipError_t launch_mfma_d32(const Params&, int32_t, bool, hipStream_t) { reached("launch_mfma_d32"); }
hipError_t launch_mfma_d64(const Params&, int32_t, bool, hipStream_t) { reached("launch_mfma_d64"); }
hipError_t launch_mfma_d128(const Params&, int32_t, bool, hipStream_t) { reached("launch_mfma_d128"); }
hipError_t launch_mfma_d256(const Params&, int32_t, bool, hipStream_t) { reached("launch_mfma_d256"); }
hipError_t launch_bwd(const Params&, const BwdParams&, int32_t, float*, size_t, hipStream_t) {
    reached("launch_bwd");
}
hipError_t launch_mask_to_kv_lengths(const uint8_t*, int64_t, int64_t, int32_t*, int32_t*, hipStream_t) {
    reached("launch_mask_to_kv_lengths");
}
}  // namespace triattn
