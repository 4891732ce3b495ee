// mask_to_kv_lengths: the helper named in the triangle_attention page's
// example, which turns a right-padded (B,N,1,1,K) bool key mask into
// (B,N,1,1,1) int32 lengths for the kv_lengths argument.  One wavefront per
// mask row: the length is the index of the first masked key (K if none),
// and a row with a valid key after its first masked key is counted as not
// right-padded.
#include "triattn_internal.h"

namespace triattn {
namespace {

constexpr int kWaves = 4;

__global__ void reset_counter_kernel(int32_t* counter) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *counter = 0;
}

__global__ __launch_bounds__(256) void mask_to_kv_lengths_kernel(const uint8_t* mask,
                                                                 int64_t rows, int32_t K,
                                                                 int32_t* lengths,
                                                                 int32_t* nonprefix) {
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
    if (row >= rows) return;
    const uint8_t* m = mask + row * static_cast<int64_t>(K);
    int32_t first_masked = K;
    int32_t last_valid = -1;
    for (int32_t j = lane; j < K; j += 64) {
        if (m[j]) {
            last_valid = j;  // j increases, so this is the lane's last one
        } else if (j < first_masked) {
            first_masked = j;
        }
    }
    for (int off = 32; off > 0; off >>= 1) {
        first_masked = min(first_masked, __shfl_xor(first_masked, off));
        last_valid = max(last_valid, __shfl_xor(last_valid, off));
    }
    if (lane == 0) {
        lengths[row] = first_masked;
        if (last_valid > first_masked) atomicAdd(nonprefix, 1);
    }
}

}  // namespace

hipError_t launch_mask_to_kv_lengths(const uint8_t* mask, int64_t rows, int64_t K,
                                     int32_t* kv_lengths, int32_t* nonprefix_rows,
                                     hipStream_t stream) {
    hipLaunchKernelGGL(reset_counter_kernel, dim3(1), dim3(64), 0, stream, nonprefix_rows);
    if (rows > 0) {
        const int64_t blocks = (rows + kWaves - 1) / kWaves;
        if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(mask_to_kv_lengths_kernel, dim3(static_cast<unsigned>(blocks)),
                           dim3(64 * kWaves), 0, stream, mask, rows, static_cast<int32_t>(K),
                           kv_lengths, nonprefix_rows);
    }
    return hipGetLastError();
}

}  // namespace triattn
