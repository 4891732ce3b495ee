// Internal declarations shared by the host entry points and the kernels of
// libtriattn.  Not part of the public ABI (that is include/triattn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "triattn.h"

namespace triattn {

// Every argument of one forward call, flattened into a POD that is passed to
// the kernels by value.
struct Params {
    const void* q;
    const void* k;
    const void* v;
    const float* bias;  // (B,1,H,Q,K) or nullptr
    void* out;
    float* lse;  // may be nullptr
    float* mx;   // may be nullptr
    int64_t B, N, H, Q, K, D;
    float scale;  // already resolved (never NaN)
    int32_t mask_kind;
    int32_t mask_mod;
    const uint8_t* dense;
    const int32_t* kv_lengths;
    const int32_t* kv_num_blocks;
    const int32_t* kv_indices;
    const int32_t* full_kv_num_blocks;
    const int32_t* full_kv_indices;
    int64_t q_block, kv_block, max_blocks, full_max_blocks;
    int64_t stride_b, stride_n, stride_h;
    int64_t n_q_rows;     // ceil(Q / q_block) (block kind)
    int64_t n_kv_blocks;  // ceil(K / kv_block) (block kind)
};

// The extra arguments of one backward call: the forward's output and the
// incoming gradient (inputs), lse and max read through Params, and the
// gradients (outputs; dbias may be nullptr).
struct BwdParams {
    const void* out;
    const void* dout;
    const float* lse;
    const float* mx;
    void* dq;
    void* dk;
    void* dv;
    float* dbias;
    float* dz;  // (B,N,H,Q,K) fp32 dz from dq_kernel for the dBias sum, or null
};

// Masked logits are carried as -inf inside the kernels: when a row has at
// least one valid key this gives exactly the weights of the -1e9
// replacement (exp underflows to 0 either way); rows with no valid key are
// detected from their running max and take the uniform-weight result.
constexpr float kMaskedLogit = -1.0e9f;

// Largest number of kv blocks a block-sparse mask may have: the kernels keep
// one visited bit and one full bit per block in LDS.
constexpr int64_t kMaxKvBlocks = 8192;

// Launchers (enqueue only; return the launch error, if any).
hipError_t launch_generic(const Params& p, int32_t dtype, hipStream_t stream);
hipError_t launch_mfma(const Params& p, int32_t dtype, hipStream_t stream);
bool mfma_supports(const Params& p, int32_t dtype);
hipError_t launch_bwd(const Params& p, const BwdParams& g, int32_t dtype, hipStream_t stream);
hipError_t launch_mask_to_kv_lengths(const uint8_t* mask, int64_t rows, int64_t K,
                                     int32_t* kv_lengths, int32_t* nonprefix_rows,
                                     hipStream_t stream);

}  // namespace triattn
