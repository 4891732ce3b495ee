// Generic forward kernel: one wavefront per query row, fp32 arithmetic.
//
// Serves every (dtype, D) in the envelope of the triangle_attention page
// (Notes item 3: D <= 32 for fp32, D <= 256 for the half types, the wider
// bound being the one that page gives its newest forward kernels) and every
// mask form; it is the path for what the MFMA kernels do not take (block
// masks with query blocks other than 32, 64 or a multiple of 128 rows, or
// key blocks that are neither 16 keys nor whole 32-key tiles;
// unaligned fp32 tensors; and
// the other half-type cases outside the MFMA kernel's envelope).  Lanes split the keys
// for the logits and the d coordinates for P.V; the softmax runs online over
// chunks of 64 keys with a running max and sum (the max-shifted evaluation of
// the page's softmax), so a row of any length needs O(D) state.
#include <math.h>

#include "triattn_internal.h"

namespace triattn {
namespace {

constexpr int kWaves = 4;
constexpr int kWords = static_cast<int>(kMaxKvBlocks / 32);

template <typename T>
__device__ __forceinline__ float to_f32(T x) {
    return static_cast<float>(x);
}

__device__ __forceinline__ float wave_max(float x) {
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

__device__ __forceinline__ bool test_bit(const uint32_t* bits, int64_t i) {
    return (bits[i >> 5] >> (i & 31)) & 1u;
}

// Sets the bit of every in-range block id among the first `count` entries
// of one BlockMask list row (the tensorplay.nn.attention page, Basics: the
// to-dense loop marks each listed block; later entries are undefined).
__device__ void mark_list(uint32_t* bits, const int32_t* counts, const int32_t* ids,
                          int64_t list_row, int64_t width, int64_t n_blocks, int lane) {
    int64_t count = counts[list_row];
    count = count < 0 ? 0 : (count > width ? width : count);
    const int32_t* row = ids + list_row * width;
    for (int64_t j = lane; j < count; j += 64) {
        const int64_t id = row[j];
        if (id >= 0 && id < n_blocks) atomicOr(&bits[id >> 5], 1u << (id & 31));
    }
}

// kOut output coordinates per lane: 2 covers D <= 128, 4 covers D <= 256.
template <typename T, int kOut>
__global__ __launch_bounds__(256) void generic_fwd_kernel(Params p) {
    __shared__ uint32_t listed_bits[kWaves][kWords];
    __shared__ uint32_t full_bits[kWaves][kWords];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t total = p.B * p.N * p.H * p.Q;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
    bool active = row < total;
    const int64_t r = active ? row : 0;
    const int64_t qi = r % p.Q;
    const int64_t h = (r / p.Q) % p.H;
    const int64_t n = (r / (p.Q * p.H)) % p.N;
    const int64_t b = r / (p.Q * p.H * p.N);
    const int64_t D = p.D;
    int64_t K = p.K;
    const int64_t bnh = (b * p.N + n) * p.H + h;
    // Rows of q / out and of k / v, and the lse / max index: the (b, n, h)
    // slices, or for packed sequences (row, head) slabs of the packed tensors.
    const bool varlen = p.mask_kind == kMaskVarlen;
    const T* qrow;
    const T* kbase;
    const T* vbase;
    int64_t kv_rs = D;
    int64_t out_row = r;
    if (varlen) {
        const SeqRows sr = seq_rows(p, b);
        active = active && qi < sr.nq;
        K = sr.nk;
        kv_rs = p.kv_rs;
        qrow = static_cast<const T*>(p.q) + (sr.q0 + qi) * p.q_rs + h * D;
        kbase = static_cast<const T*>(p.k) + sr.k0 * kv_rs + h * D;
        vbase = static_cast<const T*>(p.v) + sr.k0 * kv_rs + h * D;
        out_row = (sr.q0 + qi) * p.H + h;
    } else {
        qrow = static_cast<const T*>(p.q) + r * D;
        kbase = static_cast<const T*>(p.k) + bnh * K * D;
        vbase = static_cast<const T*>(p.v) + bnh * K * D;
    }
    const float* brow = p.bias ? p.bias + ((b * p.H + h) * p.Q + qi) * K : nullptr;
    const T* brow16 =  // a bias in the input type
        p.bias16 ? static_cast<const T*>(p.bias16) + ((b * p.H + h) * p.Q + qi) * K : nullptr;

    // Visited and full kv blocks of this row's BlockMask row.
    const bool block_kind = p.mask_kind == TRIATTN_MASK_BLOCK;
    if (block_kind) {  // uniform over the workgroup
        const int words = static_cast<int>((p.n_kv_blocks + 31) / 32);
        for (int w = lane; w < words; w += 64) {
            listed_bits[wave][w] = 0u;
            full_bits[wave][w] = 0u;
        }
        __syncthreads();
        if (active) {
            const int64_t inst = b * p.stride_b + n * p.stride_n + h * p.stride_h;
            const int64_t list_row = inst * p.n_q_rows + qi / p.q_block;
            mark_list(listed_bits[wave], p.kv_num_blocks, p.kv_indices, list_row, p.max_blocks,
                      p.n_kv_blocks, lane);
            if (p.full_kv_num_blocks) {
                mark_list(full_bits[wave], p.full_kv_num_blocks, p.full_kv_indices, list_row,
                          p.full_max_blocks, p.n_kv_blocks, lane);
                mark_list(listed_bits[wave], p.full_kv_num_blocks, p.full_kv_indices, list_row,
                          p.full_max_blocks, p.n_kv_blocks, lane);
            }
        }
        __syncthreads();
    }
    if (!active) return;

    // Keys at or past `limit` are never valid.
    int64_t limit = K;
    if (p.mask_kind == TRIATTN_MASK_KV_LENGTHS) {
        const int64_t len = p.kv_lengths[b * p.N + n];
        limit = len < 0 ? 0 : (len > K ? K : len);
    }
    if (varlen && p.causal) limit = limit < qi + 1 ? limit : qi + 1;  // keys j <= qi
    const uint8_t* mrow = p.mask_kind == TRIATTN_MASK_DENSE ? p.dense + (b * p.N + n) * K : nullptr;

    float m = -INFINITY;  // running max of the valid logits
    float l = 0.f;        // running sum of exp(z - m)
    // O[lane + 64 i], i < kOut: up to 256 coordinates
    float o[kOut];
    bool has[kOut];
#pragma unroll
    for (int i = 0; i < kOut; ++i) {
        o[i] = 0.f;
        has[i] = lane + 64 * i < D;
    }

    for (int64_t c0 = 0; c0 < limit; c0 += 64) {
        const int64_t kk = c0 + lane;
        bool valid = kk < limit;
        if (valid && mrow) valid = mrow[kk] != 0;
        if (valid && block_kind) {
            const int64_t blk = kk / p.kv_block;
            if (!test_bit(listed_bits[wave], blk)) {
                valid = false;
            } else if (!test_bit(full_bits[wave], blk) && p.mask_mod == TRIATTN_MOD_CAUSAL) {
                valid = qi >= kk;
            }
        }
        float z = -INFINITY;
        if (valid) {
            const T* krow = kbase + kk * kv_rs;
            float dot = 0.f;
            for (int64_t d = 0; d < D; ++d) dot = fmaf(to_f32(qrow[d]), to_f32(krow[d]), dot);
            z = fmaf(dot, p.scale, brow ? brow[kk] : (brow16 ? to_f32(brow16[kk]) : 0.f));
        }
        const float m_new = fmaxf(m, wave_max(z));
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = expf(m - m_use);
        const float pz = valid ? expf(z - m_use) : 0.f;
        l = l * alpha + wave_sum(pz);
#pragma unroll
        for (int i = 0; i < kOut; ++i) o[i] *= alpha;
        const int64_t jmax = (limit - c0) < 64 ? (limit - c0) : 64;
        for (int j = 0; j < jmax; ++j) {
            const float pj = __shfl(pz, j);
            if (pj == 0.f) continue;  // uniform: pj is the same in every lane
            const T* vrow = vbase + (c0 + j) * kv_rs;
#pragma unroll
            for (int i = 0; i < kOut; ++i)
                if (has[i]) o[i] = fmaf(pj, to_f32(vrow[lane + 64 * i]), o[i]);
        }
        m = m_new;
    }

    float lse, mx;
    if (m == -INFINITY) {
        // No valid key: every logit is the -1e9 replacement, so the softmax
        // is uniform over all K keys.
#pragma unroll
        for (int i = 0; i < kOut; ++i) o[i] = 0.f;
        for (int64_t kk = 0; kk < K; ++kk) {
            const T* vrow = vbase + kk * kv_rs;
#pragma unroll
            for (int i = 0; i < kOut; ++i)
                if (has[i]) o[i] += to_f32(vrow[lane + 64 * i]);
        }
        // (a packed sequence with no key at all averages nothing: 0)
        const float inv = K > 0 ? 1.0f / static_cast<float>(K) : 0.f;
#pragma unroll
        for (int i = 0; i < kOut; ++i) o[i] *= inv;
        mx = kMaskedLogit;
        lse = kMaskedLogit + (K > 0 ? logf(static_cast<float>(K)) : 0.f);
    } else {
        const float inv = 1.0f / l;
#pragma unroll
        for (int i = 0; i < kOut; ++i) o[i] *= inv;
        mx = m;
        lse = m + logf(l);
    }
    T* orow = static_cast<T*>(p.out) + out_row * D;
#pragma unroll
    for (int i = 0; i < kOut; ++i)
        if (has[i]) orow[lane + 64 * i] = static_cast<T>(o[i]);
    if (lane == 0) {
        if (p.lse) p.lse[out_row] = lse;
        if (p.mx) p.mx[out_row] = mx;
    }
}

}  // namespace

hipError_t launch_generic(const Params& p, int32_t dtype, hipStream_t stream) {
    if (dtype == TRIATTN_F32 && fp32_mfma_supports(p)) return launch_fp32_mfma(p, stream);
    const int64_t rows = p.B * p.N * p.H * p.Q;
    const int64_t blocks = (rows + kWaves - 1) / kWaves;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid(static_cast<unsigned>(blocks)), block(64 * kWaves);
    const bool wide = p.D > 128;
    switch (dtype) {
    case TRIATTN_F32:
        hipLaunchKernelGGL((generic_fwd_kernel<float, 2>), grid, block, 0, stream, p);
        break;
    case TRIATTN_F16:
        if (wide)
            hipLaunchKernelGGL((generic_fwd_kernel<_Float16, 4>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((generic_fwd_kernel<_Float16, 2>), grid, block, 0, stream, p);
        break;
    case TRIATTN_BF16:
        if (wide)
            hipLaunchKernelGGL((generic_fwd_kernel<__bf16, 4>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((generic_fwd_kernel<__bf16, 2>), grid, block, 0, stream, p);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace triattn
