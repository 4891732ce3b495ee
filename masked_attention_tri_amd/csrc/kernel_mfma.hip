// MFMA forward kernel for bf16 / fp16 inputs, D in {32, 64, 128}.
//
// Computes the triangle_attention page's equation: per (b, n, h) row,
// O_q = sum_k softmax_k(s Q_q.K_k + B_qk, masked keys excluded) V_k, with the
// lse / max auxiliaries, as a single pass over key tiles (an online,
// max-shifted softmax; the page fixes the result, not the schedule).
//
// Work decomposition: one workgroup of 4 wavefronts owns 128 query rows of
// one (b, n, h); wave w owns rows 32w .. 32w+31.  Key tiles of 64 keys are
// staged in LDS, double-buffered, straight from the row-major HBM layout.
//
// Both contractions run on v_mfma_f32_32x32x16_{bf16,f16}:
//   S^T = K . Q^T   A = K rows from LDS (16-byte reads), B = Q^T held in
//                   registers for the whole key loop.  The accumulator puts
//                   one query per lane and 16 keys per lane in registers, so
//                   the softmax row reductions are in-lane plus one exchange
//                   with the partner lane (lane ^ 32).
//   O^T = V^T . P^T B = P^T taken directly from the S^T registers (converted
//                   to bf16/fp16), A = V^T read from the row-major V tile with
//                   ds_read_b64_tr_b16, which hands each lane four keys of
//                   one column.  The query stays in the lane, so the running
//                   rescale of O is a per-lane scalar.
//
// Masks: kv_lengths and block lists cut whole tiles (tiles past the length,
// blocks not listed); element masks are applied only on tiles that need
// them (the ragged last tile, dense-mask tiles, causal partial blocks); full
// blocks skip the mask.  Masked logits are -inf internally; a row left with
// no valid key gets the page's uniform-weight result (mean of V over all K
// keys, max -1e9, lse -1e9 + ln K).
//
// Grid: one workgroup per (b, n, h, query tile), remapped so that each of the
// 8 XCDs walks a contiguous range of (b, h, n, q-tile) order: the q-tiles of
// one (n, h) share K/V in that XCD's L2 and a head's fp32 bias (shared by
// every n) stays resident there.
#include <math.h>

#include "triattn_internal.h"

namespace triattn {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQTile = 32 * kWaves;  // query rows per workgroup
constexpr int kKTile = 64;           // keys per K/V tile
constexpr int kXcds = 8;
constexpr float kLog2e = 1.4426950408889634f;

template <typename T>
struct Mma;
template <>
struct Mma<__bf16> {
    using v8 = bf16x8;
    static __device__ __forceinline__ f32x16 run(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Mma<_Float16> {
    using v8 = f16x8;
    static __device__ __forceinline__ f32x16 run(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

template <int D>
struct Tile {
    // LDS row pitches: K rows are read 16 bytes per lane down 8-row groups,
    // V rows 4x8 bytes by the transposing read; the pads keep both
    // bank-conflict free.
    static constexpr int kPitch = 2 * D + 16;
    static constexpr int vPitch = 2 * D + 32;
    static constexpr int kBytes = kKTile * kPitch;
    static constexpr int vBytes = kKTile * vPitch;
    static constexpr int stage = kBytes + vBytes;
    static constexpr int chunksPerRow = D / 8;                  // 16-byte chunks
    static constexpr int perThread = kKTile * chunksPerRow / kThreads;
    static_assert(perThread * kThreads == kKTile * chunksPerRow, "tile split");
};

__device__ __forceinline__ bool bit_set(const uint32_t* bits, int64_t i) {
    return (bits[i >> 5] >> (i & 31)) & 1u;
}

// First set bit at or after `from`, or -1.
__device__ int64_t next_set(const uint32_t* bits, int64_t from, int64_t n) {
    int64_t j = from;
    while (j < n) {
        const uint32_t w = bits[j >> 5] >> (j & 31);
        if (w) {
            const int64_t r = j + __builtin_ctz(w);
            return r < n ? r : -1;
        }
        j = (j | 31) + 1;
    }
    return -1;
}

__device__ void mark_list(uint32_t* bits, const int32_t* counts, const int32_t* ids,
                          int64_t list_row, int64_t width, int64_t n_blocks, int tid) {
    int64_t count = counts[list_row];
    count = count < 0 ? 0 : (count > width ? width : count);
    const int32_t* row = ids + list_row * width;
    for (int64_t j = tid; j < count; j += kThreads) {
        const int64_t id = row[j];
        if (id >= 0 && id < n_blocks) atomicOr(&bits[id >> 5], 1u << (id & 31));
    }
}

template <typename T, int D, int KIND, bool BIAS_VEC>
__global__ __launch_bounds__(kThreads) void mfma_fwd_kernel(Params p) {
    using M = Mma<T>;
    using v8 = typename M::v8;
    using L = Tile<D>;
    constexpr int kWords = static_cast<int>(kMaxKvBlocks / 32);
    constexpr bool kBlock = KIND == TRIATTN_MASK_BLOCK;

    __shared__ __attribute__((aligned(16))) char smem[2 * L::stage];
    __shared__ uint32_t listed_bits[kBlock ? kWords : 1];
    __shared__ uint32_t full_bits[kBlock ? kWords : 1];
    __shared__ float mean_v[D];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;  // this lane's query within the wave
    const int half = lane >> 5;

    // ---- workgroup -> (b, n, h, q tile), XCD-contiguous order -----------
    const int64_t n_qt = (p.Q + kQTile - 1) / kQTile;
    const int64_t W = gridDim.x;
    const int64_t w = blockIdx.x;
    const int64_t xcd = w % kXcds, slot = w / kXcds;
    const int64_t per = W / kXcds, rem = W % kXcds;
    const int64_t lid = xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
    const int64_t qt = lid % n_qt;
    const int64_t n = (lid / n_qt) % p.N;
    const int64_t h = (lid / (n_qt * p.N)) % p.H;
    const int64_t b = lid / (n_qt * p.N * p.H);

    const int64_t K = p.K, Q = p.Q;
    const int64_t bnh = (b * p.N + n) * p.H + h;
    const T* kbase = static_cast<const T*>(p.k) + bnh * K * D;
    const T* vbase = static_cast<const T*>(p.v) + bnh * K * D;
    const int64_t q0 = qt * kQTile;
    const int64_t q0w = q0 + 32 * wave;
    const int64_t qrow = q0w + col;  // this lane's query
    const bool row_ok = qrow < Q;
    const int64_t qload = row_ok ? qrow : Q - 1;
    const float* brow = p.bias ? p.bias + ((b * p.H + h) * Q + qload) * K : nullptr;

    // ---- visited key range / tile list -------------------------------
    int64_t limit = K;  // keys >= limit are never valid
    if (KIND == TRIATTN_MASK_KV_LENGTHS) {
        const int64_t len = p.kv_lengths[b * p.N + n];
        limit = len < 0 ? 0 : (len > K ? K : len);
    }
    const int64_t n_tiles_all = (limit + kKTile - 1) / kKTile;
    int64_t tiles_per_block = 1;
    if (kBlock) {
        tiles_per_block = p.kv_block / kKTile;
        const int words = static_cast<int>((p.n_kv_blocks + 31) / 32);
        for (int i = tid; i < words; i += kThreads) {
            listed_bits[i] = 0u;
            full_bits[i] = 0u;
        }
        __syncthreads();
        const int64_t inst = b * p.stride_b + n * p.stride_n + h * p.stride_h;
        const int64_t list_row = inst * p.n_q_rows + q0 / p.q_block;
        mark_list(listed_bits, p.kv_num_blocks, p.kv_indices, list_row, p.max_blocks,
                  p.n_kv_blocks, tid);
        if (p.full_kv_num_blocks) {
            mark_list(full_bits, p.full_kv_num_blocks, p.full_kv_indices, list_row,
                      p.full_max_blocks, p.n_kv_blocks, tid);
            mark_list(listed_bits, p.full_kv_num_blocks, p.full_kv_indices, list_row,
                      p.full_max_blocks, p.n_kv_blocks, tid);
        }
        __syncthreads();
    }
    auto first_tile = [&]() -> int64_t {
        if (!kBlock) return n_tiles_all > 0 ? 0 : -1;
        const int64_t blk = next_set(listed_bits, 0, p.n_kv_blocks);
        return blk < 0 ? -1 : blk * tiles_per_block;
    };
    auto next_tile = [&](int64_t t) -> int64_t {
        if (!kBlock) return t + 1 < n_tiles_all ? t + 1 : -1;
        if ((t + 1) % tiles_per_block != 0 && t + 1 < n_tiles_all) return t + 1;
        const int64_t blk = next_set(listed_bits, t / tiles_per_block + 1, p.n_kv_blocks);
        return blk < 0 ? -1 : blk * tiles_per_block;
    };

    // ---- Q^T operand: registers for the whole key loop ----------------
    v8 qop[D / 16];
    {
        const T* qp = static_cast<const T*>(p.q) + (bnh * Q + qload) * D + 8 * half;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            u32x4 raw = *reinterpret_cast<const u32x4*>(qp + 16 * st);
            if (!row_ok) raw = u32x4{0u, 0u, 0u, 0u};
            qop[st] = __builtin_bit_cast(v8, raw);
        }
    }

    // ---- K/V staging ---------------------------------------------------
    u32x4 kreg[L::perThread], vreg[L::perThread];
    auto load_tile = [&](int64_t t) {
#pragma unroll
        for (int i = 0; i < L::perThread; ++i) {
            const int c = tid + kThreads * i;
            const int r = c / L::chunksPerRow, cc = c % L::chunksPerRow;
            const int64_t key = t * kKTile + r;
            if (key < K) {
                kreg[i] = *reinterpret_cast<const u32x4*>(kbase + key * D + cc * 8);
                vreg[i] = *reinterpret_cast<const u32x4*>(vbase + key * D + cc * 8);
            } else {
                kreg[i] = u32x4{0u, 0u, 0u, 0u};
                vreg[i] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    lds_char* lds = (lds_char*)smem;
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < L::perThread; ++i) {
            const int c = tid + kThreads * i;
            const int r = c / L::chunksPerRow, cc = c % L::chunksPerRow;
            *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(
                lds + buf * L::stage + r * L::kPitch + cc * 16) = kreg[i];
            *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(
                lds + buf * L::stage + L::kBytes + r * L::vPitch + cc * 16) = vreg[i];
        }
    };

    // Per-lane LDS offsets of the operand reads.
    const int k_off = col * L::kPitch + 16 * half;  // K row `col`, d-slot 8*half
    // Transposing read: lane s names row 4*(s/32) + (s%16)/4 and column
    // 16*((s/16)%2) + 4*(s%4) of a 16-key x 32-column block; the result in
    // lane l is then V[key(slot)][32*db + (l % 32)] for its 4 key slots.
    const int v_off = (4 * half + (lane & 15) / 4) * L::vPitch + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY;  // running max of this lane's query row
    float l_run = 0.f;        // this lane's half of the running sum

    int64_t tile = first_tile();
    if (tile >= 0) {
        load_tile(tile);
        store_tile(0);
    }
    __syncthreads();
    int buf = 0;
    while (tile >= 0) {
        const int64_t nxt = next_tile(tile);
        if (nxt >= 0) load_tile(nxt);  // in flight while this tile computes

        const int64_t k0 = tile * kKTile;
        // ---- which element mask this tile needs (wave-uniform) ---------
        bool need_mask = k0 + kKTile > limit;
        bool causal = false;
        uint64_t dense_bits = ~0ull;
        if (KIND == TRIATTN_MASK_DENSE) {
            const int64_t key = k0 + lane;
            const bool ok = key < K && p.dense[(b * p.N + n) * K + key] != 0;
            dense_bits = __ballot(ok);
            need_mask = true;
        }
        if (kBlock && p.mask_mod == TRIATTN_MOD_CAUSAL &&
            !bit_set(full_bits, tile / tiles_per_block) && k0 + kKTile - 1 > q0w) {
            causal = true;
            need_mask = true;
        }
        const bool skip = KIND == TRIATTN_MASK_DENSE && dense_bits == 0ull;

        if (!skip) {
            // ---- bias for this lane's query and its 32 keys ------------
            float bias_v[2][16];
            if (brow) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int64_t key = k0 + 32 * kb + 8 * g + 4 * half;
                        if (BIAS_VEC) {
                            f32x4 bv = f32x4{0.f, 0.f, 0.f, 0.f};
                            if (key < K) bv = *reinterpret_cast<const f32x4*>(brow + key);
#pragma unroll
                            for (int e = 0; e < 4; ++e) bias_v[kb][4 * g + e] = bv[e];
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                bias_v[kb][4 * g + e] = key + e < K ? brow[key + e] : 0.f;
                        }
                    }
            }

            // ---- S^T = K . Q^T ------------------------------------------
            const lds_char* kl = lds + buf * L::stage;
            f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
            for (int st = 0; st < D / 16; ++st) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const v8 a = __builtin_bit_cast(
                        v8, *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
                                kl + k_off + kb * 32 * L::kPitch + 32 * st));
                    s[kb] = M::run(a, qop[st], s[kb]);
                }
            }

            // ---- logits, mask, running max -------------------------------
            float mloc = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float z = brow ? fmaf(s[kb][r], p.scale, bias_v[kb][r]) : s[kb][r] * p.scale;
                    if (need_mask) {
                        const int kl_idx = 32 * kb + 8 * (r / 4) + 4 * half + (r % 4);
                        const int64_t key = k0 + kl_idx;
                        bool ok = key < limit;
                        if (KIND == TRIATTN_MASK_DENSE) ok = ok && ((dense_bits >> kl_idx) & 1ull);
                        if (causal) ok = ok && qrow >= key;
                        z = ok ? z : -INFINITY;
                    }
                    s[kb][r] = z;
                    mloc = fmaxf(mloc, z);
                }
            mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
            const float m_new = fmaxf(m_run, mloc);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float mb = m_use * kLog2e;
            const float alpha = __builtin_amdgcn_exp2f(m_run * kLog2e - mb);
            m_run = m_new;

            // ---- probabilities, running sum, P^T operands ----------------
            v8 pop[2][2];
            float lsum = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float pz = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * t + j], kLog2e, -mb));
                        lsum += pz;
                        pop[kb][t][j] = static_cast<T>(pz);
                    }
            l_run = l_run * alpha + lsum;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;

            // ---- O^T += V^T . P^T ----------------------------------------
            const lds_char* vl = lds + buf * L::stage + L::kBytes;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const lds_char* base = vl + v_off + (32 * kb + 16 * t) * L::vPitch + 64 * db;
                        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) i16x4*)(base));
                        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) i16x4*)(base + 8 * L::vPitch));
                        const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
                        const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
                        const v8 a = __builtin_bit_cast(v8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
                        oacc[db] = M::run(a, pop[kb][t], oacc[db]);
                    }
        }

        if (nxt >= 0) store_tile(buf ^ 1);
        __syncthreads();
        buf ^= 1;
        tile = nxt;
    }

    // ---- epilogue ---------------------------------------------------------
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const bool dead = m_run == -INFINITY;
    if (__syncthreads_or(dead && row_ok)) {
        // Some row saw no valid key: its weights are uniform over all K keys.
        for (int d = tid; d < D; d += kThreads) {
            float acc = 0.f;
            for (int64_t kk = 0; kk < K; ++kk) acc += static_cast<float>(vbase[kk * D + d]);
            mean_v[d] = acc / static_cast<float>(K);
        }
        __syncthreads();
    }
    if (!row_ok) return;
    T* orow = static_cast<T*>(p.out) + (bnh * Q + qrow) * D;
    const float inv = dead ? 0.f : 1.0f / l_tot;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d0 = 32 * db + 8 * g + 4 * half;
            T o4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o4[e] = static_cast<T>(dead ? mean_v[d0 + e] : oacc[db][4 * g + e] * inv);
            *reinterpret_cast<u32x2*>(orow + d0) = __builtin_bit_cast(u32x2, o4);
        }
    if (half == 0) {
        const int64_t ridx = bnh * Q + qrow;
        if (p.lse) p.lse[ridx] = dead ? kMaskedLogit + logf(static_cast<float>(K)) : m_run + logf(l_tot);
        if (p.mx) p.mx[ridx] = dead ? kMaskedLogit : m_run;
    }
}

template <typename T, int D, int KIND>
hipError_t launch_kind(const Params& p, bool bias_vec, dim3 grid, hipStream_t stream) {
    if (bias_vec)
        hipLaunchKernelGGL((mfma_fwd_kernel<T, D, KIND, true>), grid, dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((mfma_fwd_kernel<T, D, KIND, false>), grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const Params& p, bool bias_vec, dim3 grid, hipStream_t stream) {
    switch (p.mask_kind) {
    case TRIATTN_MASK_NONE:
        return launch_kind<T, D, TRIATTN_MASK_NONE>(p, bias_vec, grid, stream);
    case TRIATTN_MASK_DENSE:
        return launch_kind<T, D, TRIATTN_MASK_DENSE>(p, bias_vec, grid, stream);
    case TRIATTN_MASK_KV_LENGTHS:
        return launch_kind<T, D, TRIATTN_MASK_KV_LENGTHS>(p, bias_vec, grid, stream);
    case TRIATTN_MASK_BLOCK:
        return launch_kind<T, D, TRIATTN_MASK_BLOCK>(p, bias_vec, grid, stream);
    }
    return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_t(const Params& p, bool bias_vec, dim3 grid, hipStream_t stream) {
    switch (p.D) {
    case 32:
        return launch_d<T, 32>(p, bias_vec, grid, stream);
    case 64:
        return launch_d<T, 64>(p, bias_vec, grid, stream);
    case 128:
        return launch_d<T, 128>(p, bias_vec, grid, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool mfma_supports(const Params& p, int32_t dtype) {
    if (dtype != TRIATTN_BF16 && dtype != TRIATTN_F16) return false;
    if (p.D != 32 && p.D != 64 && p.D != 128) return false;
    if (p.mask_kind == TRIATTN_MASK_BLOCK) {
        // one block row per workgroup, whole tiles per kv block
        if (p.q_block % kQTile != 0 || p.kv_block % kKTile != 0) return false;
    }
    return true;
}

hipError_t launch_mfma(const Params& p, int32_t dtype, hipStream_t stream) {
    const int64_t n_qt = (p.Q + kQTile - 1) / kQTile;
    const int64_t groups = p.B * p.N * p.H * n_qt;
    if (groups > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid(static_cast<unsigned>(groups));
    const bool bias_vec = p.bias && (p.K % 4 == 0) && (reinterpret_cast<uintptr_t>(p.bias) % 16 == 0);
    if (dtype == TRIATTN_BF16) return launch_t<__bf16>(p, bias_vec, grid, stream);
    return launch_t<_Float16>(p, bias_vec, grid, stream);
}

}  // namespace triattn
