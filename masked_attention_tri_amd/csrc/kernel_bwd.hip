// Backward kernels: dQ, dK, dV and dBias of the triangle attention forward.
//
// The forward (cuequivariance_torch.triangle_attention page, the defining
// equation) per (b, n, h, q) row is O_q = sum_k P_k V_k with P = softmax(z),
// z_k = s Q_q.K_k + B_qk for a valid key and the constant -1e9 otherwise.
// Differentiating O (the auxiliary lse and max carry no incoming gradient):
//
//   dV_k += P_k dO_q                      every key
//   dz_k  = P_k (dO_q.V_k - Delta_q)      Delta_q = sum_k P_k dO_q.V_k = dO_q.O_q
//   dQ_q += s dz_k K_k,  dK_k += s dz_k Q_q,  dB_qk += dz_k      valid keys only
//
// P is rebuilt from the forward's lse (P_k = exp(z_k - lse_q)); a row whose
// forward max is the -1e9 replacement had no valid key, so its P is 1/K for
// every key and it passes nothing to Q, K or the bias.  The bias is shared by
// every n, so dB sums over n.
//
// These are the general kernels: fp32 inputs, and the head dimensions and
// block sizes without an MFMA backward (mfma_bwd.h).  Three
// launches, no atomics, every sum in a fixed order:
//   dQ    dq_kernel: 32 query rows per workgroup, fp32 tiles staged in LDS
//         (see Tiles below), looping over key tiles.  dQ = s dz K.
//   dK dV dkdv_kernel: 32 keys per workgroup, looping over query tiles.
//         dV = P^T dO, dK = s dz^T Q.
//   dB    dbias_kernel: dz recomputed per (b, h, 32 query rows, 128 keys)
//         walking n in order.
// The contractions run on MFMA for bf16/fp16 (P and dz rounded to the input
// type as operands) and as fp32 FMAs from LDS for fp32.
#include <math.h>

#include <type_traits>

#include "triattn_internal.h"

namespace triattn {
namespace {

// Each thread accumulates columns d = part + 8 i of one row, i < NC (a
// template parameter: D <= 8 NC, NC in {4, 8, 16, 32}).

template <typename T>
__device__ __forceinline__ float f32(T x) {
    return static_cast<float>(x);
}

// Is block `blk` among the first count entries of list row `row`?
__device__ bool listed_in(const int32_t* counts, const int32_t* ids, int64_t row, int64_t width,
                          int64_t blk) {
    int64_t count = counts[row];
    count = count < 0 ? 0 : (count > width ? width : count);
    for (int64_t j = 0; j < count; ++j)
        if (ids[row * width + j] == blk) return true;
    return false;
}

// The key-validity predicate of every mask kind (lengths clamped to [0, K];
// block lists: visited = kv list united with the full list, mask_mod on
// blocks that are not full, out-of-range ids never match).
__device__ bool key_valid(const Params& p, int64_t b, int64_t n, int64_t h, int64_t qi,
                          int64_t kk) {
    switch (p.mask_kind) {
    case TRIATTN_MASK_DENSE:
        return p.dense[(b * p.N + n) * p.K + kk] != 0;
    case TRIATTN_MASK_KV_LENGTHS: {
        if (!p.kv_lengths) return true;
        const int64_t len = p.kv_lengths[b * p.N + n];
        return kk < (len < 0 ? 0 : (len > p.K ? p.K : len));
    }
    case TRIATTN_MASK_BLOCK: {
        const int64_t inst = b * p.stride_b + n * p.stride_n + h * p.stride_h;
        const int64_t row = inst * p.n_q_rows + qi / p.q_block;
        const int64_t blk = kk / p.kv_block;
        if (p.full_kv_num_blocks &&
            listed_in(p.full_kv_num_blocks, p.full_kv_indices, row, p.full_max_blocks, blk))
            return true;
        if (!listed_in(p.kv_num_blocks, p.kv_indices, row, p.max_blocks, blk)) return false;
        return p.mask_mod == TRIATTN_MOD_CAUSAL ? qi >= kk : true;
    }
    default:
        return true;
    }
}

// Keys at or past this limit are never valid in slice (b, n): the clamped
// length with kv_lengths, else K.  With kv_lengths and a limit of 0 every row
// of the slice has no valid key.
__device__ __forceinline__ int64_t key_limit(const Params& p, int64_t b, int64_t n) {
    if (p.mask_kind != TRIATTN_MASK_KV_LENGTHS || !p.kv_lengths) return p.K;
    const int64_t len = p.kv_lengths[b * p.N + n];
    return len < 0 ? 0 : (len > p.K ? p.K : len);
}

constexpr float kLog2e = 1.4426950408889634f;

// P = exp(s z + bias - lse) of a valid key, formed as
// 2^(z s2 + (bias log2 e - lse2)) on v_exp_f32 with s2 = s log2 e and
// lse2 = lse log2 e.  Every kernel computes s2 and lse2 by the same fp32
// products and calls this, so P (and dz) have the same bits in all of them.
__device__ __forceinline__ float softmax_p(float z, float s2, float bias, float lse2) {
    return __builtin_amdgcn_exp2f(fmaf(z, s2, fmaf(bias, kLog2e, -lse2)));
}

// ---- tiled kernels --------------------------------------------------------
// A workgroup of 256 threads works on 32 x 32 (query, key) tiles.  Rows of
// Q, dO (32 query rows) and K, V (32 keys) are staged in LDS as fp32 with a
// padded row stride (D + 1 floats, so the column reads below hit distinct
// banks), together with Delta = dO.O, lse and a no-valid-key flag per query
// row.  pair_tile then gives thread t the pairs (t / 8, t % 8 + 8 j), j < 4,
// computes z, P, dP and dz for them from LDS and stores P and dz in 32 x 33
// LDS arrays for the accumulation step of each kernel.
constexpr int kT = 32;        // tile rows (queries) and columns (keys)
constexpr int kThreads = 256;

struct Tiles {
    float* qs;   // kT x (D + 1)
    float* gos;  // kT x (D + 1): dO
    float* ks;   // kT x (D + 1)
    float* vs;   // kT x (D + 1)
    float* ps;   // kT x (kT + 1): P
    float* dzs;  // kT x (kT + 1): dz
    float* delta;  // kT
    float* lse;    // kT
    float* dead;   // kT: 1 when the row has no valid key
};

__device__ __forceinline__ Tiles carve(float* lds, int64_t D) {
    const int64_t ld = D + 1;
    Tiles t;
    t.qs = lds;
    t.gos = t.qs + kT * ld;
    t.ks = t.gos + kT * ld;
    t.vs = t.ks + kT * ld;
    t.ps = t.vs + kT * ld;
    t.dzs = t.ps + kT * (kT + 1);
    t.delta = t.dzs + kT * (kT + 1);
    t.lse = t.delta + kT;
    t.dead = t.lse + kT;
    return t;
}

size_t lds_bytes(int64_t D) {
    return static_cast<size_t>(4 * kT * (D + 1) + 2 * kT * (kT + 1) + 3 * kT) * sizeof(float);
}

// Stage `rows` rows (from row r0 of a (rows_total, D) array) into dst as
// fp32, zero past rows_total.  Coalesced: consecutive threads take
// consecutive elements.
template <typename T>
__device__ __forceinline__ void stage(float* dst, const T* src, int64_t r0, int64_t rows_total,
                                      int64_t D) {
    const int d32 = static_cast<int>(D);
    const int64_t valid_rows = rows_total - r0;  // rows of this tile that exist
    for (int e = threadIdx.x; e < kT * d32; e += kThreads) {
        const int r = e / d32, d = e - r * d32;
        dst[r * (d32 + 1) + d] = r < valid_rows ? f32(src[(r0 + r) * D + d]) : 0.f;
    }
}

// Delta, lse and the no-valid-key flag of query rows q0 .. q0 + kT - 1 of
// slice bnh (8 threads per row, d strided by 8, reduced by shuffles).
template <typename T>
__device__ __forceinline__ void stage_rows(const Params& p, const BwdParams& g, Tiles t,
                                           int64_t bnh, int64_t q0) {
    const int r = threadIdx.x >> 3, part = threadIdx.x & 7;
    const int64_t qi = q0 + r, D = p.D;
    float acc = 0.f;
    if (qi < p.Q) {
        const T* go = static_cast<const T*>(g.dout) + (bnh * p.Q + qi) * D;
        const T* o = static_cast<const T*>(g.out) + (bnh * p.Q + qi) * D;
        for (int64_t d = part; d < D; d += 8) acc = fmaf(f32(go[d]), f32(o[d]), acc);
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 4);
    if (part == 0) {
        const int64_t row = bnh * p.Q + qi;
        t.delta[r] = acc;
        t.lse[r] = qi < p.Q ? g.lse[row] : 0.f;
        t.dead[r] = qi < p.Q && g.mx[row] == kMaskedLogit ? 1.f : 0.f;
    }
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
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

// One wave: dst[j][i] = sum_d a[i][d] b[j][d] for the 32 staged rows of a
// and of b (fp32 in LDS, stride ld), on v_mfma_f32_32x32x16 with a as the A
// operand and b transposed as the B operand.  The staged values are exact
// conversions of T, so converting them back is exact.  Lane l supplies row
// l % 32, coordinates 16 st + 8 (l / 32) .. + 7 (zero past D); its result
// register r is dst[l % 32][8 (r / 4) + 4 (l / 32) + r % 4].
template <typename T>
__device__ __forceinline__ void mfma_rows(const float* a, const float* b, int64_t D, int64_t ld,
                                          float* dst) {
    using M = Mma<T>;
    using v8 = typename M::v8;
    const int lane = threadIdx.x & 63, row = lane & 31, half = lane >> 5;
    f32x16 acc = {};
    for (int64_t st = 0; st < D; st += 16) {
        v8 va, vb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t d = st + 8 * half + e;
            va[e] = static_cast<T>(d < D ? a[row * ld + d] : 0.f);
            vb[e] = static_cast<T>(d < D ? b[row * ld + d] : 0.f);
        }
        acc = M::run(va, vb, acc);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) dst[row * (kT + 1) + 8 * (r / 4) + 4 * half + (r % 4)] = acc[r];
}

// acc += A . B over c < 32 on v_mfma_f32_32x32x16, for the 32-column block
// jb of the output: A(i, c) = a[i ars + c acs] (i < 32), B(c, j) =
// b[c brs + j] with j = 32 jb + lane % 32 (zero at j >= D); A and B are
// rounded to T (P and dz enter the contraction in the input type, the
// usual choice).  Lane l then holds out[8 (r / 4) + 4 (l / 32) + r % 4][j]
// in register r.
template <typename T>
__device__ __forceinline__ f32x16 mfma_acc(f32x16 acc, const float* a, int ars, int acs,
                                           const float* b, int64_t brs, int jb, int64_t D) {
    using M = Mma<T>;
    using v8 = typename M::v8;
    const int lane = threadIdx.x & 63, row = lane & 31, half = lane >> 5;
    const int64_t j = 32 * jb + row;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        v8 va, vb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = 16 * st + 8 * half + e;
            va[e] = static_cast<T>(a[row * ars + c * acs]);
            vb[e] = static_cast<T>(j < D ? b[c * brs + j] : 0.f);
        }
        acc = M::run(va, vb, acc);
    }
    return acc;
}

// Row index of register r of lane l in an MFMA result block.
__device__ __forceinline__ int mfma_row(int r, int lane) {
    return 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
}

// P and dz of the tile's pairs, from the staged rows (see Tiles).  z = Q.K
// and dP = dO.V come from two MFMA waves for the half types (through the ps
// and dzs arrays, which every thread then overwrites only at its own
// pairs), and from fp32 FMAs for fp32 inputs.  Every thread of the
// workgroup must call it (it holds a barrier for the half types).
template <typename T>
// blk_state: -1, or (block lists whose kv block holds the whole 32-key tile)
// this row's state of that block, bit 0 listed and bit 1 full (row_block_state)
__device__ __forceinline__ void pair_tile(const Params& p, Tiles t, int64_t b, int64_t n,
                                          int64_t h, int64_t q0, int64_t k0, int blk_state = -1) {
    const int64_t D = p.D, ld = D + 1;
    const int ql = threadIdx.x >> 3, kb = threadIdx.x & 7;
    float z[4] = {0.f, 0.f, 0.f, 0.f}, dp[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (std::is_same<T, float>::value) {
        const float* qr = t.qs + ql * ld;
        const float* gr = t.gos + ql * ld;
        for (int64_t d = 0; d < D; ++d) {
            const float qd = qr[d], gd = gr[d];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int kl = kb + 8 * j;
                z[j] = fmaf(qd, t.ks[kl * ld + d], z[j]);
                dp[j] = fmaf(gd, t.vs[kl * ld + d], dp[j]);
            }
        }
    } else {
        const int wave = threadIdx.x >> 6;
        if (wave == 0) mfma_rows<T>(t.ks, t.qs, D, ld, t.ps);
        if (wave == 1) mfma_rows<T>(t.vs, t.gos, D, ld, t.dzs);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            z[j] = t.ps[ql * (kT + 1) + kb + 8 * j];
            dp[j] = t.dzs[ql * (kT + 1) + kb + 8 * j];
        }
    }
    const int64_t qi = q0 + ql;
    const bool dead = t.dead[ql] != 0.f;
    const float inv_k = 1.0f / static_cast<float>(p.K);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int kl = kb + 8 * j;
        const int64_t kk = k0 + kl;
        float pr = 0.f, dz = 0.f;
        if (qi < p.Q && kk < p.K) {
            if (dead) {
                pr = inv_k;
            } else if (blk_state >= 0
                           ? ((blk_state & 2) != 0 ||
                              ((blk_state & 1) != 0 && (p.mask_mod != TRIATTN_MOD_CAUSAL || qi >= kk)))
                           : key_valid(p, b, n, h, qi, kk)) {
                const float bias = p.bias ? p.bias[((b * p.H + h) * p.Q + qi) * p.K + kk] : 0.f;
                pr = softmax_p(z[j], p.scale * kLog2e, bias, t.lse[ql] * kLog2e);
                dz = pr * (dp[j] - t.delta[ql]);
            }
        }
        t.ps[ql * (kT + 1) + kl] = pr;
        t.dzs[ql * (kT + 1) + kl] = dz;
    }
}

// Block lists whose kv blocks are whole 32-key tiles: the state of kv block
// `blk` in the list rows of query row qi (bit 0 listed in the kv or full
// list, bit 1 in the full list), the same as key_valid's tests for every key
// of the block.  The 8 threads of a row (consecutive lanes, threadIdx.x % 8
// = kb) scan every 8th entry and combine their findings, so every thread
// must call it.
__device__ int row_block_state(const Params& p, int64_t b, int64_t n, int64_t h, int64_t qi,
                               int64_t blk, int kb) {
    const int64_t inst = b * p.stride_b + n * p.stride_n + h * p.stride_h;
    const int64_t qc = qi < p.Q ? qi : p.Q - 1;
    const int64_t row = inst * p.n_q_rows + qc / p.q_block;
    int st = 0;
    auto scan = [&](const int32_t* counts, const int32_t* ids, int64_t width, int bits) {
        int64_t count = counts[row];
        count = count < 0 ? 0 : (count > width ? width : count);
        for (int64_t j = kb; j < count; j += 8)
            if (ids[row * width + j] == blk) st |= bits;
    };
    scan(p.kv_num_blocks, p.kv_indices, p.max_blocks, 1);
    if (p.full_kv_num_blocks) scan(p.full_kv_num_blocks, p.full_kv_indices, p.full_max_blocks, 3);
    st |= __shfl_xor(st, 1);
    st |= __shfl_xor(st, 2);
    st |= __shfl_xor(st, 4);
    return st;
}

// pair_tile's blk_state for this thread's row of the tile at (q0, k0):
// the row's block state for block lists whose kv blocks are whole 32-key
// tiles, else -1 (key_valid per element).  Called by every thread.
__device__ int tile_block_state(const Params& p, int64_t b, int64_t n, int64_t h, int64_t q0,
                                int64_t k0) {
    if (p.mask_kind != TRIATTN_MASK_BLOCK || p.kv_block % kT != 0) return -1;
    const int ql = threadIdx.x >> 3, kb = threadIdx.x & 7;
    return row_block_state(p, b, n, h, q0 + ql, k0 / p.kv_block, kb);
}

// dQ: one workgroup per (b, n, h, 32 query rows); loops over key tiles.
// Thread t owns row t / 8 and columns d = t % 8 + 8 i.
template <typename T, int NC>
__global__ __launch_bounds__(kThreads) void dq_kernel(Params p, BwdParams g) {
    extern __shared__ float lds[];
    const int64_t D = p.D, ld = D + 1;
    const Tiles t = carve(lds, D);
    const int64_t n_qt = (p.Q + kT - 1) / kT;
    const int64_t bnh = blockIdx.x / n_qt, q0 = (blockIdx.x % n_qt) * kT;
    const int64_t h = bnh % p.H, n = (bnh / p.H) % p.N, b = bnh / (p.H * p.N);
    stage(t.qs, static_cast<const T*>(p.q) + bnh * p.Q * D, q0, p.Q, D);
    stage(t.gos, static_cast<const T*>(g.dout) + bnh * p.Q * D, q0, p.Q, D);
    stage_rows<T>(p, g, t, bnh, q0);
    const int r = threadIdx.x >> 3, part = threadIdx.x & 7;
    constexpr bool kMfma = !std::is_same<T, float>::value;
    // half types: wave w accumulates the 32-column blocks w, w + 4, ... of dQ
    constexpr int kPer = NC >= 32 ? 2 : 1;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n_jb = static_cast<int>((D + 31) / 32);
    f32x16 macc[kPer];
#pragma unroll
    for (int m = 0; m < kPer; ++m) macc[m] = f32x16{};
    float acc[kMfma ? 1 : NC];
#pragma unroll
    for (int i = 0; i < (kMfma ? 1 : NC); ++i) acc[i] = 0.f;
    const int64_t k_end = key_limit(p, b, n);  // dz is 0 past it (and everywhere if 0)
    for (int64_t k0 = 0; k0 < k_end; k0 += kT) {
        __syncthreads();  // previous tile's reads done
        stage(t.ks, static_cast<const T*>(p.k) + bnh * p.K * D, k0, p.K, D);
        stage(t.vs, static_cast<const T*>(p.v) + bnh * p.K * D, k0, p.K, D);
        __syncthreads();
        pair_tile<T>(p, t, b, n, h, q0, k0, tile_block_state(p, b, n, h, q0, k0));
        __syncthreads();
        if constexpr (kMfma) {
            // dQ(q, d) += sum_k dz(q, k) K(k, d)
#pragma unroll
            for (int m = 0; m < kPer; ++m) {
                const int jb = wave + 4 * m;
                if (jb < n_jb) macc[m] = mfma_acc<T>(macc[m], t.dzs, kT + 1, 1, t.ks, ld, jb, D);
            }
        } else {
            for (int kl = 0; kl < kT; ++kl) {
                const float dz = t.dzs[r * (kT + 1) + kl];
                const float* kr = t.ks + kl * ld;
#pragma unroll
                for (int i = 0; i < NC; ++i) {
                    const int64_t d = part + 8 * i;
                    if (d < D) acc[i] = fmaf(dz, kr[d], acc[i]);
                }
            }
        }
    }
    if constexpr (kMfma) {
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            const int jb = wave + 4 * m;
            const int64_t d = 32 * jb + (lane & 31);
            if (jb >= n_jb || d >= D) continue;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int64_t qi = q0 + mfma_row(rr, lane);
                if (qi < p.Q)
                    static_cast<T*>(g.dq)[(bnh * p.Q + qi) * D + d] =
                        static_cast<T>(macc[m][rr] * p.scale);
            }
        }
        return;
    }
    const int64_t qi = q0 + r;
    if (qi >= p.Q) return;
    T* dqr = static_cast<T*>(g.dq) + (bnh * p.Q + qi) * D;
#pragma unroll
    for (int i = 0; i < (kMfma ? 1 : NC); ++i) {
        const int64_t d = part + 8 * i;
        if (d < D) dqr[d] = static_cast<T>(acc[i] * p.scale);
    }
}

// dK and dV: one workgroup per (b, n, h, 32 keys); loops over query tiles.
// Thread t owns key t / 8 and columns d = t % 8 + 8 i.
template <typename T, int NC>
__global__ __launch_bounds__(kThreads) void dkdv_kernel(Params p, BwdParams g) {
    extern __shared__ float lds[];
    const int64_t D = p.D, ld = D + 1;
    const Tiles t = carve(lds, D);
    const int64_t n_kt = (p.K + kT - 1) / kT;
    const int64_t bnh = blockIdx.x / n_kt, k0 = (blockIdx.x % n_kt) * kT;
    const int64_t h = bnh % p.H, n = (bnh / p.H) % p.N, b = bnh / (p.H * p.N);
    stage(t.ks, static_cast<const T*>(p.k) + bnh * p.K * D, k0, p.K, D);
    stage(t.vs, static_cast<const T*>(p.v) + bnh * p.K * D, k0, p.K, D);
    const int kr = threadIdx.x >> 3, part = threadIdx.x & 7;
    constexpr bool kMfma = !std::is_same<T, float>::value;
    // half types: waves 0-1 accumulate dV, waves 2-3 dK, each over the
    // 32-column blocks (w % 2), (w % 2) + 2, ...
    constexpr int kPer = NC >= 16 ? NC / 8 : 1;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n_jb = static_cast<int>((D + 31) / 32);
    const bool wave_dk = wave >= 2;
    f32x16 macc[kPer];
#pragma unroll
    for (int m = 0; m < kPer; ++m) macc[m] = f32x16{};
    constexpr int kF = kMfma ? 1 : NC;
    float dk[kF], dv[kF];
#pragma unroll
    for (int i = 0; i < kF; ++i) dk[i] = dv[i] = 0.f;
    // A key tile at or past a nonzero length limit gets P = dz = 0 from every
    // row: dK = dV = 0 without the loop (a zero limit means rows without a
    // valid key, whose uniform weights reach every key).
    const int64_t lim = key_limit(p, b, n);
    const int64_t q_end = (lim > 0 && k0 >= lim) ? 0 : p.Q;
    for (int64_t q0 = 0; q0 < q_end; q0 += kT) {
        __syncthreads();
        stage(t.qs, static_cast<const T*>(p.q) + bnh * p.Q * D, q0, p.Q, D);
        stage(t.gos, static_cast<const T*>(g.dout) + bnh * p.Q * D, q0, p.Q, D);
        stage_rows<T>(p, g, t, bnh, q0);
        __syncthreads();
        pair_tile<T>(p, t, b, n, h, q0, k0, tile_block_state(p, b, n, h, q0, k0));
        __syncthreads();
        if constexpr (kMfma) {
            // dV(k, d) += sum_q P(q, k) dO(q, d);  dK(k, d) += sum_q dz(q, k) Q(q, d)
#pragma unroll
            for (int m = 0; m < kPer; ++m) {
                const int jb = (wave & 1) + 2 * m;
                if (jb < n_jb)
                    macc[m] = wave_dk ? mfma_acc<T>(macc[m], t.dzs, 1, kT + 1, t.qs, ld, jb, D)
                                      : mfma_acc<T>(macc[m], t.ps, 1, kT + 1, t.gos, ld, jb, D);
            }
        } else {
            for (int ql = 0; ql < kT; ++ql) {
                const float pr = t.ps[ql * (kT + 1) + kr], dz = t.dzs[ql * (kT + 1) + kr];
                const float* qrow = t.qs + ql * ld;
                const float* grow = t.gos + ql * ld;
#pragma unroll
                for (int i = 0; i < kF; ++i) {
                    const int64_t d = part + 8 * i;
                    if (d < D) {
                        dv[i] = fmaf(pr, grow[d], dv[i]);
                        dk[i] = fmaf(dz, qrow[d], dk[i]);
                    }
                }
            }
        }
    }
    if constexpr (kMfma) {
        T* dst = static_cast<T*>(wave_dk ? g.dk : g.dv);
        const float mul = wave_dk ? p.scale : 1.0f;
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            const int jb = (wave & 1) + 2 * m;
            const int64_t d = 32 * jb + (lane & 31);
            if (jb >= n_jb || d >= D) continue;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int64_t kk2 = k0 + mfma_row(rr, lane);
                if (kk2 < p.K) dst[(bnh * p.K + kk2) * D + d] = static_cast<T>(macc[m][rr] * mul);
            }
        }
        return;
    }
    const int64_t kk = k0 + kr;
    if (kk >= p.K) return;
    T* dkr = static_cast<T*>(g.dk) + (bnh * p.K + kk) * D;
    T* dvr = static_cast<T*>(g.dv) + (bnh * p.K + kk) * D;
#pragma unroll
    for (int i = 0; i < kF; ++i) {
        const int64_t d = part + 8 * i;
        if (d < D) {
            dkr[d] = static_cast<T>(dk[i] * p.scale);
            dvr[d] = static_cast<T>(dv[i]);
        }
    }
}

// dBias: one workgroup per (b, h, 32 query rows, kChunk key tiles); loops
// over n (in order) and, for each n, over its key tiles, adding dz into its
// own block of the output (zeroed first).  Q, dO and Delta are staged once
// per n for all the key tiles of the chunk.  Deterministic: every element
// is owned by one thread of one workgroup and summed in n order.
constexpr int kChunk = 4;  // key tiles per dBias workgroup

template <typename T, int NC>
__global__ __launch_bounds__(kThreads) void dbias_kernel(Params p, BwdParams g) {
    extern __shared__ float lds[];
    const int64_t D = p.D;
    const Tiles t = carve(lds, D);
    const int64_t n_qt = (p.Q + kT - 1) / kT;
    const int64_t n_kc = (p.K + kT * kChunk - 1) / (kT * kChunk);
    const int64_t bh = blockIdx.x / (n_qt * n_kc);
    const int64_t q0 = ((blockIdx.x / n_kc) % n_qt) * kT;
    const int64_t kc0 = (blockIdx.x % n_kc) * kT * kChunk;
    const int64_t kc1 = kc0 + kT * kChunk < p.K ? kc0 + kT * kChunk : p.K;
    const int64_t h = bh % p.H, b = bh / p.H;
    const int ql = threadIdx.x >> 3, kb = threadIdx.x & 7;
    const int64_t qi = q0 + ql;
    float* dbr = g.dbias + (bh * p.Q + qi) * p.K;  // this thread's row (when qi < Q)
    if (qi < p.Q)
        for (int64_t kk = kc0 + kb; kk < kc1; kk += 8) dbr[kk] = 0.f;
    for (int64_t n = 0; n < p.N; ++n) {
        const int64_t bnh = (b * p.N + n) * p.H + h;
        const int64_t lim = key_limit(p, b, n);
        const int64_t k_end = kc1 < lim ? kc1 : lim;  // dz = 0 at and past lim (all if 0)
        if (k_end <= kc0) continue;  // uniform
        __syncthreads();
        stage(t.qs, static_cast<const T*>(p.q) + bnh * p.Q * D, q0, p.Q, D);
        stage(t.gos, static_cast<const T*>(g.dout) + bnh * p.Q * D, q0, p.Q, D);
        stage_rows<T>(p, g, t, bnh, q0);
        for (int64_t k0 = kc0; k0 < k_end; k0 += kT) {
            __syncthreads();
            stage(t.ks, static_cast<const T*>(p.k) + bnh * p.K * D, k0, p.K, D);
            stage(t.vs, static_cast<const T*>(p.v) + bnh * p.K * D, k0, p.K, D);
            __syncthreads();
            pair_tile<T>(p, t, b, n, h, q0, k0, tile_block_state(p, b, n, h, q0, k0));
            if (qi < p.Q) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t kk = k0 + kb + 8 * j;
                    if (kk < p.K) dbr[kk] += t.dzs[ql * (kT + 1) + kb + 8 * j];
                }
            }
        }
    }
}

// The general kernels.
template <typename T, int NC>
hipError_t launch_nc(const Params& p, const BwdParams& g, hipStream_t stream) {
    const int64_t n_qt = (p.Q + kT - 1) / kT, n_kt = (p.K + kT - 1) / kT;
    const int64_t n_kc = (p.K + kT * kChunk - 1) / (kT * kChunk);
    const int64_t gq = p.B * p.N * p.H * n_qt, gk = p.B * p.N * p.H * n_kt,
                  gb = p.B * p.H * n_qt * n_kc;
    if (gq > 0x7fffffff || gk > 0x7fffffff || gb > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    const size_t shm = lds_bytes(p.D);
    const dim3 block(kThreads);
    if (shm > 65536) {
        // more than 64 KiB of LDS per workgroup (D > 64; gfx950 has 160 KiB)
        const int b = static_cast<int>(shm);
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(dq_kernel<T, NC>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, b);
        if (e == hipSuccess)
            e = hipFuncSetAttribute(reinterpret_cast<const void*>(dkdv_kernel<T, NC>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, b);
        if (e == hipSuccess)
            e = hipFuncSetAttribute(reinterpret_cast<const void*>(dbias_kernel<T, NC>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, b);
        if (e != hipSuccess) return e;
    }
    if (gq > 0)
        hipLaunchKernelGGL((dq_kernel<T, NC>), dim3(static_cast<unsigned>(gq)), block, shm, stream, p, g);
    if (gk > 0)
        hipLaunchKernelGGL((dkdv_kernel<T, NC>), dim3(static_cast<unsigned>(gk)), block, shm, stream, p, g);
    if (g.dbias && gb > 0)
        hipLaunchKernelGGL((dbias_kernel<T, NC>), dim3(static_cast<unsigned>(gb)), block, shm, stream, p, g);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const Params& p, const BwdParams& g, hipStream_t stream) {
    if (p.D <= 32) return launch_nc<T, 4>(p, g, stream);
    if (p.D <= 64) return launch_nc<T, 8>(p, g, stream);
    if (p.D <= 128) return launch_nc<T, 16>(p, g, stream);
    return launch_nc<T, 32>(p, g, stream);
}

}  // namespace

hipError_t launch_bwd(const Params& p, const BwdParams& g, int32_t dtype, float* ws,
                      size_t ws_bytes, hipStream_t stream) {
    if (bwd_mfma_supports(p, dtype))
        return p.D <= 32   ? launch_bwd_mfma_d32(p, g, dtype, ws, ws_bytes, stream)
               : p.D <= 64 ? launch_bwd_mfma_d64(p, g, dtype, ws, ws_bytes, stream)
                           : launch_bwd_mfma_d128(p, g, dtype, ws, ws_bytes, stream);
    switch (dtype) {
    case TRIATTN_F32:
        return launch_t<float>(p, g, stream);
    case TRIATTN_F16:
        return launch_t<_Float16>(p, g, stream);
    case TRIATTN_BF16:
        return launch_t<__bf16>(p, g, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace triattn
