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
// Three plain fp32 kernels, one wavefront per output row, no atomics:
//   dq_kernel    one (b,n,h,q) row: lanes split the keys (chunks of 64) for
//                z and dz, then broadcast dz_j to accumulate dQ over d.
//   dkdv_kernel  one (b,n,h,k) key: lanes split the query rows, then
//                broadcast to accumulate dK and dV over d.
//   dbias_kernel one (b,h,q) row: lanes split the keys and each lane sums
//                dz over n for its key.
// Each lane holds up to kOut = 4 coordinates of a D <= 256 vector (d = lane +
// 64 i).  These are correctness-first VALU kernels, not tuned.
#include <math.h>

#include "triattn_internal.h"

namespace triattn {
namespace {

constexpr int kWaves = 4;
constexpr int kOut = 4;

template <typename T>
__device__ __forceinline__ float f32(T x) {
    return static_cast<float>(x);
}

__device__ __forceinline__ float wave_sum(float x) {
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
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

template <typename T>
__device__ __forceinline__ float dot_rows(const T* a, const T* b, int64_t D) {
    float acc = 0.f;
    for (int64_t d = 0; d < D; ++d) acc = fmaf(f32(a[d]), f32(b[d]), acc);
    return acc;
}

// dQ: one wave per (b, n, h, q) row.
template <typename T>
__global__ __launch_bounds__(64 * kWaves) void dq_kernel(Params p, BwdParams g) {
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
    if (row >= p.B * p.N * p.H * p.Q) return;
    const int64_t qi = row % p.Q, h = (row / p.Q) % p.H, n = (row / (p.Q * p.H)) % p.N,
                  b = row / (p.Q * p.H * p.N);
    const int64_t D = p.D, K = p.K, bnh = (b * p.N + n) * p.H + h;
    const T* qr = static_cast<const T*>(p.q) + row * D;
    const T* go = static_cast<const T*>(g.dout) + row * D;
    const T* o = static_cast<const T*>(g.out) + row * D;
    const T* kb = static_cast<const T*>(p.k) + bnh * K * D;
    const T* vb = static_cast<const T*>(p.v) + bnh * K * D;
    const float* br = p.bias ? p.bias + ((b * p.H + h) * p.Q + qi) * K : nullptr;
    T* dqr = static_cast<T*>(g.dq) + row * D;

    float acc[kOut];
#pragma unroll
    for (int i = 0; i < kOut; ++i) acc[i] = 0.f;
    const bool dead = g.mx[row] == kMaskedLogit;
    if (!dead) {
        const float lse = g.lse[row];
        const float delta = dot_rows(go, o, D);  // dO . O
        for (int64_t c0 = 0; c0 < K; c0 += 64) {
            const int64_t kk = c0 + lane;
            float dz = 0.f;
            if (kk < K && key_valid(p, b, n, h, qi, kk)) {
                const float z = fmaf(dot_rows(qr, kb + kk * D, D), p.scale, br ? br[kk] : 0.f);
                const float pr = expf(z - lse);
                dz = pr * (dot_rows(go, vb + kk * D, D) - delta);
            }
            const int jmax = (K - c0) < 64 ? static_cast<int>(K - c0) : 64;
            for (int j = 0; j < jmax; ++j) {
                const float dzj = __shfl(dz, j);
                if (dzj == 0.f) continue;  // uniform across the wave
                const T* krow = kb + (c0 + j) * D;
#pragma unroll
                for (int i = 0; i < kOut; ++i)
                    if (lane + 64 * i < D) acc[i] = fmaf(dzj, f32(krow[lane + 64 * i]), acc[i]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kOut; ++i)
        if (lane + 64 * i < D) dqr[lane + 64 * i] = static_cast<T>(acc[i] * p.scale);
}

// dK and dV: one wave per (b, n, h, k) key row.
template <typename T>
__global__ __launch_bounds__(64 * kWaves) void dkdv_kernel(Params p, BwdParams g) {
    const int lane = threadIdx.x & 63;
    const int64_t krow_i = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
    if (krow_i >= p.B * p.N * p.H * p.K) return;
    const int64_t kk = krow_i % p.K, h = (krow_i / p.K) % p.H, n = (krow_i / (p.K * p.H)) % p.N,
                  b = krow_i / (p.K * p.H * p.N);
    const int64_t D = p.D, Q = p.Q, bnh = (b * p.N + n) * p.H + h;
    const T* kr = static_cast<const T*>(p.k) + krow_i * D;
    const T* vr = static_cast<const T*>(p.v) + krow_i * D;
    const T* qb = static_cast<const T*>(p.q) + bnh * Q * D;
    const T* gob = static_cast<const T*>(g.dout) + bnh * Q * D;
    const T* ob = static_cast<const T*>(g.out) + bnh * Q * D;
    const float inv_k = 1.0f / static_cast<float>(p.K);

    float dk[kOut], dv[kOut];
#pragma unroll
    for (int i = 0; i < kOut; ++i) dk[i] = dv[i] = 0.f;
    for (int64_t c0 = 0; c0 < Q; c0 += 64) {
        const int64_t qi = c0 + lane;
        float pr = 0.f, dz = 0.f;
        if (qi < Q) {
            const int64_t row = bnh * Q + qi;
            if (g.mx[row] == kMaskedLogit) {
                pr = inv_k;  // no valid key in this row: uniform weights
            } else if (key_valid(p, b, n, h, qi, kk)) {
                const float bias = p.bias ? p.bias[((b * p.H + h) * Q + qi) * p.K + kk] : 0.f;
                const float z = fmaf(dot_rows(qb + qi * D, kr, D), p.scale, bias);
                pr = expf(z - g.lse[row]);
                dz = pr * (dot_rows(gob + qi * D, vr, D) - dot_rows(gob + qi * D, ob + qi * D, D));
            }
        }
        const int jmax = (Q - c0) < 64 ? static_cast<int>(Q - c0) : 64;
        for (int j = 0; j < jmax; ++j) {
            const float pj = __shfl(pr, j), dzj = __shfl(dz, j);
            if (pj == 0.f && dzj == 0.f) continue;  // uniform across the wave
            const T* gq = gob + (c0 + j) * D;
            const T* qq = qb + (c0 + j) * D;
#pragma unroll
            for (int i = 0; i < kOut; ++i) {
                const int64_t d = lane + 64 * i;
                if (d < D) {
                    dv[i] = fmaf(pj, f32(gq[d]), dv[i]);
                    dk[i] = fmaf(dzj, f32(qq[d]), dk[i]);
                }
            }
        }
    }
    T* dkr = static_cast<T*>(g.dk) + krow_i * D;
    T* dvr = static_cast<T*>(g.dv) + krow_i * D;
#pragma unroll
    for (int i = 0; i < kOut; ++i)
        if (lane + 64 * i < D) {
            dkr[lane + 64 * i] = static_cast<T>(dk[i] * p.scale);
            dvr[lane + 64 * i] = static_cast<T>(dv[i]);
        }
}

// dBias: one wave per (b, h, q) row; each lane sums dz over n for its keys.
template <typename T>
__global__ __launch_bounds__(64 * kWaves) void dbias_kernel(Params p, BwdParams g) {
    const int lane = threadIdx.x & 63;
    const int64_t r = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
    if (r >= p.B * p.H * p.Q) return;
    const int64_t qi = r % p.Q, h = (r / p.Q) % p.H, b = r / (p.Q * p.H);
    const int64_t D = p.D, K = p.K;
    const float* br = p.bias ? p.bias + r * K : nullptr;  // (B,1,H,Q,K): row r
    float* dbr = g.dbias + r * K;
    for (int64_t c0 = 0; c0 < K; c0 += 64) {
        const int64_t kk = c0 + lane;
        float acc = 0.f;
        if (kk < K) {
            for (int64_t n = 0; n < p.N; ++n) {
                const int64_t bnh = (b * p.N + n) * p.H + h;
                const int64_t row = bnh * p.Q + qi;
                if (g.mx[row] == kMaskedLogit || !key_valid(p, b, n, h, qi, kk)) continue;
                const T* qr = static_cast<const T*>(p.q) + row * D;
                const T* go = static_cast<const T*>(g.dout) + row * D;
                const T* o = static_cast<const T*>(g.out) + row * D;
                const T* krow = static_cast<const T*>(p.k) + (bnh * K + kk) * D;
                const T* vrow = static_cast<const T*>(p.v) + (bnh * K + kk) * D;
                const float z = fmaf(dot_rows(qr, krow, D), p.scale, br ? br[kk] : 0.f);
                const float pr = expf(z - g.lse[row]);
                acc += pr * (dot_rows(go, vrow, D) - dot_rows(go, o, D));
            }
            dbr[kk] = acc;
        }
    }
}

template <typename T>
hipError_t launch_t(const Params& p, const BwdParams& g, hipStream_t stream) {
    const dim3 block(64 * kWaves);
    auto grid = [](int64_t rows) { return (rows + kWaves - 1) / kWaves; };
    const int64_t gq = grid(p.B * p.N * p.H * p.Q), gk = grid(p.B * p.N * p.H * p.K),
                  gb = grid(p.B * p.H * p.Q);
    if (gq > 0x7fffffff || gk > 0x7fffffff || gb > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    if (gq > 0) hipLaunchKernelGGL(dq_kernel<T>, dim3(static_cast<unsigned>(gq)), block, 0, stream, p, g);
    if (gk > 0)
        hipLaunchKernelGGL(dkdv_kernel<T>, dim3(static_cast<unsigned>(gk)), block, 0, stream, p, g);
    if (g.dbias && gb > 0)
        hipLaunchKernelGGL(dbias_kernel<T>, dim3(static_cast<unsigned>(gb)), block, 0, stream, p, g);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const Params& p, const BwdParams& g, int32_t dtype, hipStream_t stream) {
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
