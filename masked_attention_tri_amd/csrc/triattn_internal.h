// Internal declarations shared by the host entry points and the kernels of
// libtriattn.  Not part of the public ABI (that is include/triattn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "triattn.h"

namespace triattn {

// Every argument of one forward call, flattened into a POD that is passed to
// the kernels by value.
struct Params {
    const void* q;
    const void* k;
    const void* v;
    const float* bias;    // (B,1,H,Q,K) fp32, or nullptr
    const void* bias16;   // (B,1,H,Q,K) in the input type (then bias is nullptr), or nullptr
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
    // Packed variable-length sequences (mask kind kMaskVarlen): B counts
    // sequences, N = 1, Q and K are the largest lengths the launch covers,
    // and sequence b is rows cu_q[b] .. cu_q[b+1]-1 of q / out and cu_kv[b]
    // .. cu_kv[b+1]-1 of k / v.  Each packed row holds all H heads; q_rs and
    // kv_rs are the row strides of q and of k / v in elements (out and the
    // (row, head) lse / max are contiguous).
    const int32_t* cu_q;
    const int32_t* cu_kv;
    int64_t total_q, total_kv;  // rows of the packed tensors
    int64_t q_rs, kv_rs;
    int32_t causal;  // varlen: key j of query row i valid only if j <= i
};

// Internal mask kind of the packed variable-length layouts (not a value of
// the public tri_attn_mask_kind).
constexpr int32_t kMaskVarlen = 4;

// Rows of one packed sequence, read from the cu_seqlens arrays and clamped
// so that they always lie inside the packed tensors: the boundaries are
// clamped to [0, total] and made ascending, and the lengths to the launch's
// maxima Q and K.
struct SeqRows {
    int64_t q0, nq, k0, nk;
};
__device__ __forceinline__ SeqRows seq_rows(const Params& p, int64_t b) {
    auto clampi = [](int64_t x, int64_t lo, int64_t hi) { return x < lo ? lo : (x > hi ? hi : x); };
    SeqRows r;
    r.q0 = clampi(p.cu_q[b], 0, p.total_q);
    const int64_t q1 = clampi(p.cu_q[b + 1], r.q0, p.total_q);
    r.k0 = clampi(p.cu_kv[b], 0, p.total_kv);
    const int64_t k1 = clampi(p.cu_kv[b + 1], r.k0, p.total_kv);
    r.nq = q1 - r.q0 < p.Q ? q1 - r.q0 : p.Q;
    r.nk = k1 - r.k0 < p.K ? k1 - r.k0 : p.K;
    return r;
}

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
};

// Masked logits are carried as -inf inside the kernels: when a row has at
// least one valid key this gives exactly the weights of the -1e9
// replacement (exp underflows to 0 either way); rows with no valid key are
// detected from their running max and take the uniform-weight result.
constexpr float kMaskedLogit = -1.0e9f;

// Largest number of kv blocks a block-sparse mask may have: the kernels keep
// one visited bit and one full bit per block in LDS.
constexpr int64_t kMaxKvBlocks = 8192;

// Bytes of the backward's per-row data for `slices` (b, n, h) slices of Q
// rows: 260 per slice and 32-row tile (two planes of 32 floats and a count),
// rounded up to 16 (what follows stays 16-byte aligned); -1 past int64.
inline int64_t bwd_rows_bytes(int64_t slices, int64_t Q) {
    if (slices < 0 || Q < 0) return -1;
    const int64_t tiles = Q == 0 ? 0 : (Q - 1) / 32 + 1;
    if (tiles != 0 && slices > INT64_MAX / 272 / tiles) return -1;
    return (slices * tiles * 260 + 15) / 16 * 16;
}

// Ranges of n the MFMA dBias kernel splits its sum into for a shape: its
// workgroups cover 128 x 128 (query, key) tiles (64 x 64 at D = 128), one
// resident per CU, and there are 256 CUs; the split that fills whole rounds
// of workgroups best (ties: fewer splits), at most 8 and at least 16 n each.
// With more than one split, each needs a B H Q K fp32 plane of workspace.
inline int dbias_splits(int64_t B, int64_t N, int64_t H, int64_t Q, int64_t K, int64_t Dh) {
    // the tile width that serves head dimension Dh
    if (Dh % 8 != 0 || Dh < 8 || Dh > 128) return 1;
    const int64_t D = Dh <= 32 ? 32 : Dh <= 64 ? 64 : 128;
    // (sizes past these the kernels never take; no product below overflows)
    const int64_t lim = int64_t(1) << 31;
    if (B < 1 || H < 1 || Q < 1 || K < 1 || N < 1 || B > lim || H > lim || Q > lim || K > lim ||
        B * H > lim)
        return 1;
    const int64_t rows_q = D <= 64 ? 128 : 64, rows_k = D <= 64 ? 128 : 64;
    const double tiles = static_cast<double>(B * H) * static_cast<double>((Q - 1) / rows_q + 1) *
                         static_cast<double>((K - 1) / rows_k + 1);
    const double slots = 256.0;  // resident workgroups: one per CU
    int best = 1;
    double best_eff = 0.0;
    for (int s = 1; s <= 8 && (s == 1 || N / s >= 16); ++s) {
        const double wg = tiles * s;
        const double rounds = ceil(wg / slots);
        const double eff = wg / (rounds * slots);
        if (eff > best_eff + 1e-9) {
            best_eff = eff;
            best = s;
        }
    }
    return best;
}

// Launchers (enqueue only; return the launch error, if any).
hipError_t launch_generic(const Params& p, int32_t dtype, hipStream_t stream);
// fp32 inputs with no mask, kv_lengths or a dense mask: the MFMA kernel of
// kernel_fp32.hip (launch_generic hands them to it)
bool fp32_mfma_supports(const Params& p);
hipError_t launch_fp32_mfma(const Params& p, hipStream_t stream);
hipError_t launch_mfma(const Params& p, int32_t dtype, hipStream_t stream);
bool mfma_supports(const Params& p, int32_t dtype);
// The MFMA kernel's instantiations, one per head dimension (exact: the scale
// is folded into Q exactly).
hipError_t launch_mfma_d32(const Params& p, int32_t dtype, bool exact, hipStream_t stream);
hipError_t launch_mfma_d64(const Params& p, int32_t dtype, bool exact, hipStream_t stream);
hipError_t launch_mfma_d128(const Params& p, int32_t dtype, bool exact, hipStream_t stream);
hipError_t launch_mfma_d256(const Params& p, int32_t dtype, bool exact, hipStream_t stream);
// The backward: per-row data in `ws` (bwd_rows_bytes; the rest, if any,
// holds dBias partial sums), then dK / dV, dQ and dBias.
hipError_t launch_bwd(const Params& p, const BwdParams& g, int32_t dtype, float* ws,
                      size_t ws_bytes, hipStream_t stream);
// Calls the MFMA backward kernels (bf16 / fp16, D in {32, 64, 128}) serve,
// and their instantiations per head dimension.
bool bwd_mfma_supports(const Params& p, int32_t dtype);
hipError_t launch_bwd_mfma_d32(const Params& p, const BwdParams& g, int32_t dtype, float* ws,
                               size_t ws_bytes, hipStream_t stream);
hipError_t launch_bwd_mfma_d64(const Params& p, const BwdParams& g, int32_t dtype, float* ws,
                               size_t ws_bytes, hipStream_t stream);
hipError_t launch_bwd_mfma_d128(const Params& p, const BwdParams& g, int32_t dtype, float* ws,
                               size_t ws_bytes, hipStream_t stream);
// Host-only validation of tri_attn_bwd's arguments (the checks it returns
// before launching anything; the workspace's only with check_workspace).
triattn_status bwd_validate(const tri_attn_shape* shape, int32_t dtype, const void* q,
                            const void* k, const void* v, const float* bias,
                            const tri_attn_mask* mask, float scale, const void* out,
                            const void* dout, const float* lse, const float* max, const void* dq,
                            const void* dk, const void* dv, const float* dbias,
                            const float* workspace, size_t workspace_bytes,
                            bool check_workspace = true);
hipError_t launch_mask_to_kv_lengths(const uint8_t* mask, int64_t rows, int64_t K,
                                     int32_t* kv_lengths, int32_t* nonprefix_rows,
                                     hipStream_t stream);

}  // namespace triattn
