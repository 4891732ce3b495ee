// Host entry points of libtriattn: argument validation, instantiation
// choice and launch.  The arguments follow the triangle_attention API page
// (q, k, v, bias, mask | kv_lengths, scale; outputs O, lse, max) and the
// BlockMask list format of the tensorplay.nn.attention page; the calling
// convention (caller-owned buffers, scalar scale, stream last) follows the
// fused-attention C functions of Transformer Engine's fused_attn.h.
#include <math.h>
#include <stdint.h>

#include "triattn_internal.h"

namespace {

using triattn::Params;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// a*b without signed overflow, or -1.
int64_t mul_or_neg(int64_t a, int64_t b) {
    if (a < 0 || b < 0) return -1;
    if (a == 0 || b == 0) return 0;
    if (a > INT64_MAX / b) return -1;
    return a * b;
}

triattn_status check_impl(const tri_attn_shape* shape, int32_t dtype, const void* q,
                          const void* k, const void* v, const float* bias,
                          const tri_attn_mask* mask, float scale, const void* out,
                          const float* lse, const float* mx) {
    if (!shape) return TRIATTN_ERR_INVALID_ARG;
    const int64_t B = shape->B, N = shape->N, H = shape->H, Q = shape->Q, K = shape->K,
                  D = shape->D;
    if (B < 0 || N < 0 || H < 0 || Q < 0 || K < 1 || D < 1) return TRIATTN_ERR_INVALID_ARG;
    // With no query row there is nothing to read or write: arrays with no
    // elements may then be NULL (what an empty tensor hands over).
    const bool empty = B == 0 || N == 0 || H == 0 || Q == 0;
    if (!empty && (!q || !k || !v || !out)) return TRIATTN_ERR_INVALID_ARG;
    if (dtype != TRIATTN_F32 && dtype != TRIATTN_F16 && dtype != TRIATTN_BF16)
        return TRIATTN_ERR_INVALID_ARG;
    if (isinf(scale)) return TRIATTN_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
        return TRIATTN_ERR_INVALID_ARG;
    if (!aligned(bias, 4) || !aligned(lse, 4) || !aligned(mx, 4)) return TRIATTN_ERR_INVALID_ARG;

    if (mask) {
        switch (mask->kind) {
        case TRIATTN_MASK_NONE:
            break;
        case TRIATTN_MASK_DENSE:
            // a dense mask and kv_lengths are mutually exclusive
            if ((!mask->dense && !empty) || mask->kv_lengths) return TRIATTN_ERR_INVALID_ARG;
            break;
        case TRIATTN_MASK_KV_LENGTHS:
            if ((!mask->kv_lengths && !empty) || mask->dense) return TRIATTN_ERR_INVALID_ARG;
            break;
        case TRIATTN_MASK_BLOCK:
            if (!empty && (!mask->kv_num_blocks || !mask->kv_indices))
                return TRIATTN_ERR_INVALID_ARG;
            if (mask->dense || mask->kv_lengths) return TRIATTN_ERR_INVALID_ARG;
            if ((mask->full_kv_num_blocks == nullptr) != (mask->full_kv_indices == nullptr))
                return TRIATTN_ERR_INVALID_ARG;
            if (mask->q_block < 1 || mask->kv_block < 1 || mask->max_blocks < 1)
                return TRIATTN_ERR_INVALID_ARG;
            if (mask->full_kv_num_blocks && mask->full_max_blocks < 1)
                return TRIATTN_ERR_INVALID_ARG;
            if (mask->mask_mod != TRIATTN_MOD_NONE && mask->mask_mod != TRIATTN_MOD_CAUSAL)
                return TRIATTN_ERR_INVALID_ARG;
            if (mask->stride_b < 0 || mask->stride_n < 0 || mask->stride_h < 0)
                return TRIATTN_ERR_INVALID_ARG;
            if (!aligned(mask->kv_num_blocks, 4) || !aligned(mask->kv_indices, 4) ||
                !aligned(mask->full_kv_num_blocks, 4) || !aligned(mask->full_kv_indices, 4))
                return TRIATTN_ERR_INVALID_ARG;
            if ((K - 1) / mask->kv_block + 1 > triattn::kMaxKvBlocks)  // K >= 1
                return TRIATTN_ERR_UNSUPPORTED;
            break;
        default:
            return TRIATTN_ERR_INVALID_ARG;
        }
        if (mask->kind == TRIATTN_MASK_KV_LENGTHS && !aligned(mask->kv_lengths, 4))
            return TRIATTN_ERR_INVALID_ARG;
    }

    // Envelope of the triangle_attention page (Notes item 3).
    if (dtype == TRIATTN_F32) {
        if (D > 32 || D % 4 != 0) return TRIATTN_ERR_UNSUPPORTED;
    } else {
        if (D > 256 || D % 8 != 0) return TRIATTN_ERR_UNSUPPORTED;
    }

    // Index range: element counts must fit comfortably in int64, and the
    // row count in the launch grid.
    const int64_t rows = mul_or_neg(mul_or_neg(mul_or_neg(B, N), H), Q);
    const int64_t kv = mul_or_neg(mul_or_neg(mul_or_neg(B, N), H), K);
    const int64_t bias_elems = mul_or_neg(mul_or_neg(mul_or_neg(B, H), Q), K);
    if (rows < 0 || kv < 0 || bias_elems < 0) return TRIATTN_ERR_UNSUPPORTED;
    if (mul_or_neg(rows, D) < 0 || mul_or_neg(kv, D) < 0) return TRIATTN_ERR_UNSUPPORTED;
    if (rows > (int64_t(1) << 40) || kv > (int64_t(1) << 40)) return TRIATTN_ERR_UNSUPPORTED;
    if (mul_or_neg(mul_or_neg(B, N), K) < 0) return TRIATTN_ERR_UNSUPPORTED;
    return TRIATTN_OK;
}

Params make_params(const tri_attn_shape* s, const void* q, const void* k, const void* v,
                   const float* bias, const tri_attn_mask* mask, float scale, void* out,
                   float* lse, float* mx) {
    Params p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.bias = bias;
    p.out = out;
    p.lse = lse;
    p.mx = mx;
    p.B = s->B;
    p.N = s->N;
    p.H = s->H;
    p.Q = s->Q;
    p.K = s->K;
    p.D = s->D;
    // Default scale 1/sqrt(D), evaluated in double and rounded once.
    p.scale = isnan(scale) ? static_cast<float>(1.0 / sqrt(static_cast<double>(s->D))) : scale;
    p.mask_kind = mask ? mask->kind : TRIATTN_MASK_NONE;
    p.mask_mod = TRIATTN_MOD_NONE;
    p.q_block = p.kv_block = p.max_blocks = p.full_max_blocks = 1;
    p.n_q_rows = p.n_kv_blocks = 1;
    if (mask) {
        // only the arrays of the selected kind are forwarded to the kernels
        if (mask->kind == TRIATTN_MASK_DENSE) p.dense = mask->dense;
        if (mask->kind == TRIATTN_MASK_KV_LENGTHS) p.kv_lengths = mask->kv_lengths;
        if (mask->kind == TRIATTN_MASK_BLOCK) {
            p.mask_mod = mask->mask_mod;
            p.kv_num_blocks = mask->kv_num_blocks;
            p.kv_indices = mask->kv_indices;
            p.full_kv_num_blocks = mask->full_kv_num_blocks;
            p.full_kv_indices = mask->full_kv_indices;
            p.q_block = mask->q_block;
            p.kv_block = mask->kv_block;
            p.max_blocks = mask->max_blocks;
            p.full_max_blocks = mask->full_kv_num_blocks ? mask->full_max_blocks : 1;
            p.stride_b = mask->stride_b;
            p.stride_n = mask->stride_n;
            p.stride_h = mask->stride_h;
            // ceil(Q / q_block), ceil(K / kv_block) without overflow (any block size >= 1)
            p.n_q_rows = s->Q == 0 ? 0 : (s->Q - 1) / mask->q_block + 1;
            p.n_kv_blocks = (s->K - 1) / mask->kv_block + 1;
        }
    }
    return p;
}

// Validation of a packed variable-length call (see include/triattn.h).
triattn_status varlen_check_impl(const tri_attn_varlen* d, int32_t dtype, const void* q,
                                 const void* k, const void* v, float scale, const void* out,
                                 const float* lse, const float* mx) {
    if (!d) return TRIATTN_ERR_INVALID_ARG;
    if (d->batch < 0 || d->heads < 0 || d->head_dim < 1 || d->total_q < 0 || d->total_kv < 0 ||
        d->max_seqlen_q < 0 || d->max_seqlen_kv < 0)
        return TRIATTN_ERR_INVALID_ARG;
    if (d->layout != TRIATTN_QKV_SEPARATE && d->layout != TRIATTN_QKV_PACKED &&
        d->layout != TRIATTN_KV_PACKED)
        return TRIATTN_ERR_INVALID_ARG;
    if (d->mask_type != TRIATTN_VARLEN_NO_MASK && d->mask_type != TRIATTN_VARLEN_PADDING &&
        d->mask_type != TRIATTN_VARLEN_CAUSAL)
        return TRIATTN_ERR_INVALID_ARG;
    if (dtype != TRIATTN_F32 && dtype != TRIATTN_F16 && dtype != TRIATTN_BF16)
        return TRIATTN_ERR_INVALID_ARG;
    if (isinf(scale)) return TRIATTN_ERR_INVALID_ARG;
    const bool packed = d->layout == TRIATTN_QKV_PACKED;
    if (packed && (d->total_kv != d->total_q ||
                   (d->cu_seqlens_kv && d->cu_seqlens_kv != d->cu_seqlens_q)))
        return TRIATTN_ERR_INVALID_ARG;
    const bool empty =
        d->batch == 0 || d->heads == 0 || d->total_q == 0 || d->max_seqlen_q == 0;
    if (!empty) {
        if (!q || !out || !d->cu_seqlens_q) return TRIATTN_ERR_INVALID_ARG;
        if (d->layout != TRIATTN_QKV_PACKED && !k) return TRIATTN_ERR_INVALID_ARG;
        if (d->layout == TRIATTN_QKV_SEPARATE && !v) return TRIATTN_ERR_INVALID_ARG;
        if (!packed && !d->cu_seqlens_kv) return TRIATTN_ERR_INVALID_ARG;
    }
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(lse, 4) || !aligned(mx, 4) || !aligned(d->cu_seqlens_q, 4) ||
        !aligned(d->cu_seqlens_kv, 4))
        return TRIATTN_ERR_INVALID_ARG;
    const int64_t D = d->head_dim;
    if (dtype == TRIATTN_F32) {
        if (D > 32 || D % 4 != 0) return TRIATTN_ERR_UNSUPPORTED;
    } else {
        if (D > 256 || D % 8 != 0) return TRIATTN_ERR_UNSUPPORTED;
    }
    // element counts of the packed tensors (3 heads-slabs per row at most)
    const int64_t row = mul_or_neg(mul_or_neg(d->heads, D), 3);
    if (row < 0 || mul_or_neg(d->total_q, row) < 0 || mul_or_neg(d->total_kv, row) < 0)
        return TRIATTN_ERR_UNSUPPORTED;
    const int64_t rows = mul_or_neg(mul_or_neg(d->batch, d->heads), d->max_seqlen_q);
    if (rows < 0 || rows > (int64_t(1) << 40)) return TRIATTN_ERR_UNSUPPORTED;
    if (d->total_q > INT32_MAX || d->total_kv > INT32_MAX || d->batch > INT32_MAX - 1)
        return TRIATTN_ERR_UNSUPPORTED;  // cu_seqlens are int32
    return TRIATTN_OK;
}

}  // namespace

namespace triattn {

triattn_status bwd_validate(const tri_attn_shape* shape, int32_t dtype, const void* q,
                            const void* k, const void* v, const float* bias,
                            const tri_attn_mask* mask, float scale, const void* out,
                            const void* dout, const float* lse, const float* max, const void* dq,
                            const void* dk, const void* dv, const float* dbias,
                            const float* workspace, size_t workspace_bytes,
                            bool check_workspace) {
    // The forward's arguments (out is read, not written, here).
    triattn_status st = check_impl(shape, dtype, q, k, v, bias, mask, scale, out, lse, max);
    if (st != TRIATTN_OK) return st;
    const bool empty = shape->B == 0 || shape->N == 0 || shape->H == 0 || shape->Q == 0;
    if (!empty && (!dout || !lse || !max || !dq || !dk || !dv)) return TRIATTN_ERR_INVALID_ARG;
    if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
        !aligned(dbias, 4) || !aligned(workspace, 16))
        return TRIATTN_ERR_INVALID_ARG;
    if (!empty && check_workspace) {
        // the per-row data (more only speeds dBias up)
        const int64_t slices = mul_or_neg(mul_or_neg(shape->B, shape->N), shape->H);
        const int64_t need = slices < 0 ? -1 : triattn::bwd_rows_bytes(slices, shape->Q);
        if (need < 0) return TRIATTN_ERR_UNSUPPORTED;
        if (!workspace || workspace_bytes < static_cast<uint64_t>(need))
            return TRIATTN_ERR_INVALID_ARG;
    }
    return TRIATTN_OK;
}

}  // namespace triattn

extern "C" {

triattn_status tri_attn_check(const tri_attn_shape* shape, int32_t dtype, const void* q,
                              const void* k, const void* v, const float* bias,
                              const tri_attn_mask* mask, float scale, const void* out,
                              const float* lse, const float* max) {
    return check_impl(shape, dtype, q, k, v, bias, mask, scale, out, lse, max);
}

triattn_status tri_attn_fwd(const tri_attn_shape* shape, int32_t dtype, const void* q,
                            const void* k, const void* v, const float* bias,
                            const tri_attn_mask* mask, float scale, void* out, float* lse,
                            float* max, hipStream_t stream) {
    return tri_attn_fwd_bias_dtype(shape, dtype, q, k, v, bias, TRIATTN_F32, mask, scale, out,
                                   lse, max, stream);
}

triattn_status tri_attn_fwd_bias_dtype(const tri_attn_shape* shape, int32_t dtype, const void* q,
                                       const void* k, const void* v, const void* bias,
                                       int32_t bias_dtype, const tri_attn_mask* mask, float scale,
                                       void* out, float* lse, float* max, hipStream_t stream) {
    // fp32, or the 16-bit type of q, k and v
    const bool half_bias = bias_dtype != TRIATTN_F32;
    if (half_bias && (bias_dtype != dtype || (dtype != TRIATTN_F16 && dtype != TRIATTN_BF16)))
        return TRIATTN_ERR_INVALID_ARG;
    const triattn_status st =
        check_impl(shape, dtype, q, k, v, half_bias ? nullptr : static_cast<const float*>(bias),
                   mask, scale, out, lse, max);
    if (st != TRIATTN_OK) return st;
    if (half_bias && !aligned(bias, 2)) return TRIATTN_ERR_INVALID_ARG;
    if (shape->B == 0 || shape->N == 0 || shape->H == 0 || shape->Q == 0) return TRIATTN_OK;
    Params p = make_params(shape, q, k, v, half_bias ? nullptr : static_cast<const float*>(bias),
                           mask, scale, out, lse, max);
    if (half_bias) p.bias16 = bias;
    const hipError_t err = triattn::mfma_supports(p, dtype)
                               ? triattn::launch_mfma(p, dtype, stream)
                               : triattn::launch_generic(p, dtype, stream);
    return err == hipSuccess ? TRIATTN_OK : TRIATTN_ERR_HIP;
}

triattn_status tri_attn_varlen_check(const tri_attn_varlen* desc, int32_t dtype, const void* q,
                                     const void* k, const void* v, float scale, const void* out,
                                     const float* lse, const float* max) {
    return varlen_check_impl(desc, dtype, q, k, v, scale, out, lse, max);
}

triattn_status tri_attn_varlen_fwd(const tri_attn_varlen* d, int32_t dtype, const void* q,
                                   const void* k, const void* v, float scale, void* out,
                                   float* lse, float* max, hipStream_t stream) {
    const triattn_status st = varlen_check_impl(d, dtype, q, k, v, scale, out, lse, max);
    if (st != TRIATTN_OK) return st;
    if (d->batch == 0 || d->heads == 0 || d->total_q == 0 || d->max_seqlen_q == 0)
        return TRIATTN_OK;
    const int64_t H = d->heads, D = d->head_dim;
    const size_t esz = dtype == TRIATTN_F32 ? 4 : 2;
    Params p{};
    p.B = d->batch;
    p.N = 1;
    p.H = H;
    p.Q = d->max_seqlen_q;
    p.K = d->max_seqlen_kv;
    p.D = D;
    p.scale = isnan(scale) ? static_cast<float>(1.0 / sqrt(static_cast<double>(D))) : scale;
    p.mask_kind = triattn::kMaskVarlen;
    p.mask_mod = TRIATTN_MOD_NONE;
    p.q_block = p.kv_block = p.max_blocks = p.full_max_blocks = 1;
    p.n_q_rows = p.n_kv_blocks = 1;
    p.cu_q = d->cu_seqlens_q;
    p.cu_kv = d->layout == TRIATTN_QKV_PACKED ? d->cu_seqlens_q : d->cu_seqlens_kv;
    p.total_q = d->total_q;
    p.total_kv = d->layout == TRIATTN_QKV_PACKED ? d->total_q : d->total_kv;
    p.causal = d->mask_type == TRIATTN_VARLEN_CAUSAL;
    const char* qb = static_cast<const char*>(q);
    switch (d->layout) {
    case TRIATTN_QKV_SEPARATE:
        p.q = q;
        p.k = k;
        p.v = v;
        p.q_rs = p.kv_rs = H * D;
        break;
    case TRIATTN_QKV_PACKED:  // [T, 3, H, D]
        p.q = q;
        p.k = qb + H * D * esz;
        p.v = qb + 2 * H * D * esz;
        p.q_rs = p.kv_rs = 3 * H * D;
        break;
    default: {  // TRIATTN_KV_PACKED: q [Tq, H, D], kv [Tkv, 2, H, D]
        const char* kb = static_cast<const char*>(k);
        p.q = q;
        p.k = k;
        p.v = kb + H * D * esz;
        p.q_rs = H * D;
        p.kv_rs = 2 * H * D;
    }
    }
    p.out = out;
    p.lse = lse;
    p.mx = max;
    const hipError_t err = triattn::mfma_supports(p, dtype) ? triattn::launch_mfma(p, dtype, stream)
                                                            : triattn::launch_generic(p, dtype, stream);
    return err == hipSuccess ? TRIATTN_OK : TRIATTN_ERR_HIP;
}

triattn_status tri_attn_bwd(const tri_attn_shape* shape, int32_t dtype, const void* q,
                            const void* k, const void* v, const float* bias,
                            const tri_attn_mask* mask, float scale, const void* out,
                            const void* dout, const float* lse, const float* max, void* dq,
                            void* dk, void* dv, float* dbias, float* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    const triattn_status st =
        triattn::bwd_validate(shape, dtype, q, k, v, bias, mask, scale, out, dout, lse, max, dq,
                              dk, dv, dbias, workspace, workspace_bytes);
    if (st != TRIATTN_OK) return st;
    if (shape->B == 0 || shape->N == 0 || shape->H == 0 || shape->Q == 0) return TRIATTN_OK;
    const Params p = make_params(shape, q, k, v, bias, mask, scale, nullptr, nullptr, nullptr);
    triattn::BwdParams g{};
    g.out = out;
    g.dout = dout;
    g.lse = lse;
    g.mx = max;
    g.dq = dq;
    g.dk = dk;
    g.dv = dv;
    g.dbias = dbias;
    const hipError_t err = triattn::launch_bwd(p, g, dtype, workspace, workspace_bytes, stream);
    return err == hipSuccess ? TRIATTN_OK : TRIATTN_ERR_HIP;
}

size_t tri_attn_bwd_workspace_size(const tri_attn_shape* shape, int32_t with_dbias) {
    if (!shape || shape->B < 0 || shape->N < 0 || shape->H < 0 || shape->Q < 0 || shape->K < 0)
        return 0;
    const int64_t slices = mul_or_neg(mul_or_neg(shape->B, shape->N), shape->H);
    int64_t need = slices < 0 ? -1 : triattn::bwd_rows_bytes(slices, shape->Q);
    if (need < 0) return 0;
    if (with_dbias) {
        const int s = triattn::dbias_splits(shape->B, shape->N, shape->H, shape->Q, shape->K,
                                            shape->D);
        if (s > 1) {
            const int64_t planes = mul_or_neg(
                mul_or_neg(mul_or_neg(mul_or_neg(shape->B, shape->H), shape->Q), shape->K),
                4 * s);
            if (planes < 0 || need > INT64_MAX - planes) return 0;
            need += planes;
        }
    }
    return static_cast<size_t>(need);
}

triattn_status tri_attn_mask_to_kv_lengths(const uint8_t* mask, int64_t rows, int64_t K,
                                           int32_t* kv_lengths, int32_t* nonprefix_rows,
                                           hipStream_t stream) {
    if (rows < 0 || K < 1 || !nonprefix_rows) return TRIATTN_ERR_INVALID_ARG;
    if (rows > 0 && (!mask || !kv_lengths)) return TRIATTN_ERR_INVALID_ARG;
    if (!aligned(kv_lengths, 4) || !aligned(nonprefix_rows, 4)) return TRIATTN_ERR_INVALID_ARG;
    if (K > INT32_MAX || rows > (int64_t(1) << 40) || mul_or_neg(rows, K) < 0)
        return TRIATTN_ERR_UNSUPPORTED;
    const hipError_t err =
        triattn::launch_mask_to_kv_lengths(mask, rows, K, kv_lengths, nonprefix_rows, stream);
    return err == hipSuccess ? TRIATTN_OK : TRIATTN_ERR_HIP;
}

const char* tri_attn_status_str(triattn_status status) {
    switch (status) {
    case TRIATTN_OK:
        return "TRIATTN_OK";
    case TRIATTN_ERR_INVALID_ARG:
        return "TRIATTN_ERR_INVALID_ARG: invalid argument";
    case TRIATTN_ERR_UNSUPPORTED:
        return "TRIATTN_ERR_UNSUPPORTED: dtype, head dimension or size outside the supported "
               "envelope";
    case TRIATTN_ERR_HIP:
        return "TRIATTN_ERR_HIP: a HIP launch failed";
    }
    return "unknown triattn_status";
}

}  // extern "C"
