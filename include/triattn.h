/*
 * triattn.h -- C ABI of libtriattn, the gfx950 (MI355X) forward pass of
 * masked, biased triangle attention.
 *
 * Operation (cuEquivariance "cuequivariance_torch.triangle_attention" API
 * page, the defining equation): for every batch b, token n, head h and query
 * row q,
 *
 *     z_k = s * (Q_q . K_k) + B_qk      if key k is valid
 *     z_k = -1e9                        otherwise
 *     O_q = sum_k softmax_k(z) V_k
 *
 * with the auxiliary outputs max_q = max_k z_k and lse_q = log sum_k exp(z_k)
 * (natural log, same units as z; the page returns both as fp32 "lse" and
 * "max").  The scale multiplies Q.K only; the bias is added after it
 * (Transformer Engine fused_attn.h, NVTE_Bias_Type NVTE_POST_SCALE_BIAS).
 * A row with no valid key therefore gets uniform weights over all K keys:
 * O = mean of V, max = -1e9, lse = -1e9 + ln K rounded to fp32 (= -1e9).
 *
 * Memory layout (all contiguous, row-major, caller-owned device memory):
 *   q, out   (B, N, H, Q, D)  element type `dtype`
 *   k, v     (B, N, H, K, D)  element type `dtype`
 *   bias     (B, 1, H, Q, K)  fp32, shared by every n; NULL means no bias
 *   lse, max (B, N, H, Q)     fp32; each may be NULL (not written)
 * q, k, v and out must be 16-byte aligned; bias, lse and max 4-byte aligned.
 *
 * Supported envelope (the triangle_attention page, Notes item 3: its
 * standard kernels' fp32 bound, and for the half types the wider forward
 * bound it gives its newest kernels):
 *   TRIATTN_F32:            D <= 32 and D % 4 == 0
 *   TRIATTN_F16 / BF16:     D <= 256 and D % 8 == 0
 * Anything else returns TRIATTN_ERR_UNSUPPORTED; the library has no slower
 * fallback implementation.
 *
 * Ownership and threading: the library never allocates, frees or
 * synchronises, and keeps no mutable global state; calls are reentrant.
 * tri_attn_fwd only enqueues kernels on `stream` and returns; the outputs
 * are ready when the stream reaches that point.  Pointers must stay valid
 * until then.
 *
 * Errors: every entry point returns a triattn_status.  On
 * TRIATTN_ERR_INVALID_ARG or TRIATTN_ERR_UNSUPPORTED nothing is launched and
 * nothing is written.  TRIATTN_ERR_HIP means a launch failed (the HIP error
 * state is left for the caller to query).  Values stored in device memory
 * (kv_lengths, block counts and ids) are not validated on the host: they are
 * clamped or ignored as documented below.
 */
#ifndef TRIATTN_H
#define TRIATTN_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum triattn_status {
    TRIATTN_OK = 0,
    TRIATTN_ERR_INVALID_ARG = 1,
    TRIATTN_ERR_UNSUPPORTED = 2,
    TRIATTN_ERR_HIP = 3
} triattn_status;

/* Element type of q, k, v and out (all four share one type; the page picks
 * kernel precision from the input dtypes, Notes item 2). */
typedef enum tri_attn_dtype {
    TRIATTN_F32 = 0,
    TRIATTN_F16 = 1,
    TRIATTN_BF16 = 2
} tri_attn_dtype;

/* Sizes, in the page's notation: batch B, tokens N, heads H, query tokens Q,
 * key tokens K, attention dimension D.  B, N, H, Q may be 0 (nothing to do);
 * K and D must be at least 1. */
typedef struct tri_attn_shape {
    int64_t B, N, H, Q, K, D;
} tri_attn_shape;

typedef enum tri_attn_mask_kind {
    /* every key valid (Transformer Engine NVTE_NO_MASK) */
    TRIATTN_MASK_NONE = 0,
    /* dense key mask, the page's "mask" of shape (B,N,1,1,K) cast to bool:
     * `dense` points at B*N*K bytes, nonzero = valid.  Any pattern. */
    TRIATTN_MASK_DENSE = 1,
    /* right-padded prefix, the page's "kv_lengths" (B,N,1,1,1) int32:
     * `kv_lengths` points at B*N int32; keys j < clamp(len, 0, K) are
     * valid (values above K clamp to K as the page states; values below 0
     * are read as 0, i.e. no valid key). */
    TRIATTN_MASK_KV_LENGTHS = 2,
    /* block-sparse lists in the BlockMask format (tensorplay.nn.attention
     * page, Basics and Details items 1-2), see tri_attn_mask below. */
    TRIATTN_MASK_BLOCK = 3
} tri_attn_mask_kind;

/* Element predicate applied inside listed blocks that are not full blocks
 * (the BlockMask's mask_mod, restricted to what a C ABI can carry). */
typedef enum tri_attn_mask_mod {
    TRIATTN_MOD_NONE = 0,   /* every element of a listed block is valid */
    TRIATTN_MOD_CAUSAL = 1  /* valid iff q_idx >= kv_idx (top-left aligned) */
} tri_attn_mask_mod;

/*
 * Key-mask descriptor.  Only the fields of the selected kind are read.
 *
 * Block kind: query rows are grouped in blocks of q_block rows
 * (ROWS = ceil(Q / q_block)) and keys in blocks of kv_block keys.  For list
 * instance i and block row r:
 *   kv_num_blocks[i*ROWS + r]                      count, clamped to [0, max_blocks]
 *   kv_indices[(i*ROWS + r)*max_blocks + j]        j < count: a listed kv block id
 *   full_kv_num_blocks / full_kv_indices           the same for "full" blocks, with
 *                                                  width full_max_blocks; both NULL
 *                                                  or both non-NULL
 * The instance of (b, n, h) is i = b*stride_b + n*stride_n + h*stride_h (a
 * stride of 0 broadcasts the lists over that axis).  Visited blocks are the
 * union of both lists; ids outside [0, ceil(K/kv_block)) are ignored and
 * duplicates count once; entries past a count are never read.  A key in a
 * visited block is valid if the block is listed as full, else if mask_mod
 * holds.  All int32 arrays are device memory.
 */
typedef struct tri_attn_mask {
    int32_t kind;      /* tri_attn_mask_kind */
    int32_t mask_mod;  /* tri_attn_mask_mod (block kind only) */
    const uint8_t* dense;
    const int32_t* kv_lengths;
    const int32_t* kv_num_blocks;
    const int32_t* kv_indices;
    const int32_t* full_kv_num_blocks;
    const int32_t* full_kv_indices;
    int64_t q_block;
    int64_t kv_block;
    int64_t max_blocks;
    int64_t full_max_blocks;
    int64_t stride_b;
    int64_t stride_n;
    int64_t stride_h;
} tri_attn_mask;

/*
 * Validate the arguments of tri_attn_fwd without touching the device.
 * Pure host function: reads only `shape` and `mask` (the descriptor, not the
 * device arrays it points at) and the pointer values.
 *
 * `scale`: s in the equation; NaN selects the page's default 1/sqrt(D)
 * (computed in double, then rounded to float).  `mask` NULL means no mask.
 *
 * When B, N, H or Q is 0 there is no query row: the call does nothing and
 * returns TRIATTN_OK, and q, k, v, out and the mask's arrays may be NULL (an
 * empty tensor's address); every other rule below still applies.
 *
 * Returns TRIATTN_ERR_INVALID_ARG for: a NULL shape; a NULL q / k / v / out
 * when there is a query row; a negative size, K < 1 or D < 1; an unknown
 * dtype or mask kind; a misaligned pointer; a mask kind whose required
 * arrays are NULL when there is a query row; only one of the
 * full_kv pair (the BlockMask constructor rejects that too); q_block,
 * kv_block or max_blocks below 1; an unknown mask_mod; a negative stride;
 * an infinite scale.  TRIATTN_ERR_UNSUPPORTED for (dtype, D) outside the
 * envelope above or sizes beyond the library's index range.
 */
triattn_status tri_attn_check(const tri_attn_shape* shape, int32_t dtype, const void* q,
                              const void* k, const void* v, const float* bias,
                              const tri_attn_mask* mask, float scale, const void* out,
                              const float* lse, const float* max);

/*
 * Enqueue the forward pass on `stream` (0 = the null stream).
 * Arguments as for tri_attn_check; out, lse and max are written.
 * Returns the tri_attn_check status if it is not TRIATTN_OK (nothing is
 * launched), TRIATTN_ERR_HIP if a launch fails, else TRIATTN_OK.
 */
triattn_status tri_attn_fwd(const tri_attn_shape* shape, int32_t dtype, const void* q,
                            const void* k, const void* v, const float* bias,
                            const tri_attn_mask* mask, float scale, void* out, float* lse,
                            float* max, hipStream_t stream);

/*
 * Backward of the forward's output O (the page's backward pass; lse and max
 * carry no incoming gradient).  Per (b,n,h,q) row, with P the forward's
 * softmax weights rebuilt from lse (P_k = exp(z_k - lse)) and Delta = dO.O:
 *   dV_k += P_k dO;   dz_k = P_k (dO.V_k - Delta);
 *   for valid keys only: dQ += s dz_k K_k, dK_k += s dz_k Q, dbias_qk += dz_k,
 * dbias summed over n (the bias is shared by every n).  A row whose forward
 * max is the -1e9 replacement had no valid key: its weights are 1/K and it
 * adds dO/K to every dV_k and nothing else.
 *
 * Inputs: q, k, v, bias, mask, scale exactly as given to tri_attn_fwd; out,
 * lse and max as tri_attn_fwd wrote them for those inputs (all three
 * required here); dout (B,N,H,Q,D) of type `dtype`, 16-byte aligned.
 * Outputs (written in full, caller-owned): dq (B,N,H,Q,D), dk and dv
 * (B,N,H,K,D), all of type `dtype` and 16-byte aligned; dbias (B,1,H,Q,K)
 * fp32, or NULL to skip it.  All device memory; enqueued on `stream`.
 *
 * Workspace (used only when dbias is not NULL): NULL, or device memory of
 * at least 4*B*N*H*Q*K bytes, 16-byte aligned, caller-owned, whose contents
 * on entry do not matter and on return are unspecified.  With it, the dQ
 * pass stores every dz and dbias is their sum over n, read back at HBM
 * bandwidth; without it, dbias is recomputed per block by a latency-bound
 * walk over n (no extra memory).  Both routes add the same values in the
 * same order (n ascending) and give the same bits.  Calls that share one
 * workspace must not overlap.
 *
 * Errors: those of tri_attn_check for the forward's arguments, and
 * TRIATTN_ERR_INVALID_ARG for a NULL dout / lse / max / dq / dk / dv when
 * there is a query row, a misaligned pointer, or a workspace smaller than
 * the size above (TRIATTN_ERR_UNSUPPORTED if that size overflows int64);
 * nothing is launched then.  TRIATTN_ERR_HIP if a launch fails.  With no
 * query row the call does nothing.  Products of bf16/fp16 tiles run on
 * MFMA with fp32 accumulation, fp32 inputs on fp32 FMAs.
 */
triattn_status tri_attn_bwd(const tri_attn_shape* shape, int32_t dtype, const void* q,
                            const void* k, const void* v, const float* bias,
                            const tri_attn_mask* mask, float scale, const void* out,
                            const void* dout, const float* lse, const float* max, void* dq,
                            void* dk, void* dv, float* dbias, float* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * Count the valid prefix of each dense key-mask row: the page's
 * mask_to_kv_lengths helper, which turns a right-padded (B,N,1,1,K) bool mask
 * into (B,N,1,1,1) int32 lengths.  `mask`: rows*K bytes (nonzero = valid);
 * `kv_lengths`: rows int32, each the number of leading valid keys;
 * `nonprefix_rows`: one int32 that receives the number of rows whose valid
 * keys are not a prefix (a masked key followed by a valid one); the call
 * resets it on the stream before counting.  A nonzero count means the mask
 * is not right-padded and the lengths must not be used.  rows may be 0; K
 * must be at least 1.  All three arrays are device memory.
 */
triattn_status tri_attn_mask_to_kv_lengths(const uint8_t* mask, int64_t rows, int64_t K,
                                           int32_t* kv_lengths, int32_t* nonprefix_rows,
                                           hipStream_t stream);

/* Static, human-readable name of a status code (never NULL). */
const char* tri_attn_status_str(triattn_status status);

#ifdef __cplusplus
}
#endif

#endif /* TRIATTN_H */
