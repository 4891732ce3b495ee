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
 * tri_attn_fwd with the bias in a chosen element type.  The
 * triangle_attention page's Parameters ("bias") say that its newest kernels
 * cast the bias to the q/k/v dtype (bf16/fp16) for best performance; this
 * entry point takes such a bias as it is, instead of requiring fp32.
 *
 * `bias_dtype`: TRIATTN_F32 (then `bias` is (B,1,H,Q,K) fp32 and the call
 * is exactly tri_attn_fwd) or equal to `dtype` when that is TRIATTN_F16 or
 * TRIATTN_BF16 (then `bias` is (B,1,H,Q,K) of that type, 2-byte aligned;
 * K % 8 == 0 and 16-byte alignment keep it on the MFMA kernel).  Each bias
 * value is widened exactly to fp32 and the computation is the one of
 * tri_attn_fwd with that fp32 bias: the only difference from passing the
 * fp32 original is the bias's own rounding to 16 bits (on the order of 1e-3
 * in lse for a unit-variance bias, past the 1e-3 lse tolerance kept for fp32
 * biases).  The backward (tri_attn_bwd) takes the same values as fp32.
 * Other arguments, results and errors as tri_attn_fwd, plus
 * TRIATTN_ERR_INVALID_ARG for any other bias_dtype or a misaligned bias.
 */
triattn_status tri_attn_fwd_bias_dtype(const tri_attn_shape* shape, int32_t dtype, const void* q,
                                       const void* k, const void* v, const void* bias,
                                       int32_t bias_dtype, const tri_attn_mask* mask, float scale,
                                       void* out, float* lse, float* max, hipStream_t stream);

/*
 * ---- Packed variable-length sequences ------------------------------------
 *
 * The fused-attention layouts of Transformer Engine's fused_attn.h (release
 * 0.9.0 C API: enums NVTE_QKV_Layout and NVTE_Mask_Type, and the
 * cu_seqlens_q / cu_seqlens_kv / max_seqlen_q / max_seqlen_kv arguments of
 * nvte_fused_attn_fwd_kvpacked and _qkvpacked).  `batch` sequences are
 * packed one after the other along the row axis of each tensor; every row
 * holds all H heads.  Sequence b is rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 * of q and out and rows cu_seqlens_kv[b] .. cu_seqlens_kv[b+1]-1 of k and v,
 * and each query row attends only to the keys of its own sequence:
 *
 *     z_j = s * (Q_i . K_j)   for the keys j of i's sequence the mask allows
 *     O_i = sum_j softmax_j(z) V_j,  max_i = max_j z_j,  lse_i = log sum_j exp(z_j)
 *
 * (no bias: the page leaves the bias layout of packed sequences open).
 */

/* Layout of the packed tensors (NVTE_QKV_Layout; the page's three layouts
 * read as separate q, k, v; one interleaved qkv tensor; q with an
 * interleaved kv tensor). */
typedef enum tri_attn_qkv_layout {
    /* q [total_q, H, D]; k and v [total_kv, H, D] */
    TRIATTN_QKV_SEPARATE = 0,
    /* one tensor qkv [total, 3, H, D] passed as `q` (k and v unused; the
     * key rows are the query rows: total_kv = total_q, cu_seqlens_kv NULL
     * or equal to cu_seqlens_q) */
    TRIATTN_QKV_PACKED = 1,
    /* q [total_q, H, D]; one tensor kv [total_kv, 2, H, D] passed as `k`
     * (v unused) */
    TRIATTN_KV_PACKED = 2
} tri_attn_qkv_layout;

/* Key mask inside a sequence (NVTE_Mask_Type). */
typedef enum tri_attn_varlen_mask {
    /* every key of the query's sequence */
    TRIATTN_VARLEN_NO_MASK = 0,
    /* the same: packed sequences carry no padding rows, the padding is the
     * sequence boundary itself */
    TRIATTN_VARLEN_PADDING = 1,
    /* key j of query row i of a sequence (both counted from the sequence's
     * first row) only if j <= i, top-left aligned when the query and key
     * lengths differ */
    TRIATTN_VARLEN_CAUSAL = 2
} tri_attn_varlen_mask;

typedef struct tri_attn_varlen {
    int32_t layout;     /* tri_attn_qkv_layout */
    int32_t mask_type;  /* tri_attn_varlen_mask */
    int64_t batch;      /* number of sequences (>= 0) */
    int64_t heads;      /* H (>= 0) */
    int64_t head_dim;   /* D (>= 1) */
    int64_t total_q;    /* rows of q and out (>= 0) */
    int64_t total_kv;   /* rows of k and v (>= 0; QKV_PACKED: total_q) */
    /* batch + 1 ascending int32 row offsets each, device memory */
    const int32_t* cu_seqlens_q;
    const int32_t* cu_seqlens_kv;
    /* bounds on the sequence lengths (the page: "may be >=" the longest) */
    int64_t max_seqlen_q;
    int64_t max_seqlen_kv;
} tri_attn_varlen;

/*
 * Host-only validation of tri_attn_varlen_fwd's arguments (no device call).
 * Layouts and outputs: out [total_q, H, D] of type `dtype`; lse, max
 * [total_q, H] fp32, each nullable.  dtype and D follow the envelope of
 * tri_attn_fwd; q, k, v, out 16-byte aligned.  `scale`: NaN = 1/sqrt(D).
 * Nothing to do (OK, pointers may be NULL) when batch, heads, total_q or
 * max_seqlen_q is 0.  TRIATTN_ERR_INVALID_ARG for: a NULL descriptor; a
 * negative size, D < 1 or max_seqlen_kv < 0; an unknown layout, mask type or
 * dtype; a NULL required pointer (q; k for SEPARATE and KV_PACKED; v for
 * SEPARATE; out; cu_seqlens_q; cu_seqlens_kv unless QKV_PACKED); QKV_PACKED
 * with total_kv != total_q or a cu_seqlens_kv other than NULL or
 * cu_seqlens_q; a misaligned pointer; an infinite scale.
 * TRIATTN_ERR_UNSUPPORTED for (dtype, D) outside the envelope or sizes past
 * the library's index range.
 */
triattn_status tri_attn_varlen_check(const tri_attn_varlen* desc, int32_t dtype, const void* q,
                                     const void* k, const void* v, float scale, const void* out,
                                     const float* lse, const float* max);

/*
 * Enqueue the forward of packed sequences on `stream`: out, lse and max of
 * every row of every sequence; rows of the packed tensors outside every
 * sequence are not written.  The cu_seqlens values are device data and are
 * not validated on the host: each sequence's bounds are clamped to
 * [0, total] and made ascending, and a sequence longer than max_seqlen_q
 * (max_seqlen_kv) is computed over its first max_seqlen_q query rows (key
 * rows) only.  A query row with no key (an empty key sequence) gets O = 0,
 * max = lse = -1e9.  Returns the tri_attn_varlen_check status if not OK
 * (nothing launched), TRIATTN_ERR_HIP if a launch fails, else TRIATTN_OK.
 */
triattn_status tri_attn_varlen_fwd(const tri_attn_varlen* desc, int32_t dtype, const void* q,
                                   const void* k, const void* v, float scale, void* out,
                                   float* lse, float* max, hipStream_t stream);

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
 * Workspace (required when there is a query row): device memory of at least
 * tri_attn_bwd_workspace_size(shape, 0) bytes (260 per (b, n, h) slice and
 * 32-row tile, rounded up to 16), 16-byte aligned, caller-owned, whose
 * contents on entry do not matter and on return are unspecified.  The first
 * pass stores per-row data there (Delta = dO.O and lse of every row, and how
 * many rows of each 32-row tile have no valid key) for the passes that
 * follow.  With
 * dbias, more workspace lets the dBias pass split its sum over n into
 * ranges summed by separate workgroups and then added in range order
 * (deterministic for a given workspace size; the split changes only the
 * fp32 rounding order of dbias, never dq, dk or dv);
 * tri_attn_bwd_workspace_size gives the size that allows the library's
 * preferred split.  Calls that share one workspace must not overlap.
 *
 * Errors: those of tri_attn_check for the forward's arguments, and
 * TRIATTN_ERR_INVALID_ARG for a NULL dout / lse / max / dq / dk / dv /
 * workspace when there is a query row, a misaligned pointer, or a workspace
 * smaller than the size above (TRIATTN_ERR_UNSUPPORTED if that size
 * overflows int64);
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
 * Bytes of workspace tri_attn_bwd uses at most for `shape`: the per-row data
 * (260 bytes per (b, n, h) slice and 32-row tile, rounded up to 16; the
 * minimum tri_attn_bwd accepts), plus, when with_dbias is nonzero, the
 * planes of partial sums of the preferred dBias split (a whole number of
 * B*H*Q*K fp32 planes).  0 for a NULL shape, a negative size or a size past
 * int64.  Host only.
 */
size_t tri_attn_bwd_workspace_size(const tri_attn_shape* shape, int32_t with_dbias);

/*
 * tri_attn_bwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without the workspace, and the same results, bit for
 * bit, as tri_attn_bwd given a workspace of TRIATTN_BWD_NOALLOC_BYTES bytes.
 * That workspace is a fixed array of this library (48 MiB) per GPU that
 * loads it, held until the process ends; the call allocates and frees
 * nothing.  It needs tri_attn_bwd_workspace_size(shape, 0) <=
 * TRIATTN_BWD_NOALLOC_BYTES (about 6 Mi rows when Q is a multiple of 32)
 * and returns TRIATTN_ERR_UNSUPPORTED (nothing launched) for larger
 * problems.  All calls on one GPU share the array: calls that overlap in
 * time on one GPU race and must not be issued.  The calling thread's
 * current device must be the stream's.  Errors otherwise as tri_attn_bwd
 * (TRIATTN_ERR_HIP also if the array's address cannot be obtained).
 */
#define TRIATTN_BWD_NOALLOC_BYTES (48 * 1024 * 1024)
triattn_status tri_attn_bwd_noalloc(const tri_attn_shape* shape, int32_t dtype, const void* q,
                                    const void* k, const void* v, const float* bias,
                                    const tri_attn_mask* mask, float scale, const void* out,
                                    const void* dout, const float* lse, const float* max,
                                    void* dq, void* dk, void* dv, float* dbias,
                                    hipStream_t stream);

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
