/*
 * triattn_oracle.c -- plain fp64 CPU oracle for the masked, biased triangle
 * attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker the GPU library is
 * measured against; it is never part of the product path.  Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header, table or helper with the HIP library.
 *
 * What it computes (cuEquivariance "cuequivariance_torch.triangle_attention"
 * API page, the defining equation): for every query row q of every (b,n,h),
 *
 *     z_k = s * (Q_q . K_k) + B_qk      if key k is valid (M_k = 1)
 *     z_k = -1e9                        otherwise
 *     O_q = sum_k softmax_k(z) V_k
 *
 * The equation has no approximation, so the oracle is that definition
 * written out in fp64, one row at a time, with no blocking, no streaming
 * softmax and no reordering:
 *     m   = max_k z_k                    (the "max" auxiliary output)
 *     l   = sum_k exp(z_k - m)
 *     O_d = sum_k exp(z_k - m) V_kd / l
 *     lse = m + log(l)                   (the "lse" auxiliary output)
 * Subtracting m is the textbook way to evaluate softmax without overflow; it
 * changes nothing mathematically.  lse and max are in natural-log units of z.
 *
 * Inputs (all row-major, fp64; the caller upcasts storage dtypes exactly):
 *   q    (B,N,H,Q,D)      k, v (B,N,H,K,D)
 *   bias (B,1,H,Q,K) or NULL (no bias == zero bias; Transformer Engine
 *        fused_attn.h, NVTE_Bias_Type NVTE_NO_BIAS).  The bias is added after
 *        the scale (same page, NVTE_POST_SCALE_BIAS; the triangle_attention
 *        equation multiplies only Q.K by s).
 *   scale: NaN selects the default s = 1/sqrt(D) (triangle_attention page,
 *        "scale" parameter).
 *
 * Key-validity predicate M (one of):
 *   NONE        every key is valid.
 *   DENSE       mask (B,N,K) bytes, nonzero = valid; the page's mask has
 *               shape (B,N,1,1,K), is cast to bool and broadcasts over H, Q.
 *   KV_LENGTHS  len (B,N) int32; keys j < clamp(len,0,K) are valid
 *               (triangle_attention page, "kv_lengths": values above K clamp
 *               to K; values below 0 are read as 0, i.e. no valid key).
 *   BLOCK       block-sparse lists in the BlockMask format of the
 *               "tensorplay.nn.attention" page (Basics; Details items 1-2):
 *               for query row q, r = q / q_block is its row of blocks; the
 *               listed kv blocks are kv_indices[r][0:kv_num_blocks[r]] united
 *               with full_kv_indices[r][0:full_kv_num_blocks[r]]; entries past
 *               the count are never read (the page calls them undefined);
 *               indices outside [0, ceil(K/kv_block)) are ignored and
 *               duplicates are idempotent (the page's to-dense loop assigns 1).
 *               A key in a listed block is valid if its block is a full
 *               block, or else if mask_mod(q, k) holds (mask_mod NONE: true;
 *               CAUSAL: q >= k).  Counts are clamped to [0, max_blocks].
 *               The (b,n,h) instance i = b*stride_b + n*stride_n + h*stride_h
 *               selects the lists (stride 0 broadcasts).
 *
 * Rows: rows == NULL computes every (b,n,h,q) row in order; otherwise the
 * n_rows flat indices ((b*N+n)*H+h)*Q+q are computed, in the given order.
 * Outputs: out (n_rows, D), lse (n_rows), mx (n_rows), all fp64.
 *
 * Returns 0 on success, a negative value on a bad argument or allocation
 * failure.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_MASK_NONE 0
#define ORACLE_MASK_DENSE 1
#define ORACLE_MASK_KV_LENGTHS 2
#define ORACLE_MASK_BLOCK 3

#define ORACLE_MOD_NONE 0
#define ORACLE_MOD_CAUSAL 1

/* The replacement logit of a masked key, from the defining equation. */
#define MASKED_LOGIT (-1.0e9)

typedef struct {
    int64_t B, N, H, Q, K, D;
    const double *q, *k, *v, *bias;
    int mask_kind;
    const uint8_t *dense;
    const int32_t *kv_lengths;
    const int32_t *kv_num_blocks, *kv_indices;
    const int32_t *full_kv_num_blocks, *full_kv_indices;
    int64_t q_block, kv_block, max_blocks, full_max_blocks;
    int mask_mod;
    int64_t stride_b, stride_n, stride_h;
    double scale;
    int64_t n_rows;
    const int64_t *rows;
    double *out, *lse, *mx;
} oracle_args;

typedef struct {
    const oracle_args *a;
    int64_t first, last; /* [first, last) positions in the row list */
    int status;
} oracle_job;

/* Mark the listed blocks of one BlockMask row: listed[j] = 1 for every kv
 * block j that appears in the row's first `count` entries. */
static void mark_blocks(const int32_t *counts, const int32_t *indices, int64_t list_row,
                        int64_t width, int64_t n_kv_blocks, unsigned char *listed)
{
    int64_t count = counts[list_row];
    if (count < 0) count = 0;
    if (count > width) count = width;
    const int32_t *idx = indices + list_row * width;
    for (int64_t j = 0; j < count; ++j) {
        int64_t blk = idx[j];
        if (blk >= 0 && blk < n_kv_blocks) listed[blk] = 1;
    }
}

static void compute_row(const oracle_args *a, int64_t pos, double *z,
                        unsigned char *listed, unsigned char *full)
{
    const int64_t Q = a->Q, K = a->K, D = a->D, H = a->H, N = a->N;
    const int64_t row = a->rows ? a->rows[pos] : pos;
    const int64_t qi = row % Q;
    const int64_t h = (row / Q) % H;
    const int64_t n = (row / (Q * H)) % N;
    const int64_t b = row / (Q * H * N);

    const double *qrow = a->q + row * D;
    const int64_t bnh = (b * N + n) * H + h;
    const double *kbase = a->k + bnh * K * D;
    const double *vbase = a->v + bnh * K * D;
    /* bias is (B,1,H,Q,K): the same bias for every n. */
    const double *brow = a->bias ? a->bias + ((b * H + h) * Q + qi) * K : NULL;

    int64_t valid_len = K;
    if (a->mask_kind == ORACLE_MASK_KV_LENGTHS) {
        int64_t len = a->kv_lengths[b * N + n];
        valid_len = len < 0 ? 0 : (len > K ? K : len);
    }
    int64_t n_kv_blocks = 0;
    if (a->mask_kind == ORACLE_MASK_BLOCK) {
        n_kv_blocks = (K + a->kv_block - 1) / a->kv_block;
        const int64_t n_q_rows = (Q + a->q_block - 1) / a->q_block;
        const int64_t inst = b * a->stride_b + n * a->stride_n + h * a->stride_h;
        const int64_t list_row = inst * n_q_rows + qi / a->q_block;
        memset(listed, 0, (size_t)n_kv_blocks);
        memset(full, 0, (size_t)n_kv_blocks);
        mark_blocks(a->kv_num_blocks, a->kv_indices, list_row, a->max_blocks, n_kv_blocks,
                    listed);
        if (a->full_kv_num_blocks) {
            mark_blocks(a->full_kv_num_blocks, a->full_kv_indices, list_row,
                        a->full_max_blocks, n_kv_blocks, full);
            for (int64_t j = 0; j < n_kv_blocks; ++j)
                if (full[j]) listed[j] = 1; /* full blocks are visited too */
        }
    }

    /* Logits, with the masked-key replacement. */
    for (int64_t kk = 0; kk < K; ++kk) {
        int valid = 1;
        switch (a->mask_kind) {
        case ORACLE_MASK_DENSE:
            valid = a->dense[(b * N + n) * K + kk] != 0;
            break;
        case ORACLE_MASK_KV_LENGTHS:
            valid = kk < valid_len;
            break;
        case ORACLE_MASK_BLOCK: {
            const int64_t blk = kk / a->kv_block;
            if (!listed[blk]) {
                valid = 0;
            } else if (!full[blk]) {
                valid = (a->mask_mod == ORACLE_MOD_CAUSAL) ? (qi >= kk) : 1;
            }
            break;
        }
        default:
            break;
        }
        if (valid) {
            const double *krow = kbase + kk * D;
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d) dot += qrow[d] * krow[d];
            z[kk] = a->scale * dot + (brow ? brow[kk] : 0.0);
        } else {
            z[kk] = MASKED_LOGIT;
        }
    }

    /* softmax_k(z) V, evaluated with the row maximum subtracted. */
    double m = z[0];
    for (int64_t kk = 1; kk < K; ++kk)
        if (z[kk] > m) m = z[kk];
    double l = 0.0;
    for (int64_t kk = 0; kk < K; ++kk) {
        z[kk] = exp(z[kk] - m); /* z now holds the unnormalised weights */
        l += z[kk];
    }
    double *orow = a->out + pos * D;
    for (int64_t d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int64_t kk = 0; kk < K; ++kk) acc += z[kk] * vbase[kk * D + d];
        orow[d] = acc / l;
    }
    a->lse[pos] = m + log(l);
    a->mx[pos] = m;
}

static void *run_job(void *arg)
{
    oracle_job *job = (oracle_job *)arg;
    const oracle_args *a = job->a;
    int64_t nkb = 1;
    if (a->mask_kind == ORACLE_MASK_BLOCK) nkb = (a->K + a->kv_block - 1) / a->kv_block;
    double *z = (double *)malloc((size_t)a->K * sizeof(double));
    unsigned char *listed = (unsigned char *)malloc((size_t)nkb);
    unsigned char *full = (unsigned char *)malloc((size_t)nkb);
    if (!z || !listed || !full) {
        job->status = -2;
    } else {
        for (int64_t pos = job->first; pos < job->last; ++pos) compute_row(a, pos, z, listed, full);
        job->status = 0;
    }
    free(z);
    free(listed);
    free(full);
    return NULL;
}

int tri_oracle_fwd(int64_t B, int64_t N, int64_t H, int64_t Q, int64_t K, int64_t D,
                   const double *q, const double *k, const double *v, const double *bias,
                   int mask_kind, const uint8_t *dense, const int32_t *kv_lengths,
                   const int32_t *kv_num_blocks, const int32_t *kv_indices,
                   const int32_t *full_kv_num_blocks, const int32_t *full_kv_indices,
                   int64_t q_block, int64_t kv_block, int64_t max_blocks,
                   int64_t full_max_blocks, int mask_mod, int64_t stride_b, int64_t stride_n,
                   int64_t stride_h, double scale, int64_t n_rows, const int64_t *rows,
                   double *out, double *lse, double *mx, int n_threads)
{
    if (B < 0 || N < 0 || H < 0 || Q < 0 || K < 1 || D < 1) return -1;
    if (!q || !k || !v || !out || !lse || !mx) return -1;
    const int64_t total_rows = B * N * H * Q;
    if (!rows) n_rows = total_rows;
    if (n_rows < 0) return -1;
    if (rows)
        for (int64_t i = 0; i < n_rows; ++i)
            if (rows[i] < 0 || rows[i] >= total_rows) return -1;
    switch (mask_kind) {
    case ORACLE_MASK_NONE:
        break;
    case ORACLE_MASK_DENSE:
        if (!dense) return -1;
        break;
    case ORACLE_MASK_KV_LENGTHS:
        if (!kv_lengths) return -1;
        break;
    case ORACLE_MASK_BLOCK:
        if (!kv_num_blocks || !kv_indices || q_block < 1 || kv_block < 1 || max_blocks < 1)
            return -1;
        if ((full_kv_num_blocks == NULL) != (full_kv_indices == NULL)) return -1;
        if (full_kv_num_blocks && full_max_blocks < 1) return -1;
        if (mask_mod != ORACLE_MOD_NONE && mask_mod != ORACLE_MOD_CAUSAL) return -1;
        break;
    default:
        return -1;
    }
    if (n_rows == 0) return 0;

    oracle_args a;
    a.B = B; a.N = N; a.H = H; a.Q = Q; a.K = K; a.D = D;
    a.q = q; a.k = k; a.v = v; a.bias = bias;
    a.mask_kind = mask_kind; a.dense = dense; a.kv_lengths = kv_lengths;
    a.kv_num_blocks = kv_num_blocks; a.kv_indices = kv_indices;
    a.full_kv_num_blocks = full_kv_num_blocks; a.full_kv_indices = full_kv_indices;
    a.q_block = q_block; a.kv_block = kv_block;
    a.max_blocks = max_blocks; a.full_max_blocks = full_max_blocks;
    a.mask_mod = mask_mod;
    a.stride_b = stride_b; a.stride_n = stride_n; a.stride_h = stride_h;
    a.scale = isnan(scale) ? 1.0 / sqrt((double)D) : scale;
    a.n_rows = n_rows; a.rows = rows;
    a.out = out; a.lse = lse; a.mx = mx;

    if (n_threads <= 0) {
        long hc = sysconf(_SC_NPROCESSORS_ONLN);
        n_threads = hc > 0 ? (int)hc : 1;
    }
    if ((int64_t)n_threads > n_rows) n_threads = (int)n_rows;

    oracle_job *jobs = (oracle_job *)calloc((size_t)n_threads, sizeof(oracle_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)n_threads, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(jobs);
        free(tids);
        return -2;
    }
    for (int t = 0; t < n_threads; ++t) {
        jobs[t].a = &a;
        jobs[t].first = n_rows * t / n_threads;
        jobs[t].last = n_rows * (t + 1) / n_threads;
        jobs[t].status = -3;
    }
    int started = 0;
    for (int t = 1; t < n_threads; ++t) {
        if (pthread_create(&tids[t], NULL, run_job, &jobs[t]) != 0) break;
        started = t;
    }
    run_job(&jobs[0]);
    /* Any job whose thread failed to start runs here, in this thread. */
    for (int t = started + 1; t < n_threads; ++t) run_job(&jobs[t]);
    for (int t = 1; t <= started; ++t) pthread_join(tids[t], NULL);
    int status = 0;
    for (int t = 0; t < n_threads; ++t)
        if (jobs[t].status != 0) status = jobs[t].status;
    free(jobs);
    free(tids);
    return status;
}

/* Number of threads the oracle uses when asked for 0 (all online cores). */
int tri_oracle_default_threads(void)
{
    long hc = sysconf(_SC_NPROCESSORS_ONLN);
    return hc > 0 ? (int)hc : 1;
}
