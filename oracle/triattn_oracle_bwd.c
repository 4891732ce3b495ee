/*
 * triattn_oracle_bwd.c -- plain fp64 CPU oracle for the gradient of the
 * masked, biased triangle attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  The checker the GPU backward is measured
 * against; never part of the product path.  It shares no code, header, table
 * or helper with the HIP library, nor with the forward oracle (it evaluates
 * the forward of each row itself, from the same definition).
 *
 * Forward (cuEquivariance "cuequivariance_torch.triangle_attention" API page,
 * the defining equation), per query row q of every (b,n,h):
 *
 *     z_k = s * (Q_q . K_k) + B_qk      if key k is valid
 *     z_k = -1e9                        otherwise (a constant)
 *     P_k = softmax_k(z),   O_q = sum_k P_k V_k
 *
 * Backward of O (the page's backward pass differentiates the output; the lse
 * and max auxiliaries carry no incoming gradient here).  With dO the
 * gradient of O_q, the chain rule through the softmax gives
 *
 *     dV_k  += P_k dO                              every key k
 *     dP_k   = dO . V_k
 *     dz_k   = P_k (dP_k - sum_j P_j dP_j)
 *     dQ_q  += s dz_k K_k,   dK_k += s dz_k Q_q,   dB_qk += dz_k
 *                                                  valid keys only
 *
 * A masked key's logit is the constant -1e9, so nothing flows through it to
 * Q, K or the bias.  In a row with no valid key every logit is that constant:
 * P_k = 1/K, dV_k += dO / K, and the row contributes nothing else.  The bias
 * is shared by every n (shape (B,1,H,Q,K)), so its gradient sums over n.
 *
 * The key-validity predicate and all argument conventions are those of the
 * forward oracle (triattn_oracle.c): NONE, DENSE (B,N,K) bytes, KV_LENGTHS
 * (B,N) int32 clamped to [0,K], BLOCK lists in the BlockMask format of the
 * "tensorplay.nn.attention" page (visited = kv lists united with full lists,
 * mask_mod on non-full blocks only, counts clamped, out-of-range ids
 * ignored).  scale NaN selects 1/sqrt(D).
 *
 * Outputs (fp64, written in full): dq (B,N,H,Q,D); dk, dv (B,N,H,K,D);
 * dbias (B,1,H,Q,K) or NULL (not computed).  Work is split over (b,h)
 * pairs, each of which owns its slice of every output.
 *
 * Optional row subset: with qsel non-NULL only the query rows listed in
 * qsel[0..n_qsel) (each in [0,Q), no repeats) are evaluated, for every
 * (b,n,h).  dq and dbias are then exact on those rows and zero elsewhere;
 * dk and dv hold only those rows' contributions.  This lets a test check
 * the bias gradient (a sum over every n) on a few rows of a large case.
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

enum { BWD_MASK_NONE = 0, BWD_MASK_DENSE = 1, BWD_MASK_KV_LENGTHS = 2, BWD_MASK_BLOCK = 3 };
enum { BWD_MOD_NONE = 0, BWD_MOD_CAUSAL = 1 };

typedef struct {
    int64_t B, N, H, Q, K, D;
    const double *q, *k, *v, *bias, *dout;
    int mask_kind;
    const uint8_t *dense;
    const int32_t *kv_lengths;
    const int32_t *kv_num_blocks, *kv_indices;
    const int32_t *full_kv_num_blocks, *full_kv_indices;
    int64_t q_block, kv_block, max_blocks, full_max_blocks;
    int mask_mod;
    int64_t stride_b, stride_n, stride_h;
    double scale;
    double *dq, *dk, *dv, *dbias;
    int64_t n_qsel;
    const int64_t *qsel; /* NULL: every query row */
} bwd_args;

typedef struct {
    const bwd_args *a;
    int64_t first, last; /* [first, last) of the (b,h) pairs */
    int status;
} bwd_job;

/* listed[j] = 1 for the kv blocks among a list row's first `count` ids. */
static void bwd_mark(const int32_t *counts, const int32_t *ids, int64_t list_row, int64_t width,
                     int64_t n_blocks, unsigned char *listed)
{
    int64_t count = counts[list_row];
    if (count < 0) count = 0;
    if (count > width) count = width;
    for (int64_t j = 0; j < count; ++j) {
        const int64_t id = ids[list_row * width + j];
        if (id >= 0 && id < n_blocks) listed[id] = 1;
    }
}

/* valid[k] for query row qi of slice (b,n,h). */
static void bwd_valid_keys(const bwd_args *a, int64_t b, int64_t n, int64_t h, int64_t qi,
                           unsigned char *valid, unsigned char *listed, unsigned char *full)
{
    const int64_t K = a->K;
    for (int64_t kk = 0; kk < K; ++kk) valid[kk] = 1;
    if (a->mask_kind == BWD_MASK_DENSE) {
        for (int64_t kk = 0; kk < K; ++kk) valid[kk] = a->dense[(b * a->N + n) * K + kk] != 0;
    } else if (a->mask_kind == BWD_MASK_KV_LENGTHS) {
        int64_t len = a->kv_lengths[b * a->N + n];
        if (len < 0) len = 0;
        if (len > K) len = K;
        for (int64_t kk = 0; kk < K; ++kk) valid[kk] = kk < len;
    } else if (a->mask_kind == BWD_MASK_BLOCK) {
        const int64_t nkb = (K + a->kv_block - 1) / a->kv_block;
        const int64_t rows = (a->Q + a->q_block - 1) / a->q_block;
        const int64_t inst = b * a->stride_b + n * a->stride_n + h * a->stride_h;
        const int64_t list_row = inst * rows + qi / a->q_block;
        memset(listed, 0, (size_t)nkb);
        memset(full, 0, (size_t)nkb);
        bwd_mark(a->kv_num_blocks, a->kv_indices, list_row, a->max_blocks, nkb, listed);
        if (a->full_kv_num_blocks)
            bwd_mark(a->full_kv_num_blocks, a->full_kv_indices, list_row, a->full_max_blocks,
                     nkb, full);
        for (int64_t kk = 0; kk < K; ++kk) {
            const int64_t blk = kk / a->kv_block;
            if (full[blk]) continue;  /* a full block: every key valid */
            if (!listed[blk]) valid[kk] = 0;
            else if (a->mask_mod == BWD_MOD_CAUSAL) valid[kk] = qi >= kk;
        }
    }
}

static void bwd_pair(const bwd_args *a, int64_t bh, double *z, double *dp, unsigned char *valid,
                     unsigned char *listed, unsigned char *full)
{
    const int64_t N = a->N, H = a->H, Q = a->Q, K = a->K, D = a->D;
    const int64_t b = bh / H, h = bh % H;
    double *dbias = a->dbias ? a->dbias + (b * H + h) * Q * K : NULL;
    if (dbias) memset(dbias, 0, (size_t)(Q * K) * sizeof(double));
    for (int64_t n = 0; n < N; ++n) {
        const int64_t bnh = (b * N + n) * H + h;
        const double *kb = a->k + bnh * K * D, *vb = a->v + bnh * K * D;
        double *dkb = a->dk + bnh * K * D, *dvb = a->dv + bnh * K * D;
        memset(dkb, 0, (size_t)(K * D) * sizeof(double));
        memset(dvb, 0, (size_t)(K * D) * sizeof(double));
        if (a->qsel) memset(a->dq + bnh * Q * D, 0, (size_t)(Q * D) * sizeof(double));
        const int64_t n_q = a->qsel ? a->n_qsel : Q;
        for (int64_t qj = 0; qj < n_q; ++qj) {
            const int64_t qi = a->qsel ? a->qsel[qj] : qj;
            const int64_t row = bnh * Q + qi;
            const double *qr = a->q + row * D, *go = a->dout + row * D;
            double *dqr = a->dq + row * D;
            const double *br = a->bias ? a->bias + ((b * H + h) * Q + qi) * K : NULL;
            bwd_valid_keys(a, b, n, h, qi, valid, listed, full);
            /* forward of this row: logits, then the softmax weights in z */
            int any = 0;
            for (int64_t kk = 0; kk < K; ++kk) {
                if (valid[kk]) {
                    double dot = 0.0;
                    for (int64_t d = 0; d < D; ++d) dot += qr[d] * kb[kk * D + d];
                    z[kk] = a->scale * dot + (br ? br[kk] : 0.0);
                    any = 1;
                } else {
                    z[kk] = -1.0e9;
                }
            }
            double m = z[0];
            for (int64_t kk = 1; kk < K; ++kk) m = z[kk] > m ? z[kk] : m;
            double l = 0.0;
            for (int64_t kk = 0; kk < K; ++kk) {
                z[kk] = exp(z[kk] - m);
                l += z[kk];
            }
            for (int64_t kk = 0; kk < K; ++kk) z[kk] /= l;
            /* dV, dP and the softmax's backward */
            double delta = 0.0;
            for (int64_t kk = 0; kk < K; ++kk) {
                double g = 0.0;
                for (int64_t d = 0; d < D; ++d) {
                    dvb[kk * D + d] += z[kk] * go[d];
                    g += go[d] * vb[kk * D + d];
                }
                dp[kk] = g;
                delta += z[kk] * g;
            }
            for (int64_t d = 0; d < D; ++d) dqr[d] = 0.0;
            if (!any) continue; /* every logit a constant: no gradient to q, k, bias */
            for (int64_t kk = 0; kk < K; ++kk) {
                if (!valid[kk]) continue;
                const double dz = z[kk] * (dp[kk] - delta);
                for (int64_t d = 0; d < D; ++d) {
                    dqr[d] += a->scale * dz * kb[kk * D + d];
                    dkb[kk * D + d] += a->scale * dz * qr[d];
                }
                if (dbias) dbias[qi * K + kk] += dz;
            }
        }
    }
}

static void *bwd_run(void *arg)
{
    bwd_job *job = (bwd_job *)arg;
    const bwd_args *a = job->a;
    const int64_t nkb = a->mask_kind == BWD_MASK_BLOCK ? (a->K + a->kv_block - 1) / a->kv_block : 1;
    double *z = (double *)malloc((size_t)a->K * sizeof(double));
    double *dp = (double *)malloc((size_t)a->K * sizeof(double));
    unsigned char *valid = (unsigned char *)malloc((size_t)a->K);
    unsigned char *listed = (unsigned char *)malloc((size_t)nkb);
    unsigned char *full = (unsigned char *)malloc((size_t)nkb);
    if (!z || !dp || !valid || !listed || !full) {
        job->status = -2;
    } else {
        for (int64_t bh = job->first; bh < job->last; ++bh) bwd_pair(a, bh, z, dp, valid, listed, full);
        job->status = 0;
    }
    free(z);
    free(dp);
    free(valid);
    free(listed);
    free(full);
    return NULL;
}

int tri_oracle_bwd(int64_t B, int64_t N, int64_t H, int64_t Q, int64_t K, int64_t D,
                   const double *q, const double *k, const double *v, const double *bias,
                   int mask_kind, const uint8_t *dense, const int32_t *kv_lengths,
                   const int32_t *kv_num_blocks, const int32_t *kv_indices,
                   const int32_t *full_kv_num_blocks, const int32_t *full_kv_indices,
                   int64_t q_block, int64_t kv_block, int64_t max_blocks,
                   int64_t full_max_blocks, int mask_mod, int64_t stride_b, int64_t stride_n,
                   int64_t stride_h, double scale, const double *dout, double *dq, double *dk,
                   double *dv, double *dbias, int64_t n_qsel, const int64_t *qsel,
                   int n_threads)
{
    if (B < 0 || N < 0 || H < 0 || Q < 0 || K < 1 || D < 1) return -1;
    if (qsel) {
        if (n_qsel < 0) return -1;
        for (int64_t j = 0; j < n_qsel; ++j)
            if (qsel[j] < 0 || qsel[j] >= Q) return -1;
    }
    if (!q || !k || !v || !dout || !dq || !dk || !dv) return -1;
    if (mask_kind == BWD_MASK_DENSE && !dense) return -1;
    if (mask_kind == BWD_MASK_KV_LENGTHS && !kv_lengths) return -1;
    if (mask_kind == BWD_MASK_BLOCK) {
        if (!kv_num_blocks || !kv_indices || q_block < 1 || kv_block < 1 || max_blocks < 1)
            return -1;
        if ((full_kv_num_blocks == NULL) != (full_kv_indices == NULL)) return -1;
        if (full_kv_num_blocks && full_max_blocks < 1) return -1;
        if (mask_mod != BWD_MOD_NONE && mask_mod != BWD_MOD_CAUSAL) return -1;
    } else if (mask_kind < 0 || mask_kind > BWD_MASK_BLOCK) {
        return -1;
    }
    const int64_t pairs = B * H;
    if (pairs == 0) return 0;

    bwd_args a;
    a.B = B; a.N = N; a.H = H; a.Q = Q; a.K = K; a.D = D;
    a.q = q; a.k = k; a.v = v; a.bias = bias; a.dout = dout;
    a.mask_kind = mask_kind; a.dense = dense; a.kv_lengths = kv_lengths;
    a.kv_num_blocks = kv_num_blocks; a.kv_indices = kv_indices;
    a.full_kv_num_blocks = full_kv_num_blocks; a.full_kv_indices = full_kv_indices;
    a.q_block = q_block; a.kv_block = kv_block;
    a.max_blocks = max_blocks; a.full_max_blocks = full_max_blocks; a.mask_mod = mask_mod;
    a.stride_b = stride_b; a.stride_n = stride_n; a.stride_h = stride_h;
    a.scale = isnan(scale) ? 1.0 / sqrt((double)D) : scale;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dbias = bias ? dbias : NULL;
    a.n_qsel = n_qsel; a.qsel = qsel;
    if (dbias && !bias) memset(dbias, 0, (size_t)(B * H * Q * K) * sizeof(double));

    if (n_threads <= 0) {
        const long hc = sysconf(_SC_NPROCESSORS_ONLN);
        n_threads = hc > 0 ? (int)hc : 1;
    }
    if ((int64_t)n_threads > pairs) n_threads = (int)pairs;
    bwd_job *jobs = (bwd_job *)calloc((size_t)n_threads, sizeof(bwd_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)n_threads, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(jobs);
        free(tids);
        return -2;
    }
    for (int t = 0; t < n_threads; ++t) {
        jobs[t].a = &a;
        jobs[t].first = pairs * t / n_threads;
        jobs[t].last = pairs * (t + 1) / n_threads;
        jobs[t].status = -3;
    }
    int started = 0;
    for (int t = 1; t < n_threads; ++t) {
        if (pthread_create(&tids[t], NULL, bwd_run, &jobs[t]) != 0) break;
        started = t;
    }
    bwd_run(&jobs[0]);
    for (int t = started + 1; t < n_threads; ++t) bwd_run(&jobs[t]);
    for (int t = 1; t <= started; ++t) pthread_join(tids[t], NULL);
    int status = 0;
    for (int t = 0; t < n_threads; ++t)
        if (jobs[t].status != 0) status = jobs[t].status;
    free(jobs);
    free(tids);
    return status;
}
