/* Runs the fp64 oracle (forward, or backward with -DORACLE_BWD) on small
 * edge cases under AddressSanitizer / UndefinedBehaviorSanitizer: every mask
 * kind, lengths past both clamps, rows with no valid key, block lists with
 * duplicate, negative and out-of-range ids, counts past the list width,
 * full lists, the causal mask_mod, row subsets, a zero and a default scale.
 * Exits 0 when every call succeeds with finite results (a sanitizer report
 * aborts the process). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int tri_oracle_fwd(int64_t B, int64_t N, int64_t H, int64_t Q, int64_t K, int64_t D,
                   const double *q, const double *k, const double *v, const double *bias,
                   int mask_kind, const uint8_t *dense, const int32_t *kv_lengths,
                   const int32_t *kv_num_blocks, const int32_t *kv_indices,
                   const int32_t *full_kv_num_blocks, const int32_t *full_kv_indices,
                   int64_t q_block, int64_t kv_block, int64_t max_blocks,
                   int64_t full_max_blocks, int mask_mod, int64_t stride_b, int64_t stride_n,
                   int64_t stride_h, double scale, int64_t n_rows, const int64_t *rows,
                   double *out, double *lse, double *mx, int n_threads);
int tri_oracle_bwd(int64_t B, int64_t N, int64_t H, int64_t Q, int64_t K, int64_t D,
                   const double *q, const double *k, const double *v, const double *bias,
                   int mask_kind, const uint8_t *dense, const int32_t *kv_lengths,
                   const int32_t *kv_num_blocks, const int32_t *kv_indices,
                   const int32_t *full_kv_num_blocks, const int32_t *full_kv_indices,
                   int64_t q_block, int64_t kv_block, int64_t max_blocks,
                   int64_t full_max_blocks, int mask_mod, int64_t stride_b, int64_t stride_n,
                   int64_t stride_h, double scale, const double *dout, double *dq, double *dk,
                   double *dv, double *dbias, int64_t n_qsel, const int64_t *qsel,
                   int n_threads);

static uint64_t state = 12345;
static double rnd(void) {
    state = state * 6364136223846793005ULL + 1442695040888963407ULL;
    return (double)(state >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}
static double *fill(int64_t n) {
    double *p = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) p[i] = rnd();
    return p;
}
static int finite_all(const double *p, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) return 0;
    return 1;
}

struct blk {
    int32_t *num, *idx, *fnum, *fidx;
    int64_t qb, kb, width, fwidth;
    int mod;
};

static int run(int64_t B, int64_t N, int64_t H, int64_t Q, int64_t K, int64_t D, int kind,
               const uint8_t *dense, const int32_t *lens, const struct blk *bl, double scale,
               int with_bias, int subset) {
    double *q = fill(B * N * H * Q * D), *k = fill(B * N * H * K * D), *v = fill(B * N * H * K * D);
    double *bias = with_bias ? fill(B * H * Q * K) : NULL;
    int64_t sel[3] = {0, Q > 2 ? Q - 1 : 0, Q / 2};
    int64_t nsel = subset ? (Q > 2 ? 3 : 1) : 0;
    int rc;
#ifdef ORACLE_BWD
    double *dout = fill(B * N * H * Q * D);
    double *dq = fill(B * N * H * Q * D), *dk = fill(B * N * H * K * D), *dv = fill(B * N * H * K * D);
    double *db = with_bias ? fill(B * H * Q * K) : NULL;
    rc = tri_oracle_bwd(B, N, H, Q, K, D, q, k, v, bias, kind, dense, lens, bl ? bl->num : NULL,
                        bl ? bl->idx : NULL, bl ? bl->fnum : NULL, bl ? bl->fidx : NULL,
                        bl ? bl->qb : 0, bl ? bl->kb : 0, bl ? bl->width : 0, bl ? bl->fwidth : 0,
                        bl ? bl->mod : 0, 0, 0, 0, scale, dout, dq, dk, dv, db, nsel,
                        nsel ? sel : NULL, 2);
    if (rc == 0 && !(finite_all(dq, B * N * H * Q * D) && finite_all(dk, B * N * H * K * D) &&
                     finite_all(dv, B * N * H * K * D) && (!db || finite_all(db, B * H * Q * K))))
        rc = 99;
    free(dout); free(dq); free(dk); free(dv); free(db);
#else
    double *out = fill(B * N * H * Q * D), *lse = fill(B * N * H * Q), *mx = fill(B * N * H * Q);
    rc = tri_oracle_fwd(B, N, H, Q, K, D, q, k, v, bias, kind, dense, lens, bl ? bl->num : NULL,
                        bl ? bl->idx : NULL, bl ? bl->fnum : NULL, bl ? bl->fidx : NULL,
                        bl ? bl->qb : 0, bl ? bl->kb : 0, bl ? bl->width : 0, bl ? bl->fwidth : 0,
                        bl ? bl->mod : 0, 0, 0, 0, scale, nsel, nsel ? sel : NULL, out, lse, mx, 2);
    if (rc == 0 && nsel == 0 &&
        !(finite_all(out, B * N * H * Q * D) && finite_all(lse, B * N * H * Q) && finite_all(mx, B * N * H * Q)))
        rc = 99;
    free(out); free(lse); free(mx);
#endif
    free(q); free(k); free(v); free(bias);
    return rc;
}

int main(void) {
    int bad = 0;
    /* no mask; a default and a zero scale; a row subset */
    bad |= run(1, 2, 2, 5, 7, 8, 0, NULL, NULL, NULL, NAN, 1, 0) != 0;
    bad |= run(2, 1, 1, 3, 1, 4, 0, NULL, NULL, NULL, 0.0, 1, 1) != 0;
    /* dense mask: one (b, n) row with no valid key */
    {
        uint8_t dense[2 * 9] = {1, 0, 1, 1, 0, 0, 1, 0, 1, 0, 0, 0, 0, 0, 0, 0, 0, 0};
        bad |= run(1, 2, 1, 3, 9, 4, 1, dense, NULL, NULL, 0.5, 1, 0) != 0;
    }
    /* lengths past both clamps, and 0 */
    {
        int32_t lens[4] = {-3, 0, 4, 100};
        bad |= run(2, 2, 1, 6, 5, 8, 2, NULL, lens, NULL, NAN, 1, 1) != 0;
    }
    /* block lists: q_block 2, kv_block 3 over Q = 7, K = 8 (4 rows, 3 kv
       blocks); counts -1 and past the width, ids negative, duplicate and out
       of range, full lists, causal */
    {
        int32_t num[4] = {2, -1, 7, 3};
        int32_t idx[4 * 3] = {0, 2, 1, 1, 1, 1, -5, 99, 2, 2, 2, 0};
        int32_t fnum[4] = {1, 0, 2, 1};
        int32_t fidx[4 * 2] = {1, 0, 0, 0, 0, 2, 7, 0};
        struct blk b = {num, idx, fnum, fidx, 2, 3, 3, 2, 1};
        bad |= run(1, 1, 1, 7, 8, 4, 3, NULL, NULL, &b, NAN, 1, 0) != 0;
        b.mod = 0;
        b.fnum = NULL;
        b.fidx = NULL;
        b.fwidth = 0;
        bad |= run(1, 1, 1, 7, 8, 4, 3, NULL, NULL, &b, 0.25, 0, 1) != 0;
    }
    /* empty batch and head */
    bad |= run(0, 2, 2, 4, 4, 8, 0, NULL, NULL, NULL, NAN, 1, 0) != 0;
    bad |= run(1, 1, 0, 4, 4, 8, 0, NULL, NULL, NULL, NAN, 1, 0) != 0;
    printf(bad ? "oracle driver: FAILED\n" : "oracle driver: ok\n");
    return bad;
}
