/*
 * oracle.c -- plain fp64 CPU reference for exact attention forward.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h): used by the tests, the smoke entry
 * point and the benchmark's CPU-baseline leg, never by the product path.
 *
 * This is the naive attention workflow written out in double precision
 * (chenyy20.com "抱infra脚", section Flash Attention 基本原理 / 核心技术:
 * S = QK^T is materialised, softmax turns it into P, and O = PV), which is the
 * result FlashAttention must reproduce exactly ("推理加速" interview notes,
 * section FlashAttention: not an approximation, mathematically equal to
 * standard attention).  There is no tiling, no online softmax and no reduced
 * precision here: every score row is complete before its softmax is taken.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One (batch, query head) pair seen as a plain matrix problem: query row i
 * lives at q + i * q_rs, key / value row j at k + j * kv_rs (v likewise). */
typedef struct {
    const float *q, *k, *v;
    long q_rs, kv_rs;
    long Sq, Sk, D;
    int causal;
    double scale;
} head_view;

/* Causal visibility, bottom-right aligned: with Sq queries ending at the same
 * position as the Sk keys, query i may attend to key j iff j <= i + (Sk - Sq).
 * Without the causal flag every key is visible. */
static int visible(const head_view *hv, long i, long j)
{
    if (!hv->causal) return 1;
    return j <= i + (hv->Sk - hv->Sq);
}

/* Evaluate query rows rows_i[0..n) of one head.
 *   SP        scratch of n * Sk doubles: first the scores S, then P in place
 *   o_out     row r written at o_out + r * o_rs (D doubles)
 *   lse_out   row r written at lse_out[r * lse_rs]
 */
static void attend_rows(const head_view *hv, const long *rows_i, long n,
                        double *SP, double *o_out, long o_rs,
                        double *lse_out, long lse_rs)
{
    const long Sk = hv->Sk, D = hv->D;

    for (long r = 0; r < n; ++r) {
        const long i = rows_i[r];
        const float *qi = hv->q + i * hv->q_rs;
        double *S = SP + r * Sk;

        /* Step 1: scaled scores S[i, j] = scale * <q_i, k_j>; masked -> -inf. */
        for (long j = 0; j < Sk; ++j) {
            if (!visible(hv, i, j)) { S[j] = -INFINITY; continue; }
            const float *kj = hv->k + j * hv->kv_rs;
            double dot = 0.0;
            for (long d = 0; d < D; ++d) dot += (double)qi[d] * (double)kj[d];
            S[j] = hv->scale * dot;
        }

        /* Step 2: softmax over the visible entries of the row.  The row max m
         * is subtracted only to keep exp() in range; softmax does not depend
         * on it.  P overwrites S. */
        double m = -INFINITY;
        for (long j = 0; j < Sk; ++j)
            if (S[j] > m) m = S[j];

        double *oi = o_out + r * o_rs;
        if (m == -INFINITY) {              /* no visible key at all */
            for (long j = 0; j < Sk; ++j) S[j] = 0.0;
            for (long d = 0; d < D; ++d) oi[d] = 0.0;
            lse_out[r * lse_rs] = -INFINITY;
            continue;
        }
        double l = 0.0;
        for (long j = 0; j < Sk; ++j) {
            double e = (S[j] == -INFINITY) ? 0.0 : exp(S[j] - m);
            S[j] = e;
            l += e;
        }
        for (long j = 0; j < Sk; ++j) S[j] /= l;

        /* Step 3: O[i, :] = sum_j P[i, j] * V[j, :]; keys with P = 0 because
         * they are masked are not read at all. */
        for (long d = 0; d < D; ++d) oi[d] = 0.0;
        for (long j = 0; j < Sk; ++j) {
            if (!visible(hv, i, j)) continue;
            const float *vj = hv->v + j * hv->kv_rs;
            const double p = S[j];
            for (long d = 0; d < D; ++d) oi[d] += p * (double)vj[d];
        }

        /* Log-sum-exp of the visible scaled scores, natural log. */
        lse_out[r * lse_rs] = m + log(l);
    }
}

static int dims_ok(long B, long Sq, long Sk, long Hq, long Hkv, long D)
{
    if (B < 0 || Sq < 0 || Sk < 0 || Hq <= 0 || Hkv <= 0 || D <= 0) return 0;
    if (Hq % Hkv != 0) return 0;
    return 1;
}

static head_view make_view(const float *q, const float *k, const float *v,
                           long b, long hq, long Sq, long Sk, long Hq, long Hkv,
                           long D, int causal, double scale)
{
    const long group = Hq / Hkv;
    const long hk = hq / group;            /* consecutive query heads share a KV head */
    head_view hv;
    hv.q = q + (b * Sq * Hq + hq) * D;
    hv.k = k + (b * Sk * Hkv + hk) * D;
    hv.v = v + (b * Sk * Hkv + hk) * D;
    hv.q_rs = Hq * D;
    hv.kv_rs = Hkv * D;
    hv.Sq = Sq; hv.Sk = Sk; hv.D = D;
    hv.causal = causal;
    hv.scale = scale;
    return hv;
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_attention(const float *q, const float *k, const float *v,
                     double *o, double *lse,
                     long B, long Sq, long Sk, long Hq, long Hkv, long D,
                     int causal, double scale, int nthreads)
{
    if (!dims_ok(B, Sq, Sk, Hq, Hkv, D)) return -1;
    if (B == 0 || Sq == 0) return 0;
    set_threads(nthreads);

    long *rows = (long *)malloc((size_t)Sq * sizeof(long));
    if (!rows) return -2;
    for (long i = 0; i < Sq; ++i) rows[i] = i;

    int failed = 0;
    const long pairs = B * Hq;
#pragma omp parallel for schedule(dynamic, 1)
    for (long p = 0; p < pairs; ++p) {
        const long b = p / Hq, hq = p % Hq;
        /* The whole Sq x Sk score matrix of this head, then P in its place. */
        double *SP = (double *)malloc((size_t)Sq * (size_t)(Sk > 0 ? Sk : 1) * sizeof(double));
        if (!SP) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        head_view hv = make_view(q, k, v, b, hq, Sq, Sk, Hq, Hkv, D, causal, scale);
        attend_rows(&hv, rows, Sq, SP,
                    o + (b * Sq * Hq + hq) * D, Hq * D,
                    lse + (b * Hq + hq) * Sq, 1);
        free(SP);
    }
    free(rows);
    return failed ? -2 : 0;
}

int oracle_attention_rows(const float *q, const float *k, const float *v,
                          long B, long Sq, long Sk, long Hq, long Hkv, long D,
                          int causal, double scale,
                          const long *row_b, const long *row_h, const long *row_i,
                          long nrows, double *o, double *lse, int nthreads)
{
    if (!dims_ok(B, Sq, Sk, Hq, Hkv, D) || nrows < 0) return -1;
    for (long r = 0; r < nrows; ++r)
        if (row_b[r] < 0 || row_b[r] >= B || row_h[r] < 0 || row_h[r] >= Hq ||
            row_i[r] < 0 || row_i[r] >= Sq)
            return -1;
    set_threads(nthreads);

    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (long r = 0; r < nrows; ++r) {
        double *SP = (double *)malloc((size_t)(Sk > 0 ? Sk : 1) * sizeof(double));
        if (!SP) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        head_view hv = make_view(q, k, v, row_b[r], row_h[r], Sq, Sk, Hq, Hkv, D,
                                 causal, scale);
        attend_rows(&hv, &row_i[r], 1, SP, o + r * D, D, lse + r, 1);
        free(SP);
    }
    return failed ? -2 : 0;
}

int oracle_scores_probs(const float *q, const float *k,
                        long B, long Sq, long Sk, long Hq, long Hkv, long D,
                        int causal, double scale, long b, long hq,
                        double *S, double *P)
{
    if (!dims_ok(B, Sq, Sk, Hq, Hkv, D)) return -1;
    if (b < 0 || b >= B || hq < 0 || hq >= Hq) return -1;
    /* V is not needed for S and P; point it at K so the view is complete. */
    head_view hv = make_view(q, k, k, b, hq, Sq, Sk, Hq, Hkv, D, causal, scale);

    for (long i = 0; i < Sq; ++i) {
        const float *qi = hv.q + i * hv.q_rs;
        for (long j = 0; j < Sk; ++j) {
            if (!visible(&hv, i, j)) { S[i * Sk + j] = -INFINITY; continue; }
            const float *kj = hv.k + j * hv.kv_rs;
            double dot = 0.0;
            for (long d = 0; d < D; ++d) dot += (double)qi[d] * (double)kj[d];
            S[i * Sk + j] = scale * dot;
        }
    }
    /* P from the same attend_rows path the outputs use, so the pins on P
     * test the code that produces O. */
    long *rows = (long *)malloc((size_t)(Sq > 0 ? Sq : 1) * sizeof(long));
    double *o = (double *)malloc((size_t)(Sq > 0 ? Sq : 1) * (size_t)D * sizeof(double));
    double *l = (double *)malloc((size_t)(Sq > 0 ? Sq : 1) * sizeof(double));
    if (!rows || !o || !l) { free(rows); free(o); free(l); return -2; }
    for (long i = 0; i < Sq; ++i) rows[i] = i;
    attend_rows(&hv, rows, Sq, P, o, D, l, 1);
    free(rows); free(o); free(l);
    return 0;
}

int oracle_decode(const float *q, const float *k_log, const float *v_log,
                  const long *seq_off, const long *ctx,
                  long B, long Hq, long Hkv, long D, double scale,
                  double *o, double *lse, int nthreads)
{
    if (!dims_ok(B, 1, 0, Hq, Hkv, D)) return -1;
    for (long b = 0; b < B; ++b)
        if (ctx[b] < 0 || seq_off[b] < 0) return -1;
    set_threads(nthreads);

    const long group = Hq / Hkv;
    int failed = 0;
    const long pairs = B * Hq;
#pragma omp parallel for schedule(dynamic, 1)
    for (long p = 0; p < pairs; ++p) {
        const long b = p / Hq, hq = p % Hq, hk = hq / group;
        double *SP = (double *)malloc((size_t)(ctx[b] > 0 ? ctx[b] : 1) * sizeof(double));
        if (!SP) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        /* A decode step is attention of one query row against every cached
         * key of its sequence: Sq = 1, Sk = ctx[b], all keys visible. */
        head_view hv;
        hv.q = q + (b * Hq + hq) * D;
        hv.k = k_log + (seq_off[b] * Hkv + hk) * D;
        hv.v = v_log + (seq_off[b] * Hkv + hk) * D;
        hv.q_rs = D;
        hv.kv_rs = Hkv * D;
        hv.Sq = 1; hv.Sk = ctx[b]; hv.D = D;
        hv.causal = 0;
        hv.scale = scale;
        const long row0 = 0;
        attend_rows(&hv, &row0, 1, SP, o + (b * Hq + hq) * D, D, lse + b * Hq + hq, 1);
        free(SP);
    }
    return failed ? -2 : 0;
}

int oracle_lse_combine(const double *o_parts, const double *lse_parts, long n,
                       long D, double *o, double *lse)
{
    if (n < 0 || D <= 0) return -1;
    /* Partial s holds O_s = (sum_{j in s} e^{S_j} V_j) / l_s and
     * lse_s = ln l_s with l_s = sum_{j in s} e^{S_j}.  Over the union,
     * l = sum_s l_s and O = sum_s l_s O_s / l.  Taking M = max_s lse_s and
     * w_s = e^{lse_s - M} (= l_s / e^M) keeps the weights in range. */
    double M = -INFINITY;
    for (long s = 0; s < n; ++s)
        if (lse_parts[s] > M) M = lse_parts[s];
    for (long d = 0; d < D; ++d) o[d] = 0.0;
    if (M == -INFINITY) {                  /* every part is empty */
        *lse = -INFINITY;
        return 0;
    }
    double wsum = 0.0;
    for (long s = 0; s < n; ++s) {
        if (lse_parts[s] == -INFINITY) continue;
        const double w = exp(lse_parts[s] - M);
        wsum += w;
        for (long d = 0; d < D; ++d) o[d] += w * o_parts[s * D + d];
    }
    for (long d = 0; d < D; ++d) o[d] /= wsum;
    *lse = M + log(wsum);
    return 0;
}
