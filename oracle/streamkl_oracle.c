/*
 * Attention KL-divergence oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, fp64 CPU definition of what the fused attention-KL primitive
 * computes.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline leg may load this library; the product path never does.  It shares
 * no code, header or constant with the GPU library.
 *
 * What is computed (StreamKL, arXiv 2606.20005; abstract on paperdance.org /
 * fugumt.com, and gist.science "Declaracion del Problema"): for one
 * (batch, head) slice, teacher P1 = softmax(scale * Q1 K1^T) and student
 * P2 = softmax(scale * Q2 K2^T), each row restricted to the visible keys, and
 * the per-row divergence KL_i = sum_j P1_ij * log(P1_ij / P2_ij).
 *
 * Readings taken where the pages leave a step open:
 *  - visible keys of row i: j < NK and, when causal, j <= i + NK - NQ
 *    (bottom-right alignment; masked keys carry probability 0 and add nothing);
 *  - LSE_t = log sum_j exp(s_t,ij) in natural-log units of the scaled logits,
 *    the quantity the pages save for the backward ("LSE_t = m_t + log l_t",
 *    gist.science "Formulacion Online");
 *  - log(P1/P2) is taken as (s1 - LSE1) - (s2 - LSE2), from logits rather than
 *    from logs of probabilities (gist.science "Estabilidad Numerica");
 *  - the loss is L = sum_i g_i * KL_i; the gradients w.r.t. the logits are
 *    dS2_ij = g_i (P2_ij - P1_ij)                      (student, "Configuracion 1")
 *    dS1_ij = g_i P1_ij (log P1_ij - log P2_ij - KL_i) (teacher, "Configuracion 2")
 *    and, through s = scale * q.k, dQ_t = scale * dS_t K_t, dK_t = scale * dS_t^T Q_t.
 *    These follow from differentiating the definition; the pages print no
 *    gradient formula (gist.science "Estrategia de Recomputacion").
 *
 * Every function takes one (batch, head) slice: q* is [nq, d], k* is [nk, d],
 * row-major fp64.  `rows` lists the query rows to evaluate (any subset, any
 * order); per-row outputs are indexed by position in `rows`.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static int visible(int64_t i, int64_t j, int64_t nq, int64_t nk, int causal)
{
    if (j < 0 || j >= nk) return 0;
    if (!causal) return 1;
    return j <= i + (nk - nq);
}

static double dot(const double *a, const double *b, int64_t d)
{
    double s = 0.0;
    for (int64_t k = 0; k < d; ++k) s += a[k] * b[k];
    return s;
}

/* log-sum-exp over the visible entries of one row, two passes (max, then sum). */
static double row_lse(const double *s, const unsigned char *vis, int64_t nk)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < nk; ++j)
        if (vis[j] && s[j] > m) m = s[j];
    if (m == -INFINITY) return -INFINITY;
    double acc = 0.0;
    for (int64_t j = 0; j < nk; ++j)
        if (vis[j]) acc += exp(s[j] - m);
    return m + log(acc);
}

/*
 * Row statistics for row i: logits of both distributions, both LSEs and KL.
 * s1, s2, vis are caller scratch of length nk.
 */
static void row_forward(int64_t i, int64_t nq, int64_t nk, int64_t d, double scale, int causal,
                        const double *q1, const double *k1, const double *q2, const double *k2,
                        double *s1, double *s2, unsigned char *vis,
                        double *kl_out, double *lse1_out, double *lse2_out)
{
    const double *q1i = q1 + i * d, *q2i = q2 + i * d;
    for (int64_t j = 0; j < nk; ++j) {
        vis[j] = (unsigned char)visible(i, j, nq, nk, causal);
        if (vis[j]) {
            s1[j] = scale * dot(q1i, k1 + j * d, d);
            s2[j] = scale * dot(q2i, k2 + j * d, d);
        } else {
            s1[j] = s2[j] = 0.0;
        }
    }
    double lse1 = row_lse(s1, vis, nk);
    double lse2 = row_lse(s2, vis, nk);
    double kl = 0.0;
    for (int64_t j = 0; j < nk; ++j) {
        if (!vis[j]) continue;
        double logp1 = s1[j] - lse1;
        double logp2 = s2[j] - lse2;
        double p1 = exp(logp1);
        kl += p1 * (logp1 - logp2);
    }
    *kl_out = kl;
    *lse1_out = lse1;
    *lse2_out = lse2;
}

/* Number of OpenMP threads the oracle uses (1 without OpenMP). */
int skl_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Forward: KL, LSE1, LSE2 for the listed rows of one (batch, head) slice.
 * Returns 0, or -1 on allocation failure / bad argument.
 */
int skl_oracle_fwd(int64_t nq, int64_t nk, int64_t d, double scale, int causal,
                   const double *q1, const double *k1, const double *q2, const double *k2,
                   const int64_t *rows, int64_t nrows,
                   double *kl, double *lse1, double *lse2)
{
    if (nq < 0 || nk < 0 || d <= 0 || nrows < 0) return -1;
    int err = 0;
#pragma omp parallel
    {
        double *s1 = (double *)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
        double *s2 = (double *)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
        unsigned char *vis = (unsigned char *)malloc((size_t)(nk > 0 ? nk : 1));
        if (!s1 || !s2 || !vis) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < nrows; ++r) {
                row_forward(rows[r], nq, nk, d, scale, causal, q1, k1, q2, k2, s1, s2, vis,
                            &kl[r], &lse1[r], &lse2[r]);
            }
        }
        free(s1);
        free(s2);
        free(vis);
    }
    return err ? -1 : 0;
}

/*
 * Backward for the listed rows of one (batch, head) slice, with upstream
 * gradient g[r] for row rows[r] (rows not listed have g = 0).
 *
 * Outputs: kl/lse1/lse2 per listed row (recomputed here from the definition,
 * never taken from elsewhere), dq1/dq2 as [nrows, d], and dk1/dk2 as [nk, d]
 * holding the contribution of the listed rows (overwritten).
 */
int skl_oracle_bwd(int64_t nq, int64_t nk, int64_t d, double scale, int causal,
                   const double *q1, const double *k1, const double *q2, const double *k2,
                   const int64_t *rows, int64_t nrows, const double *g,
                   double *kl, double *lse1, double *lse2,
                   double *dq1, double *dq2, double *dk1, double *dk2)
{
    if (nq < 0 || nk < 0 || d <= 0 || nrows < 0) return -1;
    int err = 0;

    /* Pass 1, per row: statistics, then dQ_t[i] = scale * sum_j dS_t,ij K_t[j]. */
#pragma omp parallel
    {
        double *s1 = (double *)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
        double *s2 = (double *)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
        unsigned char *vis = (unsigned char *)malloc((size_t)(nk > 0 ? nk : 1));
        if (!s1 || !s2 || !vis) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < nrows; ++r) {
                int64_t i = rows[r];
                row_forward(i, nq, nk, d, scale, causal, q1, k1, q2, k2, s1, s2, vis,
                            &kl[r], &lse1[r], &lse2[r]);
                double *dq1r = dq1 + r * d, *dq2r = dq2 + r * d;
                for (int64_t k = 0; k < d; ++k) dq1r[k] = dq2r[k] = 0.0;
                for (int64_t j = 0; j < nk; ++j) {
                    if (!vis[j]) continue;
                    double logp1 = s1[j] - lse1[r];
                    double logp2 = s2[j] - lse2[r];
                    double p1 = exp(logp1), p2 = exp(logp2);
                    double ds2 = g[r] * (p2 - p1);
                    double ds1 = g[r] * p1 * (logp1 - logp2 - kl[r]);
                    const double *k1j = k1 + j * d, *k2j = k2 + j * d;
                    for (int64_t k = 0; k < d; ++k) {
                        dq1r[k] += ds1 * k1j[k];
                        dq2r[k] += ds2 * k2j[k];
                    }
                }
                for (int64_t k = 0; k < d; ++k) {
                    dq1r[k] *= scale;
                    dq2r[k] *= scale;
                }
            }
        }
        free(s1);
        free(s2);
        free(vis);
    }
    if (err) return -1;

    /* Pass 2, per key: dK_t[j] = scale * sum_i dS_t,ij Q_t[i], rows in list order. */
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t j = 0; j < nk; ++j) {
        double *dk1j = dk1 + j * d, *dk2j = dk2 + j * d;
        for (int64_t k = 0; k < d; ++k) dk1j[k] = dk2j[k] = 0.0;
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t i = rows[r];
            if (!visible(i, j, nq, nk, causal)) continue;
            const double *q1i = q1 + i * d, *q2i = q2 + i * d;
            double s1 = scale * dot(q1i, k1 + j * d, d);
            double s2 = scale * dot(q2i, k2 + j * d, d);
            double logp1 = s1 - lse1[r];
            double logp2 = s2 - lse2[r];
            double p1 = exp(logp1), p2 = exp(logp2);
            double ds2 = g[r] * (p2 - p1);
            double ds1 = g[r] * p1 * (logp1 - logp2 - kl[r]);
            for (int64_t k = 0; k < d; ++k) {
                dk1j[k] += ds1 * q1i[k];
                dk2j[k] += ds2 * q2i[k];
            }
        }
        for (int64_t k = 0; k < d; ++k) {
            dk1j[k] *= scale;
            dk2j[k] *= scale;
        }
    }
    return 0;
}
