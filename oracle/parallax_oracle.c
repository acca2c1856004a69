/*
 * parallax_oracle.c -- fp64 CPU oracle of the Parallax attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it, to check and to time the GPU library against an
 * independent, plain definition.  It shares no code, header, table or helper
 * with the HIP library.
 *
 * What it computes (one "query row" at a time, every step in fp64):
 *
 *   The gist.science technical summary of Parallax, section "Method:
 *   Parallax / core mechanism", gives the output as the standard softmax
 *   attention output minus the KV covariance matrix of query i applied to
 *   the learned probe rho_i:   o_i = o^SA_i - Sigma^(i)_KV rho_i.
 *   The same page, "key design choices", and the news.chathome.org article,
 *   section "How does the mechanism work?", fix the boundary-amplification
 *   factor eta_i to zero, so no other term appears.
 *
 * Readings taken where the pages are silent:
 *   - Sigma^(i)_KV is weighted by query i's softmax weights p_ij (the (i)
 *     superscript makes it query dependent); population form, the weights
 *     sum to one, no Bessel correction.
 *   - Rows of Sigma_KV are indexed by the value coordinate, columns by the
 *     key coordinate, so rho pairs with keys (the probe is "query-like").
 *   - The softmax scale tau multiplies q.k only; rho.k is not scaled.
 *   - A row with an empty context returns 0.
 *
 * Two independently written forms are provided:
 *   form 0 (explicit):  Sigma_KV is built as a d x d matrix from its
 *                       definition and multiplied by rho.
 *   form 1 (expanded):  corr = sum_j p_j r_j v_j - rbar * o^SA with
 *                       r_j = <rho, k_j>, rbar = sum_j p_j r_j; O(L d) per
 *                       row.  Expanding the covariance gives this identity:
 *                       sum_j p_j (v_j - o)(r_j - rbar) = sum_j p_j r_j v_j
 *                       - rbar o.
 * The two share no helper so that a slip in one shows up as a disagreement.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------- */
/* form 0: the covariance matrix written out                                  */
/* ------------------------------------------------------------------------- */

/* One query row, explicit covariance.  K and V hold L keys/values of length
 * d, consecutive keys `stride` doubles apart.  work must hold d*d + 2*d + L
 * doubles.  rho may be NULL (probe of zero). */
static void row_explicit(const double *q, const double *rho, const double *K,
                         const double *V, int64_t stride, int64_t L, int d,
                         double tau, double *out, double *work)
{
    double *sigma = work;              /* d x d, sigma[a*d + b] */
    double *mu_k = sigma + (size_t)d * d;
    double *mu_v = mu_k + d;
    double *p = mu_v + d;              /* L softmax weights */
    int64_t j;
    int a, b;

    if (L == 0) {
        for (a = 0; a < d; ++a) out[a] = 0.0;
        return;
    }

    /* softmax weights of standard attention: p_j = exp(s_j) / sum exp(s) */
    double smax = -INFINITY;
    for (j = 0; j < L; ++j) {
        const double *kj = K + j * stride;
        double s = 0.0;
        for (a = 0; a < d; ++a) s += q[a] * kj[a];
        s *= tau;
        p[j] = s;
        if (s > smax) smax = s;
    }
    double z = 0.0;
    for (j = 0; j < L; ++j) {
        p[j] = exp(p[j] - smax);
        z += p[j];
    }
    for (j = 0; j < L; ++j) p[j] /= z;

    /* weighted means of keys and values; mu_v is the softmax output o^SA */
    for (a = 0; a < d; ++a) { mu_k[a] = 0.0; mu_v[a] = 0.0; }
    for (j = 0; j < L; ++j) {
        const double *kj = K + j * stride;
        const double *vj = V + j * stride;
        for (a = 0; a < d; ++a) {
            mu_k[a] += p[j] * kj[a];
            mu_v[a] += p[j] * vj[a];
        }
    }

    /* Sigma_KV[a][b] = sum_j p_j (v_j[a] - mu_v[a]) (k_j[b] - mu_k[b]) */
    memset(sigma, 0, sizeof(double) * (size_t)d * d);
    for (j = 0; j < L; ++j) {
        const double *kj = K + j * stride;
        const double *vj = V + j * stride;
        for (a = 0; a < d; ++a) {
            double dv = p[j] * (vj[a] - mu_v[a]);
            for (b = 0; b < d; ++b) sigma[(size_t)a * d + b] += dv * (kj[b] - mu_k[b]);
        }
    }

    /* o = o^SA - Sigma_KV rho   (eta = 0: nothing else is added) */
    for (a = 0; a < d; ++a) {
        double corr = 0.0;
        if (rho)
            for (b = 0; b < d; ++b) corr += sigma[(size_t)a * d + b] * rho[b];
        out[a] = mu_v[a] - corr;
    }
}

/* ------------------------------------------------------------------------- */
/* form 1: the expanded, O(L d) form                                          */
/* ------------------------------------------------------------------------- */

/* work must hold 2*L + 2*d doubles. */
static void row_expanded(const double *q, const double *rho, const double *K,
                         const double *V, int64_t stride, int64_t L, int d,
                         double tau, double *out, double *work)
{
    double *w = work;          /* L unnormalised weights */
    double *r = w + L;         /* L probe scores <rho, k_j> */
    double *osa = r + L;       /* d */
    double *prv = osa + d;     /* d: sum_j p_j r_j v_j */
    int64_t j;
    int a;

    if (L == 0) {
        for (a = 0; a < d; ++a) out[a] = 0.0;
        return;
    }

    double m = -INFINITY;
    for (j = 0; j < L; ++j) {
        const double *kj = K + j * stride;
        double qk = 0.0, rk = 0.0;
        for (a = 0; a < d; ++a) {
            qk += q[a] * kj[a];
            if (rho) rk += rho[a] * kj[a];
        }
        w[j] = tau * qk;
        r[j] = rk;
        if (w[j] > m) m = w[j];
    }
    double total = 0.0;
    for (j = 0; j < L; ++j) {
        w[j] = exp(w[j] - m);
        total += w[j];
    }

    double rbar = 0.0;
    for (a = 0; a < d; ++a) { osa[a] = 0.0; prv[a] = 0.0; }
    for (j = 0; j < L; ++j) {
        const double *vj = V + j * stride;
        double pj = w[j] / total;
        rbar += pj * r[j];
        for (a = 0; a < d; ++a) {
            osa[a] += pj * vj[a];
            prv[a] += pj * r[j] * vj[a];
        }
    }
    for (a = 0; a < d; ++a) out[a] = osa[a] - (prv[a] - rbar * osa[a]);
}

/* ------------------------------------------------------------------------- */
/* exported entry points                                                      */
/* ------------------------------------------------------------------------- */

/* Evaluate n_rows independent query rows.
 *   q, rho      [n_rows, d] (rho may be NULL)
 *   k, v        base pointers; row i reads key_len[i] keys starting at
 *               element key_off[i], consecutive keys key_stride elements apart
 *   form        0 = explicit covariance, 1 = expanded
 *   out         [n_rows, d]
 * Returns 0 on success, -1 on a bad argument, -2 if scratch memory fails. */
int plx_oracle_rows(const double *q, const double *rho, const double *k,
                    const double *v, const int64_t *key_off,
                    const int64_t *key_len, int64_t key_stride, int64_t n_rows,
                    int32_t d, double tau, int32_t form, double *out)
{
    if (!q || !k || !v || !key_off || !key_len || !out) return -1;
    if (d <= 0 || n_rows < 0 || (form != 0 && form != 1)) return -1;
    int64_t max_len = 0;
    for (int64_t i = 0; i < n_rows; ++i) {
        if (key_len[i] < 0 || key_off[i] < 0) return -1;
        if (key_len[i] > max_len) max_len = key_len[i];
    }
    size_t work_n = form == 0 ? (size_t)d * d + 2 * (size_t)d + (size_t)max_len
                              : 2 * (size_t)max_len + 2 * (size_t)d;
    int failed = 0;

#pragma omp parallel
    {
        double *work = (double *)malloc(sizeof(double) * (work_n + 1));
        if (!work) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < n_rows; ++i) {
            if (!work) continue;
            const double *qi = q + i * d;
            const double *ri = rho ? rho + i * d : NULL;
            const double *ki = k + key_off[i];
            const double *vi = v + key_off[i];
            if (form == 0)
                row_explicit(qi, ri, ki, vi, key_stride, key_len[i], d, tau, out + i * d, work);
            else
                row_expanded(qi, ri, ki, vi, key_stride, key_len[i], d, tau, out + i * d, work);
        }
        free(work);
    }
    return failed ? -2 : 0;
}

/* Number of threads plx_oracle_rows runs with (for reporting). */
int plx_oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set the thread count used by plx_oracle_rows (n <= 0 leaves it alone). */
void plx_oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
