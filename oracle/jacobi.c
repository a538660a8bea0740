/*
 * fp64 one-sided Jacobi (Hestenes) thin SVD -- part of the CPU ORACLE.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
 * its Python binding) includes, links or calls this file; only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg load it.
 *
 * What it computes: the singular value decomposition M = U S V^T that the
 * spectral-correction optimizer takes of the anchor momentum ("Key design 3",
 * spectral-correction optimizer, papernotes.org notes on "Communication-
 * Efficient LLM Adaptation over Decentralized GPU Meshes": SVD of the anchor
 * momentum, U spanning the output-feature column space, V the input-feature
 * row space).  The pages do not say how the SVD is obtained; this is the
 * textbook one-sided Jacobi method (Hestenes 1958; Golub & Van Loan, "Matrix
 * Computations", one-sided Jacobi; Demmel & Veselic 1992), thin, nothing
 * truncated:
 *
 *   A = M if m >= n, else A = M^T; A is K x k with K >= k; V = I_k.
 *   Repeat sweeps.  A sweep visits every column pair (p, q), p < q, once:
 *     alpha = a_p.a_p, beta = a_q.a_q, gamma = a_p.a_q   (fresh for every pair)
 *     skip if alpha == 0, beta == 0 or |gamma| <= tol * sqrt(alpha * beta)
 *     zeta = (beta - alpha) / (2 gamma)
 *     t = sign(zeta) / (|zeta| + sqrt(1 + zeta^2)),  sign(0) = +1
 *     c = 1 / sqrt(1 + t^2),  s = c t
 *     [a_p, a_q] <- [c a_p - s a_q, s a_p + c a_q], same rotation on [v_p, v_q]
 *   Stop after a sweep that rotates nothing; tol = sqrt(K) * 2^-53.
 *   Then s_j = ||a_j||, u_j = a_j / s_j (u_j = 0 when s_j = 0); sort by s
 *   descending (ties by column index).  If A was M^T, U and V swap roles.
 *
 * Pair order: the round-robin ("circle") parallel ordering of Brent & Luk
 * (1985): k' - 1 rounds (k' = k rounded up to even; a dummy column pads odd
 * k) of k'/2 disjoint pairs.  Pairs of one round touch disjoint columns, so
 * they run on separate threads; every pair's arithmetic is independent of
 * the thread count, so results are bitwise identical for any thread count.
 *
 * Dot products use four interleaved partial sums added in a fixed order
 * (a rounding-order choice only).
 */
#define _POSIX_C_SOURCE 200809L
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t K, k, kp;   /* column length, columns, columns rounded up to even */
    double *A;          /* column-major K x k: column j at A + j*K */
    double *V;          /* column-major k x k */
    double tol;
    int max_sweeps;
    int nthreads;
    pthread_barrier_t bar;
    int64_t *rot_count; /* per thread, per sweep */
    int stop;           /* decided by thread 0 between sweeps */
    int sweeps;         /* sweeps executed */
    int converged;
} jac_t;

typedef struct { jac_t *J; int tid; } jarg_t;

static double dot(const double *x, const double *y, int64_t n) {
    double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
    int64_t i = 0;
    for (; i + 4 <= n; i += 4) {
        s0 += x[i] * y[i];
        s1 += x[i + 1] * y[i + 1];
        s2 += x[i + 2] * y[i + 2];
        s3 += x[i + 3] * y[i + 3];
    }
    for (; i < n; ++i) s0 += x[i] * y[i];
    return (s0 + s1) + (s2 + s3);
}

/* alpha = x.x, beta = y.y, gamma = x.y in one pass; each sum has four
 * interleaved partial sums added in the same fixed order as dot(). */
static void gram2(const double *x, const double *y, int64_t n, double *alpha, double *beta,
                  double *gamma) {
    double a0 = 0, a1 = 0, a2 = 0, a3 = 0, b0 = 0, b1 = 0, b2 = 0, b3 = 0;
    double g0 = 0, g1 = 0, g2 = 0, g3 = 0;
    int64_t i = 0;
    for (; i + 4 <= n; i += 4) {
        double x0 = x[i], x1 = x[i + 1], x2 = x[i + 2], x3 = x[i + 3];
        double y0 = y[i], y1 = y[i + 1], y2 = y[i + 2], y3 = y[i + 3];
        a0 += x0 * x0; a1 += x1 * x1; a2 += x2 * x2; a3 += x3 * x3;
        b0 += y0 * y0; b1 += y1 * y1; b2 += y2 * y2; b3 += y3 * y3;
        g0 += x0 * y0; g1 += x1 * y1; g2 += x2 * y2; g3 += x3 * y3;
    }
    for (; i < n; ++i) {
        a0 += x[i] * x[i];
        b0 += y[i] * y[i];
        g0 += x[i] * y[i];
    }
    *alpha = (a0 + a1) + (a2 + a3);
    *beta = (b0 + b1) + (b2 + b3);
    *gamma = (g0 + g1) + (g2 + g3);
}

static void rotate(double *x, double *y, int64_t n, double c, double s) {
    for (int64_t i = 0; i < n; ++i) {
        double a = x[i], b = y[i];
        x[i] = c * a - s * b;
        y[i] = s * a + c * b;
    }
}

/* Round-robin pairing: round r in [0, kp-1), slot i in [0, kp/2). */
static void rr_pair(int64_t kp, int64_t r, int64_t i, int64_t *p, int64_t *q) {
    int64_t n = kp - 1, a, b;
    if (i == 0) {
        a = kp - 1;
        b = r;
    } else {
        a = (r + i) % n;
        b = (r - i + n) % n;
    }
    *p = a < b ? a : b;
    *q = a < b ? b : a;
}

/* One column-pair step; returns 1 if a rotation was applied. */
static int pair_step(jac_t *J, int64_t p, int64_t q) {
    double *ap = J->A + p * J->K, *aq = J->A + q * J->K;
    double alpha, beta, gamma;
    gram2(ap, aq, J->K, &alpha, &beta, &gamma);
    if (alpha == 0.0 || beta == 0.0) return 0;
    if (fabs(gamma) <= J->tol * sqrt(alpha * beta)) return 0;
    double zeta = (beta - alpha) / (2.0 * gamma);
    double t = (zeta >= 0.0 ? 1.0 : -1.0) / (fabs(zeta) + hypot(1.0, zeta));
    double c = 1.0 / sqrt(1.0 + t * t);
    double s = c * t;
    rotate(ap, aq, J->K, c, s);
    rotate(J->V + p * J->k, J->V + q * J->k, J->k, c, s);
    return 1;
}

static void *worker(void *arg) {
    jarg_t *a = (jarg_t *)arg;
    jac_t *J = a->J;
    int tid = a->tid;
    int64_t half = J->kp / 2;
    for (;;) {
        int64_t rots = 0;
        for (int64_t r = 0; r < J->kp - 1; ++r) {
            for (int64_t i = tid; i < half; i += J->nthreads) {
                int64_t p, q;
                rr_pair(J->kp, r, i, &p, &q);
                if (q >= J->k) continue; /* dummy column */
                rots += pair_step(J, p, q);
            }
            pthread_barrier_wait(&J->bar);
        }
        J->rot_count[tid] = rots;
        pthread_barrier_wait(&J->bar);
        if (tid == 0) {
            int64_t tot = 0;
            for (int t = 0; t < J->nthreads; ++t) tot += J->rot_count[t];
            J->sweeps += 1;
            if (tot == 0) {
                J->converged = 1;
                J->stop = 1;
            } else if (J->sweeps >= J->max_sweeps) {
                J->stop = 1;
            }
        }
        pthread_barrier_wait(&J->bar);
        if (J->stop) break;
    }
    return NULL;
}

typedef struct { double s; int64_t j; } sj_t;

static int cmp_sj(const void *x, const void *y) {
    const sj_t *a = (const sj_t *)x, *b = (const sj_t *)y;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->j > b->j) - (a->j < b->j);
}

/*
 * Thin SVD of the m x n row-major matrix M (fp64).
 * Outputs, r = min(m, n): U (m x r, row-major), s (r), V (n x r, row-major).
 * Returns the number of sweeps executed, negated when the sweep cap was hit
 * before a rotation-free sweep, or 0 on allocation failure / bad arguments.
 */
int oracle_jacobi_svd(int64_t m, int64_t n, const double *M, double *U, double *s, double *V,
                      int max_sweeps, int nthreads) {
    if (m <= 0 || n <= 0 || max_sweeps <= 0) return 0;
    if (nthreads < 1) nthreads = 1;
    int trans = m < n;
    int64_t K = trans ? n : m, k = trans ? m : n;
    jac_t J;
    memset(&J, 0, sizeof(J));
    J.K = K;
    J.k = k;
    J.kp = k + (k & 1);
    if (J.kp < 2) J.kp = 2;
    J.tol = sqrt((double)K) * ldexp(1.0, -53);
    J.max_sweeps = max_sweeps;
    J.nthreads = nthreads;
    J.A = (double *)malloc(sizeof(double) * K * k);
    J.V = (double *)calloc((size_t)(k * k), sizeof(double));
    J.rot_count = (int64_t *)calloc((size_t)nthreads, sizeof(int64_t));
    sj_t *ord = (sj_t *)malloc(sizeof(sj_t) * k);
    if (!J.A || !J.V || !J.rot_count || !ord) {
        free(J.A); free(J.V); free(J.rot_count); free(ord);
        return 0;
    }
    /* A column j: for m >= n column j of M; for m < n row j of M. */
    for (int64_t j = 0; j < k; ++j)
        for (int64_t i = 0; i < K; ++i)
            J.A[j * K + i] = trans ? M[j * n + i] : M[i * n + j];
    for (int64_t j = 0; j < k; ++j) J.V[j * k + j] = 1.0;

    if (k > 1) {
        pthread_barrier_init(&J.bar, NULL, (unsigned)nthreads);
        pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
        jarg_t *args = (jarg_t *)malloc(sizeof(jarg_t) * nthreads);
        for (int t = 0; t < nthreads; ++t) {
            args[t].J = &J;
            args[t].tid = t;
            if (t > 0) pthread_create(&th[t], NULL, worker, &args[t]);
        }
        worker(&args[0]);
        for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
        pthread_barrier_destroy(&J.bar);
        free(th);
        free(args);
    } else {
        J.sweeps = 1;
        J.converged = 1;
    }

    for (int64_t j = 0; j < k; ++j) {
        ord[j].s = sqrt(dot(J.A + j * K, J.A + j * K, K));
        ord[j].j = j;
    }
    qsort(ord, (size_t)k, sizeof(sj_t), cmp_sj);

    /* Left factor of A (K x k): columns a_j / s_j.  Right factor: V. */
    double *L = trans ? V : U; /* receives A's left vectors: K x r row-major */
    double *R = trans ? U : V; /* receives A's right vectors: k x r row-major */
    for (int64_t c = 0; c < k; ++c) {
        int64_t j = ord[c].j;
        double sj = ord[c].s;
        s[c] = sj;
        const double *aj = J.A + j * K;
        for (int64_t i = 0; i < K; ++i) L[i * k + c] = sj > 0.0 ? aj[i] / sj : 0.0;
        const double *vj = J.V + j * k;
        for (int64_t i = 0; i < k; ++i) R[i * k + c] = vj[i];
    }
    int sweeps = J.converged ? J.sweeps : -J.sweeps;
    free(J.A); free(J.V); free(J.rot_count); free(ord);
    return sweeps;
}
