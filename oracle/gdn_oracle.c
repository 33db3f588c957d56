/*
 * gdn_oracle.c -- plain, slow, obviously-correct CPU oracle for the gated delta
 * rule.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
 * CPU-baseline leg call it; the GPU library never links or calls it, and it shares
 * no code with the GPU library.
 *
 * What it computes.  The pages ("Optimizing on-device inference for Apple Silicon",
 * section "Qwen creates three distinct workload shapes") describe the Gated DeltaNet
 * layer as a fixed-size recurrent state: a learned gate decides how much of the old
 * state is kept, and a delta update writes the current token in; every token depends
 * on the state left by the previous one.  Written out, per batch b and value head h
 * (which reads query/key head hk = h / (Hv / Hk)), with S a dv x dk matrix:
 *
 *     a_t = exp(g_t)
 *     S_t = a_t * S_{t-1} * (I - beta_t * k_t k_t^T) + beta_t * v_t k_t^T
 *     o_t = S_t q_t                      (the state after the update is read)
 *
 * This file evaluates the update in its expanded rank-1 form, which is the same
 * matrix algebra with the product multiplied out:
 *
 *     u   = S_{t-1} k_t                  (dv-vector)
 *     S_t = a_t S_{t-1} + beta_t (v_t - a_t u) k_t^T
 *
 * Written per state row i this shows that every row S[i,:] evolves on its own
 * (it only needs v_t[i] besides k_t, q_t, a_t, beta_t), so the work is split over
 * (b, h, block of rows) across threads.  Nothing else is reordered: tokens are
 * visited one at a time in order, dot products are summed left to right.
 *
 * Precision.  The pages ("Keep the recurrent state on chip") keep the state and the
 * gate in fp32 because rounding errors accumulate over sequential updates; the oracle
 * goes further and runs in fp64.  Inputs arrive as fp32 arrays holding the exact
 * values the GPU receives (bf16 values are exactly representable in fp32) and are
 * widened to double exactly.  An fp32 twin exists only to measure how large the
 * rounding drift of a single-precision scan is.
 *
 * Normalised variant.  The same pages' section "Reduce intermediate and state traffic"
 * fuses the query/key preparation into the kernels that follow it.  That preparation is
 * read here as per-head L2 normalisation, the form Gated DeltaNet gives q and k:
 *     x <- x / sqrt(sum_j x_j^2 + 1e-6)          (eps keeps a zero vector finite)
 * applied to k_t and q_t in fp64 after widening, before the update above.
 *
 * Layouts (contiguous, row-major):
 *   q, k      [B, T, Hk, dk]      v        [B, T, Hv, dv]
 *   g, beta   [B, T, Hv]          state_in [B, Hv, dv, dk] (NULL = zero state)
 * Outputs are written for a caller-chosen list of (b, h) pairs:
 *   o_sel     [n_sel, T, dv]      s_sel    [n_sel, dv, dk]
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const float *q, *k, *v, *g, *beta;
    const double *state_in;
    const int *sel;        /* n_sel pairs (b, h), flattened */
    int n_sel;
    int B, T, Hk, Hv, dk, dv;
    int rows_per_item;
    int n_items;
    int next_item;         /* guarded by lock */
    pthread_mutex_t lock;
    void *o_sel, *s_sel;   /* double* or float* */
    int use_f32;
    int qk_norm;           /* normalise k_t and q_t first (fp64 scan only) */
} job_t;

#define GDN_ORACLE_NORM_EPS 1e-6

/* x <- x / sqrt(|x|^2 + eps), in place */
static void l2_normalise(double *x, int n)
{
    double ss = 0.0;
    for (int j = 0; j < n; ++j) ss += x[j] * x[j];
    const double inv = 1.0 / sqrt(ss + GDN_ORACLE_NORM_EPS);
    for (int j = 0; j < n; ++j) x[j] *= inv;
}

/* One work item: rows [r0, r1) of the state of pair sel[2*p], sel[2*p+1]. */
static void run_item_f64(job_t *J, int p, int r0, int r1)
{
    const int b = J->sel[2 * p], h = J->sel[2 * p + 1];
    const int T = J->T, Hk = J->Hk, Hv = J->Hv, dk = J->dk, dv = J->dv;
    const int hk = h / (Hv / Hk);
    double *S = (double *)malloc(sizeof(double) * (size_t)dk);
    double *kk = (double *)malloc(sizeof(double) * (size_t)dk);
    double *qq = (double *)malloc(sizeof(double) * (size_t)dk);
    double *o = (double *)J->o_sel + (size_t)p * T * dv;
    double *sout = (double *)J->s_sel + (size_t)p * dv * dk;
    for (int i = r0; i < r1; ++i) {
        /* load row i of the starting state */
        for (int j = 0; j < dk; ++j)
            S[j] = J->state_in ? J->state_in[(((size_t)b * Hv + h) * dv + i) * dk + j] : 0.0;
        for (int t = 0; t < T; ++t) {
            const size_t tok = (size_t)b * T + t;
            const float *kt = J->k + (tok * Hk + hk) * dk;
            const float *qt = J->q + (tok * Hk + hk) * dk;
            const double a = exp((double)J->g[tok * Hv + h]);
            const double bt = (double)J->beta[tok * Hv + h];
            const double vi = (double)J->v[(tok * Hv + h) * dv + i];
            for (int j = 0; j < dk; ++j) { kk[j] = (double)kt[j]; qq[j] = (double)qt[j]; }
            if (J->qk_norm) { l2_normalise(kk, dk); l2_normalise(qq, dk); }
            double u = 0.0;                       /* (S_{t-1} k_t)[i] */
            for (int j = 0; j < dk; ++j) u += S[j] * kk[j];
            const double delta = bt * (vi - a * u);
            double oi = 0.0;                      /* (S_t q_t)[i] */
            for (int j = 0; j < dk; ++j) {
                S[j] = a * S[j] + delta * kk[j];
                oi += S[j] * qq[j];
            }
            o[(size_t)t * dv + i] = oi;
        }
        for (int j = 0; j < dk; ++j) sout[(size_t)i * dk + j] = S[j];
    }
    free(S); free(kk); free(qq);
}

/* Same scan carried out in single precision (only used to size rounding drift). */
static void run_item_f32(job_t *J, int p, int r0, int r1)
{
    const int b = J->sel[2 * p], h = J->sel[2 * p + 1];
    const int T = J->T, Hk = J->Hk, Hv = J->Hv, dk = J->dk, dv = J->dv;
    const int hk = h / (Hv / Hk);
    float *S = (float *)malloc(sizeof(float) * (size_t)dk);
    float *o = (float *)J->o_sel + (size_t)p * T * dv;
    float *sout = (float *)J->s_sel + (size_t)p * dv * dk;
    for (int i = r0; i < r1; ++i) {
        for (int j = 0; j < dk; ++j)
            S[j] = J->state_in ? (float)J->state_in[(((size_t)b * Hv + h) * dv + i) * dk + j] : 0.0f;
        for (int t = 0; t < T; ++t) {
            const size_t tok = (size_t)b * T + t;
            const float *kt = J->k + (tok * Hk + hk) * dk;
            const float *qt = J->q + (tok * Hk + hk) * dk;
            const float a = expf(J->g[tok * Hv + h]);
            const float bt = J->beta[tok * Hv + h];
            const float vi = J->v[(tok * Hv + h) * dv + i];
            float u = 0.0f;
            for (int j = 0; j < dk; ++j) u += S[j] * kt[j];
            const float delta = bt * (vi - a * u);
            float oi = 0.0f;
            for (int j = 0; j < dk; ++j) {
                S[j] = a * S[j] + delta * kt[j];
                oi += S[j] * qt[j];
            }
            o[(size_t)t * dv + i] = oi;
        }
        for (int j = 0; j < dk; ++j) sout[(size_t)i * dk + j] = S[j];
    }
    free(S);
}

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    const int blocks_per_pair = (J->dv + J->rows_per_item - 1) / J->rows_per_item;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        const int it = J->next_item++;
        pthread_mutex_unlock(&J->lock);
        if (it >= J->n_items) break;
        const int p = it / blocks_per_pair;
        const int r0 = (it % blocks_per_pair) * J->rows_per_item;
        int r1 = r0 + J->rows_per_item;
        if (r1 > J->dv) r1 = J->dv;
        if (J->use_f32) run_item_f32(J, p, r0, r1);
        else run_item_f64(J, p, r0, r1);
    }
    return NULL;
}

static int run(job_t *J, int nthreads)
{
    if (J->B < 0 || J->T < 0 || J->Hk <= 0 || J->Hv <= 0 || J->dk <= 0 || J->dv <= 0) return 1;
    if (J->Hv % J->Hk != 0) return 2;
    for (int p = 0; p < J->n_sel; ++p) {
        if (J->sel[2 * p] < 0 || J->sel[2 * p] >= J->B) return 3;
        if (J->sel[2 * p + 1] < 0 || J->sel[2 * p + 1] >= J->Hv) return 3;
    }
    if (nthreads < 1) nthreads = 1;
    if (J->rows_per_item < 1) J->rows_per_item = 1;
    J->n_items = J->n_sel * ((J->dv + J->rows_per_item - 1) / J->rows_per_item);
    J->next_item = 0;
    pthread_mutex_init(&J->lock, NULL);
    if (nthreads == 1) {
        worker(J);
    } else {
        pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
        int started = 0;
        for (int i = 0; i < nthreads; ++i)
            if (pthread_create(&th[i], NULL, worker, J) == 0) ++started;
        if (started == 0) worker(J);
        for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
        free(th);
    }
    pthread_mutex_destroy(&J->lock);
    return 0;
}

/* fp64 sequential scan.  Returns 0 on success, nonzero on bad arguments. */
int gdn_oracle_seq_f64(const float *q, const float *k, const float *v, const float *g,
                       const float *beta, const double *state_in, const int *sel, int n_sel,
                       double *o_sel, double *s_sel, int B, int T, int Hk, int Hv, int dk,
                       int dv, int nthreads, int rows_per_item)
{
    job_t J;
    memset(&J, 0, sizeof(J));
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.state_in = state_in;
    J.sel = sel; J.n_sel = n_sel; J.o_sel = o_sel; J.s_sel = s_sel;
    J.B = B; J.T = T; J.Hk = Hk; J.Hv = Hv; J.dk = dk; J.dv = dv;
    J.rows_per_item = rows_per_item; J.use_f32 = 0;
    return run(&J, nthreads);
}

/* fp64 sequential scan with q_t and k_t L2-normalised first (see the header). */
int gdn_oracle_seq_f64_qknorm(const float *q, const float *k, const float *v, const float *g,
                              const float *beta, const double *state_in, const int *sel,
                              int n_sel, double *o_sel, double *s_sel, int B, int T, int Hk,
                              int Hv, int dk, int dv, int nthreads, int rows_per_item)
{
    job_t J;
    memset(&J, 0, sizeof(J));
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.state_in = state_in;
    J.sel = sel; J.n_sel = n_sel; J.o_sel = o_sel; J.s_sel = s_sel;
    J.B = B; J.T = T; J.Hk = Hk; J.Hv = Hv; J.dk = dk; J.dv = dv;
    J.rows_per_item = rows_per_item; J.use_f32 = 0; J.qk_norm = 1;
    return run(&J, nthreads);
}

/* fp32 twin of the same scan (rounding-drift yardstick only). */
int gdn_oracle_seq_f32(const float *q, const float *k, const float *v, const float *g,
                       const float *beta, const double *state_in, const int *sel, int n_sel,
                       float *o_sel, float *s_sel, int B, int T, int Hk, int Hv, int dk,
                       int dv, int nthreads, int rows_per_item)
{
    job_t J;
    memset(&J, 0, sizeof(J));
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.state_in = state_in;
    J.sel = sel; J.n_sel = n_sel; J.o_sel = o_sel; J.s_sel = s_sel;
    J.B = B; J.T = T; J.Hk = Hk; J.Hv = Hv; J.dk = dk; J.dv = dv;
    J.rows_per_item = rows_per_item; J.use_f32 = 1;
    return run(&J, nthreads);
}
