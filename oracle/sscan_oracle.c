/*
 * sscan_oracle.c -- plain, sequential fp64 oracle of the selective scan (S6).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code with the HIP path.
 *
 * What it computes, per batch b, channel d and direction (all arithmetic in fp64,
 * inputs widened exactly from their stored dtype by the caller):
 *
 *   dt_t  = softplus(delta_t + bias_d)  if softplus, else delta_t + bias_d
 *           (Hand-written simplified Mamba2 page, sections 4.2 and 4.4: the step
 *            size comes out of a biased projection followed by softplus)
 *   h_n   = 0 (or h0 when given)        (same page, section 4.3: state starts at zero)
 *   for t = 0..L-1 (forward) or t = L-1..0 (reverse):
 *     h_n <- exp(dt_t * A[d,n]) * h_n + dt_t * B[b,n,t] * u_t
 *           (same page, section 2.2: zero-order hold gives Abar = exp(dt*A); the
 *            Mamba family keeps the first-order input matrix Bbar = dt*B)
 *     y_t += sum_n C[b,n,t] * h_n + D_d * u_t
 *           (same page, section 2.2 output equation and section 4.4 skip term)
 *   bidirectional: y_t = y_t(forward params) + y_t(reverse params)
 *           (Reproducing Vision Mamba page, section 3.2: scan, flip, scan with the
 *            second parameter set, flip back, add)
 *   out_t = y_t * silu(z_t), silu(x) = x / (1 + exp(-x))  (z == NULL: out = y)
 *           (Hand-written simplified Mamba2 page, section 4.4 gate)
 *
 * The state is carried across the whole sequence: the chunk-local reset of the
 * teaching code in section 4.4 of the Mamba2 page is, by that page's own remark,
 * a simplification and not the method.
 *
 * Layouts (row-major, contiguous): u, delta, z, out: [batch, dim, len];
 * B, C: [batch, dstate, len]; A: [dim, dstate]; D, bias: [dim]; h0, h_last:
 * [batch, dim, dstate].  Rows (b, d) are independent; with nthreads > 1 they are
 * split over POSIX threads, each row still strictly sequential in t.
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* softplus(x) = log(1 + e^x), written in the overflow-free exact form
 * max(x, 0) + log1p(exp(-|x|)); no threshold. */
static double oracle_softplus(double x) {
    if (isnan(x)) return x;
    return fmax(x, 0.0) + log1p(exp(-fabs(x)));
}

static double oracle_silu(double x) { return x / (1.0 + exp(-x)); }

typedef struct {
    const double* delta;
    const double* delta_bias; /* nullable: 0 */
    const double* A;
    const double* B;
    const double* C;
    const double* D; /* nullable: 0 */
    int reverse;
} dir_params;

typedef struct {
    const double* u;
    const double* z; /* nullable: no gate */
    double* out;
    const dir_params* dirs;
    int ndir;
    int softplus;
    int64_t batch, dim, len, dstate;
    const double* h0;  /* nullable, only with ndir == 1 */
    double* h_last;    /* nullable, only with ndir == 1 */
    int64_t row_begin, row_end;
    int status;
} job;

/* One (b, d) row, one direction: accumulates scan + D*u into y[0..len). */
static int scan_row(const job* jb, const dir_params* p, int64_t b, int64_t d, double* y) {
    const int64_t L = jb->len, N = jb->dstate;
    const double* u = jb->u + (b * jb->dim + d) * L;
    const double* dl = p->delta + (b * jb->dim + d) * L;
    const double* A = p->A + d * N;
    const double* Bm = p->B + b * N * L;
    const double* Cm = p->C + b * N * L;
    const double bias = p->delta_bias ? p->delta_bias[d] : 0.0;
    const double Dd = p->D ? p->D[d] : 0.0;
    double* h = (double*)malloc(sizeof(double) * (size_t)N);
    if (!h) return -1;
    for (int64_t n = 0; n < N; ++n)
        h[n] = jb->h0 ? jb->h0[(b * jb->dim + d) * N + n] : 0.0;
    for (int64_t k = 0; k < L; ++k) {
        const int64_t t = p->reverse ? L - 1 - k : k;
        const double x = dl[t] + bias;
        const double dt = jb->softplus ? oracle_softplus(x) : x;
        double s = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            h[n] = exp(dt * A[n]) * h[n] + dt * Bm[n * L + t] * u[t];
            s += Cm[n * L + t] * h[n];
        }
        y[t] += s + Dd * u[t];
    }
    if (jb->h_last)
        for (int64_t n = 0; n < N; ++n) jb->h_last[(b * jb->dim + d) * N + n] = h[n];
    free(h);
    return 0;
}

static void* run_rows(void* arg) {
    job* jb = (job*)arg;
    const int64_t L = jb->len;
    for (int64_t r = jb->row_begin; r < jb->row_end; ++r) {
        const int64_t b = r / jb->dim, d = r % jb->dim;
        double* y = jb->out + r * L;
        for (int64_t t = 0; t < L; ++t) y[t] = 0.0;
        for (int k = 0; k < jb->ndir; ++k)
            if (scan_row(jb, &jb->dirs[k], b, d, y) != 0) { jb->status = -1; return NULL; }
        if (jb->z) {
            const double* z = jb->z + r * L;
            for (int64_t t = 0; t < L; ++t) y[t] *= oracle_silu(z[t]);
        }
    }
    return NULL;
}

static int run(job proto, int nthreads) {
    const int64_t rows = proto.batch * proto.dim;
    if (proto.batch < 0 || proto.dim < 0 || proto.len < 0 || proto.dstate < 0) return -2;
    /* with no tokens the rows still run: each copies its entry state to h_last */
    if (rows == 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > rows) nthreads = (int)rows;
    job* jobs = (job*)calloc((size_t)nthreads, sizeof(job));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return -1; }
    int status = 0;
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = proto;
        jobs[i].row_begin = rows * i / nthreads;
        jobs[i].row_end = rows * (i + 1) / nthreads;
        jobs[i].status = 0;
    }
    if (nthreads == 1) {
        run_rows(&jobs[0]);
    } else {
        int started = 0;
        for (; started < nthreads; ++started)
            if (pthread_create(&th[started], NULL, run_rows, &jobs[started]) != 0) break;
        for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
        for (int i = started; i < nthreads; ++i) run_rows(&jobs[i]);
    }
    for (int i = 0; i < nthreads; ++i)
        if (jobs[i].status) status = jobs[i].status;
    free(jobs);
    free(th);
    return status;
}

/* Single direction.  h0 / h_last (nullable) are the state before the first
 * processed token and after the last one, [batch, dim, dstate]. */
int oracle_sscan_fwd(const double* u, const double* delta, const double* delta_bias, int softplus,
                     const double* A, const double* B, const double* C, const double* D,
                     const double* z, double* out, int64_t batch, int64_t dim, int64_t len,
                     int64_t dstate, int reverse, const double* h0, double* h_last, int nthreads) {
    dir_params p = {delta, delta_bias, A, B, C, D, reverse};
    job jb;
    memset(&jb, 0, sizeof(jb));
    jb.u = u; jb.z = z; jb.out = out; jb.dirs = &p; jb.ndir = 1; jb.softplus = softplus;
    jb.batch = batch; jb.dim = dim; jb.len = len; jb.dstate = dstate;
    jb.h0 = h0; jb.h_last = h_last;
    return run(jb, nthreads);
}

/* Both directions with separate parameter sets, summed, then gated once. */
int oracle_sscan_bidir(const double* u, const double* z, double* out,
                       const double* delta_f, const double* bias_f, const double* A_f,
                       const double* B_f, const double* C_f, const double* D_f,
                       const double* delta_r, const double* bias_r, const double* A_r,
                       const double* B_r, const double* C_r, const double* D_r,
                       int softplus, int64_t batch, int64_t dim, int64_t len, int64_t dstate,
                       int nthreads) {
    dir_params p[2] = {{delta_f, bias_f, A_f, B_f, C_f, D_f, 0},
                       {delta_r, bias_r, A_r, B_r, C_r, D_r, 1}};
    job jb;
    memset(&jb, 0, sizeof(jb));
    jb.u = u; jb.z = z; jb.out = out; jb.dirs = p; jb.ndir = 2; jb.softplus = softplus;
    jb.batch = batch; jb.dim = dim; jb.len = len; jb.dstate = dstate;
    return run(jb, nthreads);
}

/* Exposed for the tests of the oracle's own scalar helpers. */
double oracle_softplus_f64(double x) { return oracle_softplus(x); }
double oracle_silu_f64(double x) { return oracle_silu(x); }
