/*
 * sscan_oracle_bwd.c -- plain, sequential fp64 gradients of the selective scan.
 *
 * TEST INFRASTRUCTURE ONLY (see sscan_oracle.c).  Shares no code with the HIP path.
 *
 * The forward computation is the one in sscan_oracle.c (Hand-written simplified
 * Mamba2 page, sections 2.2 and 4.2-4.4; Reproducing Vision Mamba page, section 3.2
 * for the two directions summed before the gate).  Training runs the scan
 * backwards with hand-written gradients and recomputes the forward states instead
 * of storing them (Reproducing Vision Mamba page, section 1.3; Mamba2 page,
 * section 5.1).  Given g = dLoss/dout, this file returns the exact gradients of
 *   out_t = (sum_dir y_t^dir) * silu(z_t)   (or without the gate when z is NULL)
 * with respect to u, z and every direction's delta, delta_bias, A, B, C and D.
 *
 * Derivation (reverse-mode differentiation of the recurrence, written out):
 *   dy_t = g_t * silu(z_t)                         dz_t = g_t * y_t * silu'(z_t)
 *   silu'(x) = s (1 + x (1 - s)), s = 1 / (1 + exp(-x))
 * per direction, with k the position in scan order, t = t_k the token, a_k,n =
 * exp(dt_t A_n), h^k the state after token t_k and h^-1 = 0:
 *   lambda_n = C[n,t] dy_t + mu_n      (mu = a_{k+1} * lambda^{k+1}; mu = 0 after the last)
 *   dC[n,t] += dy_t h^k_n              dB[n,t] += lambda_n dt_t u_t
 *   du_t    += D dy_t + sum_n lambda_n dt_t B[n,t]
 *   ddt     = sum_n lambda_n (B[n,t] u_t + A_n a_k,n h^{k-1}_n)
 *   dA_n    += lambda_n dt_t a_k,n h^{k-1}_n         dD += dy_t u_t
 *   ddelta_t = ddt * sigmoid(delta_t + bias)  (softplus' ; ddt itself without softplus)
 *   dbias   += ddelta_t                      mu_n = a_k,n lambda_n
 * Sums over tokens and batch rows (dA, dD, dbias) and over channels (dB, dC) are
 * accumulated per thread and added in thread order.
 *
 * State I/O (one direction; the forward of sscan_oracle.c with h0 and h_last): the
 * forward sweep starts from h^-1 = h0 instead of 0, so the first token's previous
 * state in dA and ddt is h0; the reverse sweep starts from mu = dLoss/dh_last (the
 * gradient reaching the final state from outside, 0 when absent) instead of 0; and
 * the gradient of the entry state is what the adjoint carries past the first token
 * in scan order:  dh0_n = a_0,n lambda^0_n  (the mu left after the sweep; with no
 * tokens at all, dh0 = dLoss/dh_last, as h_last = h0).
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bwd_softplus(double x) {
    if (isnan(x)) return x;
    return fmax(x, 0.0) + log1p(exp(-fabs(x)));
}

static double bwd_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

enum { IN_DELTA, IN_BIAS, IN_A, IN_B, IN_C, IN_D, N_IN };
enum { OUT_DDELTA, OUT_DBIAS, OUT_DA, OUT_DB, OUT_DC, OUT_DD, N_OUT };

typedef struct {
    const double* u;
    const double* z;
    const double* g;
    double* du;
    double* dz;
    int ndir;
    const double* const* dir_in; /* ndir * N_IN */
    const int* reverse;          /* ndir */
    double* const* dir_out;      /* ndir * N_OUT (each nullable) */
    int softplus;
    int64_t batch, dim, len, dstate;
    int64_t row_begin, row_end;
    /* per-thread accumulators, per direction: dA [dim][N], dD [dim], dbias [dim],
     * and dB, dC for the batch rows this thread touches [nb][N][len] */
    int64_t b_first, nb;
    double* acc;
    const double* h0;       /* nullable, [batch, dim, dstate], one direction only */
    const double* dh_last;  /* nullable, [batch, dim, dstate] */
    double* dh0;            /* nullable, [batch, dim, dstate] */
    int status;
} bwd_job;

static size_t acc_dir_size(const bwd_job* jb) {
    return (size_t)(jb->dim * jb->dstate + 2 * jb->dim + 2 * jb->nb * jb->dstate * jb->len);
}

static void* bwd_rows(void* arg) {
    bwd_job* jb = (bwd_job*)arg;
    const int64_t L = jb->len, N = jb->dstate;
    double* hist = (double*)malloc(sizeof(double) * (size_t)(L * N));
    double* ysum = (double*)malloc(sizeof(double) * (size_t)L);
    double* dy = (double*)malloc(sizeof(double) * (size_t)L);
    double* lam = (double*)malloc(sizeof(double) * (size_t)N);
    double* mu = (double*)malloc(sizeof(double) * (size_t)N);
    double* h = (double*)malloc(sizeof(double) * (size_t)N);
    if (!hist || !ysum || !dy || !lam || !mu || !h) {
        jb->status = -1;
        goto done;
    }
    for (int64_t r = jb->row_begin; r < jb->row_end; ++r) {
        const int64_t b = r / jb->dim, d = r % jb->dim;
        const double* u = jb->u + r * L;
        const double* gg = jb->g + r * L;
        const double* z = jb->z ? jb->z + r * L : NULL;
        double* du = jb->du + r * L;
        for (int64_t t = 0; t < L; ++t) {
            ysum[t] = 0.0;
            du[t] = 0.0;
            dy[t] = z ? gg[t] * z[t] * bwd_sigmoid(z[t]) : gg[t];
        }
        for (int k = 0; k < jb->ndir; ++k) {
            const double* const* in = jb->dir_in + k * N_IN;
            double* const* out = jb->dir_out + k * N_OUT;
            const double* dl = in[IN_DELTA] + r * L;
            const double bias = in[IN_BIAS] ? in[IN_BIAS][d] : 0.0;
            const double* A = in[IN_A] + d * N;
            const double* Bm = in[IN_B] + b * N * L;
            const double* Cm = in[IN_C] + b * N * L;
            const double Dd = in[IN_D] ? in[IN_D][d] : 0.0;
            double* acc = jb->acc + (size_t)k * acc_dir_size(jb);
            double* dA = acc;
            double* dD = dA + jb->dim * N;
            double* dbias = dD + jb->dim;
            double* dB = dbias + jb->dim + (b - jb->b_first) * N * L;
            double* dC = dB + jb->nb * N * L;
            /* forward sweep: states after every token (in scan order) and y */
            const double* h0 = jb->h0 ? jb->h0 + r * N : NULL;
            for (int64_t n = 0; n < N; ++n) h[n] = h0 ? h0[n] : 0.0;
            for (int64_t s = 0; s < L; ++s) {
                const int64_t t = jb->reverse[k] ? L - 1 - s : s;
                const double x = dl[t] + bias;
                const double dt = jb->softplus ? bwd_softplus(x) : x;
                double yv = Dd * u[t];
                for (int64_t n = 0; n < N; ++n) {
                    h[n] = exp(dt * A[n]) * h[n] + dt * Bm[n * L + t] * u[t];
                    hist[s * N + n] = h[n];
                    yv += Cm[n * L + t] * h[n];
                }
                ysum[t] += yv;
            }
            /* reverse sweep */
            for (int64_t n = 0; n < N; ++n) mu[n] = jb->dh_last ? jb->dh_last[r * N + n] : 0.0;
            for (int64_t s = L - 1; s >= 0; --s) {
                const int64_t t = jb->reverse[k] ? L - 1 - s : s;
                const double x = dl[t] + bias;
                const double dt = jb->softplus ? bwd_softplus(x) : x;
                double ddt = 0.0, dus = Dd * dy[t];
                dD[d] += dy[t] * u[t];
                for (int64_t n = 0; n < N; ++n) {
                    const double a = exp(dt * A[n]);
                    const double hprev = s > 0 ? hist[(s - 1) * N + n] : (h0 ? h0[n] : 0.0);
                    lam[n] = Cm[n * L + t] * dy[t] + mu[n];
                    dC[n * L + t] += dy[t] * hist[s * N + n];
                    dB[n * L + t] += lam[n] * dt * u[t];
                    dus += lam[n] * dt * Bm[n * L + t];
                    ddt += lam[n] * (Bm[n * L + t] * u[t] + A[n] * a * hprev);
                    dA[d * N + n] += lam[n] * dt * a * hprev;
                    mu[n] = a * lam[n];
                }
                du[t] += dus;
                const double dd = jb->softplus ? ddt * bwd_sigmoid(x) : ddt;
                if (out[OUT_DDELTA]) out[OUT_DDELTA][r * L + t] = dd;
                dbias[d] += dd;
            }
            if (jb->dh0)
                for (int64_t n = 0; n < N; ++n) jb->dh0[r * N + n] = mu[n];
        }
        if (z && jb->dz) {
            double* dz = jb->dz + r * L;
            for (int64_t t = 0; t < L; ++t) {
                const double sg = bwd_sigmoid(z[t]);
                dz[t] = gg[t] * ysum[t] * sg * (1.0 + z[t] * (1.0 - sg));
            }
        }
    }
done:
    free(hist);
    free(ysum);
    free(dy);
    free(lam);
    free(mu);
    free(h);
    return NULL;
}

/* Gradients of sum(g * out).  dir_in holds, per direction, the pointers delta,
 * delta_bias (nullable), A, B, C, D (nullable); dir_out, per direction, ddelta
 * [batch, dim, len], ddelta_bias [dim], dA [dim, dstate], dB, dC [batch, dstate,
 * len], dD [dim] (each nullable: not returned).  du is required, dz is written
 * only when z is given.  The directions' outputs are their own: when two
 * directions share one delta tensor, its gradient is the sum of the two ddelta. */
int oracle_sscan_bwd_state(const double* u, const double* z, const double* g, double* du, double* dz, int ndir,
                           const double* const* dir_in, const int* reverse, double* const* dir_out, int softplus,
                           int64_t batch, int64_t dim, int64_t len, int64_t dstate, const double* h0,
                           const double* dh_last, double* dh0, int nthreads) {
    if (batch < 0 || dim < 0 || len < 0 || dstate < 0 || ndir < 1 || ndir > 2) return -2;
    if ((h0 || dh_last || dh0) && ndir != 1) return -3;
    const int64_t rows = batch * dim, N = dstate;
    if (dh0 && len == 0) {
        for (int64_t i = 0; i < rows * N; ++i) dh0[i] = dh_last ? dh_last[i] : 0.0;
    }
    for (int k = 0; k < ndir; ++k) {
        double* const* out = dir_out + k * N_OUT;
        if (out[OUT_DBIAS]) memset(out[OUT_DBIAS], 0, sizeof(double) * (size_t)dim);
        if (out[OUT_DA]) memset(out[OUT_DA], 0, sizeof(double) * (size_t)(dim * N));
        if (out[OUT_DD]) memset(out[OUT_DD], 0, sizeof(double) * (size_t)dim);
        if (out[OUT_DB]) memset(out[OUT_DB], 0, sizeof(double) * (size_t)(batch * N * len));
        if (out[OUT_DC]) memset(out[OUT_DC], 0, sizeof(double) * (size_t)(batch * N * len));
    }
    if (rows == 0 || len == 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > rows) nthreads = (int)rows;
    bwd_job* jobs = (bwd_job*)calloc((size_t)nthreads, sizeof(bwd_job));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    int status = 0;
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return -1;
    }
    for (int i = 0; i < nthreads; ++i) {
        bwd_job* jb = &jobs[i];
        jb->u = u; jb->z = z; jb->g = g; jb->du = du; jb->dz = dz; jb->ndir = ndir;
        jb->dir_in = dir_in; jb->reverse = reverse; jb->dir_out = dir_out; jb->softplus = softplus;
        jb->batch = batch; jb->dim = dim; jb->len = len; jb->dstate = dstate;
        jb->h0 = h0; jb->dh_last = dh_last; jb->dh0 = dh0;
        jb->row_begin = rows * i / nthreads;
        jb->row_end = rows * (i + 1) / nthreads;
        if (jb->row_end > jb->row_begin) {
            jb->b_first = jb->row_begin / dim;
            jb->nb = (jb->row_end - 1) / dim - jb->b_first + 1;
        }
        jb->acc = (double*)calloc((size_t)ndir * acc_dir_size(jb) + 1, sizeof(double));
        if (!jb->acc) status = -1;
    }
    if (status == 0) {
        int started = 0;
        for (; started < nthreads; ++started)
            if (pthread_create(&th[started], NULL, bwd_rows, &jobs[started]) != 0) break;
        for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
        for (int i = started; i < nthreads; ++i) bwd_rows(&jobs[i]);
        /* shared sums, in thread order */
        for (int i = 0; i < nthreads && status == 0; ++i) {
            const bwd_job* jb = &jobs[i];
            if (jb->status) status = jb->status;
            for (int k = 0; k < ndir; ++k) {
                double* const* out = dir_out + k * N_OUT;
                const double* acc = jb->acc + (size_t)k * acc_dir_size(jb);
                const double* dA = acc;
                const double* dD = dA + dim * N;
                const double* dbias = dD + dim;
                const double* dB = dbias + dim;
                const double* dC = dB + jb->nb * N * len;
                for (int64_t j = 0; j < dim * N; ++j)
                    if (out[OUT_DA]) out[OUT_DA][j] += dA[j];
                for (int64_t j = 0; j < dim; ++j) {
                    if (out[OUT_DD]) out[OUT_DD][j] += dD[j];
                    if (out[OUT_DBIAS]) out[OUT_DBIAS][j] += dbias[j];
                }
                const int64_t off = jb->b_first * N * len, cnt = jb->nb * N * len;
                for (int64_t j = 0; j < cnt; ++j) {
                    if (out[OUT_DB]) out[OUT_DB][off + j] += dB[j];
                    if (out[OUT_DC]) out[OUT_DC][off + j] += dC[j];
                }
            }
        }
    }
    for (int i = 0; i < nthreads; ++i) free(jobs[i].acc);
    free(jobs);
    free(th);
    return status;
}

/* Without state I/O: the entry state and the final state's gradient are zero. */
int oracle_sscan_bwd(const double* u, const double* z, const double* g, double* du, double* dz, int ndir,
                     const double* const* dir_in, const int* reverse, double* const* dir_out, int softplus,
                     int64_t batch, int64_t dim, int64_t len, int64_t dstate, int nthreads) {
    return oracle_sscan_bwd_state(u, z, g, du, dz, ndir, dir_in, reverse, dir_out, softplus, batch, dim, len, dstate,
                                  NULL, NULL, NULL, nthreads);
}
