/*
 * Selective-scan oracle: plain, slow, sequential, fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may call this code.  It shares nothing with the HIP library
 * (no headers, helpers or tables) and must never be on the product path.
 *
 * What it computes (one channel d of one batch row b at a time, t ascending):
 *
 *   Delta_t = softplus(delta[b,t,d] + bias[d])
 *       softplus applied once, to the projection plus its bias: "Understanding
 *       Mamba" (aiattnstudio.link), section 2.3, and the forward pass of
 *       "State Space Models and Mamba" (metaphor-xennon.pages.dev), which adds
 *       the dt_proj bias inside the softplus.
 *   Abar_t[n] = exp(Delta_t * A[d,n]),   Bbar_t[n] = Delta_t * B[b,t,n]
 *       the diagonal discretisation the pages' selective_scan code uses
 *       ("Understanding Mamba" section 4.4 steps 1-2 and section 5.2
 *       _selective_scan; metaphor-xennon selective_scan).
 *   h_t[n] = Abar_t[n] * h_{t-1}[n] + Bbar_t[n] * u[b,t,d]
 *       the recurrence h_t = Abar_t h_{t-1} + Bbar_t x_t (hnwysp.cn slides,
 *       sections 2.1 and 3.1); h_{-1} = h0[b,d,:] or 0.
 *   y[b,t,d] = sum_n C[b,t,n] h_t[n] + D[d] u[b,t,d]
 *       readout from the updated state (einsum 'bdn,bn->bd' of the
 *       metaphor-xennon selective_scan) plus the skip term y = C x + D u
 *       ("Understanding Mamba" section 12, "Mamba output").
 *   y[b,t,d] *= silu(z[b,t,d])          if z is given
 *       the gate y * silu(z) applied after the scan (MambaBlock.forward,
 *       "Understanding Mamba" section 5.2).
 *   h_last[b,d,:] = h_{L-1}
 *
 * Readings taken where the pages disagree or are silent: softplus is applied
 * exactly once; Bbar is the Euler form Delta*B used by all of the pages' code,
 * and on request (zoh != 0) the zero-order hold of their equations,
 * Bbar = A^-1 (exp(Delta A) - I) B ("Understanding Mamba" section 12; "State
 * Space Models and Mamba", ZOH), i.e. (exp(Delta A[d,n]) - 1) / A[d,n] * B[n] for
 * the diagonal A, with the A -> 0 limit Delta*B; y_t reads the state
 * after the update with u_t; D*u uses the raw u and is added before the gate;
 * a missing D, bias or h0 means zero and a missing z means no gate.  All
 * arithmetic is double precision with libm exp/log1p and nothing is rounded to
 * a storage type; compile without -ffast-math.  Threads split the independent
 * (b, d) channels only, so the result does not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

/* softplus(x) = log(1 + e^x), evaluated without overflow or cancellation. */
double oracle_softplus(double x)
{
    if (x > 0.0)
        return x + log1p(exp(-x));
    return log1p(exp(x));
}

/* silu(z) = z * sigmoid(z) = z / (1 + e^-z). */
double oracle_silu(double z)
{
    return z / (1.0 + exp(-z));
}

typedef struct {
    const double *u, *delta, *A, *B, *C, *D, *z, *bias, *h0;
    double *y, *h_last;
    int64_t batch, L, Dn, N;
    int64_t chan_begin, chan_end; /* channel index c = b * Dn + d */
    int zoh;
} scan_job;

/* Bbar[n] for step size dt, state coefficient a = A[d,n] and input coefficient b = B[n]:
 * Euler dt * b, or the zero-order hold (exp(dt a) - 1) / a * b (limit dt * b at a = 0). */
static double oracle_bbar(double dt, double a, double b, int zoh)
{
    if (!zoh || a == 0.0)
        return dt * b;
    return expm1(dt * a) / a * b;
}

static void scan_channels(const scan_job *j)
{
    const int64_t L = j->L, Dn = j->Dn, N = j->N;
    double *h = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
    for (int64_t c = j->chan_begin; c < j->chan_end; ++c) {
        const int64_t b = c / Dn, d = c % Dn;
        for (int64_t n = 0; n < N; ++n)
            h[n] = j->h0 ? j->h0[(b * Dn + d) * N + n] : 0.0;

        for (int64_t t = 0; t < L; ++t) {
            const int64_t bld = (b * L + t) * Dn + d; /* (B, L, D) layout */
            const int64_t bln = (b * L + t) * N;      /* (B, L, N) layout */
            const double ut = j->u[bld];

            /* step size */
            const double dt = oracle_softplus(j->delta[bld] + (j->bias ? j->bias[d] : 0.0));

            /* discretise and advance the state */
            for (int64_t n = 0; n < N; ++n) {
                const double abar = exp(dt * j->A[d * N + n]);
                const double bbar = oracle_bbar(dt, j->A[d * N + n], j->B[bln + n], j->zoh);
                h[n] = abar * h[n] + bbar * ut;
            }

            /* readout, skip term, gate */
            double yt = 0.0;
            for (int64_t n = 0; n < N; ++n)
                yt += j->C[bln + n] * h[n];
            yt += (j->D ? j->D[d] : 0.0) * ut;
            if (j->z)
                yt *= oracle_silu(j->z[bld]);
            j->y[bld] = yt;
        }

        if (j->h_last)
            for (int64_t n = 0; n < N; ++n)
                j->h_last[(b * Dn + d) * N + n] = h[n];
    }
    free(h);
}

static void *scan_thread(void *arg)
{
    scan_channels((const scan_job *)arg);
    return NULL;
}

/*
 * Full scan over (batch, L, d_inner) with state size d_state.
 * Layouts (row-major, last index fastest): u, delta, z, y: (batch, L, d_inner);
 * B, C: (batch, L, d_state); A: (d_inner, d_state); D, bias: (d_inner);
 * h0, h_last: (batch, d_inner, d_state).  D, z, bias, h0 and h_last may be NULL.
 * zoh selects the zero-order-hold Bbar instead of Euler's.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_scan(const double *u, const double *delta, const double *A, const double *B,
                const double *C, const double *D, const double *z, const double *bias,
                const double *h0, double *y, double *h_last, int64_t batch, int64_t L,
                int64_t d_inner, int64_t d_state, int nthreads, int zoh)
{
    if (batch < 0 || L < 0 || d_inner < 0 || d_state < 0)
        return -1;
    if ((L > 0 && (!u || !delta || !B || !C || !y)) || (d_state > 0 && !A))
        return -1;
    const int64_t chans = batch * d_inner;
    if (L == 0) { /* nothing to scan: the final state is the initial state */
        if (h_last)
            for (int64_t i = 0; i < chans * d_state; ++i)
                h_last[i] = h0 ? h0[i] : 0.0;
        return 0;
    }
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > chans)
        nthreads = (int)(chans > 0 ? chans : 1);

    scan_job *jobs = (scan_job *)calloc((size_t)nthreads, sizeof(scan_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    for (int i = 0; i < nthreads; ++i) {
        scan_job *j = &jobs[i];
        j->u = u; j->delta = delta; j->A = A; j->B = B; j->C = C;
        j->D = D; j->z = z; j->bias = bias; j->h0 = h0; j->y = y; j->h_last = h_last;
        j->batch = batch; j->L = L; j->Dn = d_inner; j->N = d_state;
        j->chan_begin = chans * i / nthreads;
        j->chan_end = chans * (i + 1) / nthreads;
        j->zoh = zoh;
    }
    for (int i = 1; i < nthreads; ++i)
        pthread_create(&tids[i], NULL, scan_thread, &jobs[i]);
    scan_channels(&jobs[0]);
    for (int i = 1; i < nthreads; ++i)
        pthread_join(tids[i], NULL);
    free(tids);
    free(jobs);
    return 0;
}

/*
 * One recurrent decode step: the body of the time loop above, once, for every
 * (b, d), with the state carried by the caller ("output, h = ssm(token, h)" in
 * the MambaDecoder loop of metaphor-xennon).
 * h: (batch, d_inner, d_state), updated in place.  u, delta, z, y: (batch, d_inner);
 * B, C: (batch, d_state).
 */
int oracle_step(double *h, const double *u, const double *delta, const double *A,
                const double *B, const double *C, const double *D, const double *z,
                const double *bias, double *y, int64_t batch, int64_t d_inner, int64_t d_state,
                int zoh)
{
    if (!h || !u || !delta || !A || !B || !C || !y || batch < 0 || d_inner < 0 || d_state < 0)
        return -1;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < d_inner; ++d) {
            const int64_t bd = b * d_inner + d;
            double *hb = h + bd * d_state;
            const double ut = u[bd];
            const double dt = oracle_softplus(delta[bd] + (bias ? bias[d] : 0.0));
            for (int64_t n = 0; n < d_state; ++n) {
                const double abar = exp(dt * A[d * d_state + n]);
                const double bbar = oracle_bbar(dt, A[d * d_state + n], B[b * d_state + n], zoh);
                hb[n] = abar * hb[n] + bbar * ut;
            }
            double yt = 0.0;
            for (int64_t n = 0; n < d_state; ++n)
                yt += C[b * d_state + n] * hb[n];
            yt += (D ? D[d] : 0.0) * ut;
            if (z)
                yt *= oracle_silu(z[bd]);
            y[bd] = yt;
        }
    }
    return 0;
}
