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
 * a missing D, bias or h0 means zero and a missing z means no gate.
 *
 * Two further options of the Mamba-3 section of "State space models and the Mamba
 * series" (jsqmd.com), sections 2.1 and 2.2, taken as the page writes them:
 *   - exponential-trapezoidal rule (lam given): the input term is
 *       (1 - lam_t) Delta_t B_{t-1}[n] u_{t-1} + lam_t Delta_t B_t[n] u_t
 *     with the data-dependent mixing coefficient lam[b,t,d] in [0,1], and the input
 *     before t = 0 taken from u_prev[b,d], B_prev[b,:] (zero when not given).  The page
 *     writes the look-back term without a decay factor; that is what is computed.
 *   - data-dependent rotation (theta given): h_t = exp(Delta_t A) R(Delta_t theta_t)
 *     h_{t-1} + (input term), R the 2x2 rotation [[cos, -sin], [sin, cos]] acting on
 *     each state pair (2k, 2k+1) with the angle Delta_t * theta[b,t,k]; the rotation
 *     is applied before the decay, as the product exp(Delta A) R is written.
 * All
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
    const double *lam, *u_prev, *B_prev, *theta; /* trapezoid, rotation (NULL: off) */
    double *y, *h_last;
    int64_t batch, L, Dn, N;
    int64_t chan_begin, chan_end; /* channel index c = b * Dn + d */
    int zoh;
} scan_job;

/* Rotate each state pair (2k, 2k+1) by dt * theta[k]: [[cos, -sin], [sin, cos]]. */
static void oracle_rotate(double *h, const double *theta, double dt, int64_t N)
{
    for (int64_t k = 0; k < N / 2; ++k) {
        const double phi = dt * theta[k];
        const double c = cos(phi), s = sin(phi);
        const double x = h[2 * k], w = h[2 * k + 1];
        h[2 * k] = c * x - s * w;
        h[2 * k + 1] = s * x + c * w;
    }
}

/* Exponential-trapezoidal input term of one state index: (1 - lam) dt b_prev u_prev +
 * lam dt b u. */
static double oracle_trap_input(double lam, double dt, double b, double u, double b_prev,
                                double u_prev)
{
    return (1.0 - lam) * dt * b_prev * u_prev + lam * dt * b * u;
}

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
        /* the input of the step before t = 0 (trapezoidal look-back) */
        double u_lb = j->u_prev ? j->u_prev[b * Dn + d] : 0.0;
        const double *B_lb = j->B_prev ? j->B_prev + b * N : NULL;

        for (int64_t t = 0; t < L; ++t) {
            const int64_t bld = (b * L + t) * Dn + d; /* (B, L, D) layout */
            const int64_t bln = (b * L + t) * N;      /* (B, L, N) layout */
            const double ut = j->u[bld];

            /* step size */
            const double dt = oracle_softplus(j->delta[bld] + (j->bias ? j->bias[d] : 0.0));

            /* data-dependent rotation of the previous state, before its decay */
            if (j->theta)
                oracle_rotate(h, j->theta + (b * j->L + t) * (N / 2), dt, N);

            /* discretise and advance the state */
            for (int64_t n = 0; n < N; ++n) {
                const double abar = exp(dt * j->A[d * N + n]);
                const double bbar = oracle_bbar(dt, j->A[d * N + n], j->B[bln + n], j->zoh);
                if (j->lam)
                    h[n] = abar * h[n] + oracle_trap_input(j->lam[bld], dt, j->B[bln + n], ut,
                                                           B_lb ? B_lb[n] : 0.0, u_lb);
                else
                    h[n] = abar * h[n] + bbar * ut;
            }
            u_lb = ut;
            B_lb = j->B + bln;

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
int oracle_scan_ext(const double *u, const double *delta, const double *A, const double *B,
                    const double *C, const double *D, const double *z, const double *bias,
                    const double *h0, double *y, double *h_last, int64_t batch, int64_t L,
                    int64_t d_inner, int64_t d_state, int nthreads, int zoh, const double *lam,
                    const double *u_prev, const double *B_prev, const double *theta)
{
    if (batch < 0 || L < 0 || d_inner < 0 || d_state < 0)
        return -1;
    if ((theta && d_state % 2 != 0) || (lam && zoh))
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
        j->lam = lam; j->u_prev = u_prev; j->B_prev = B_prev; j->theta = theta;
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

/* The scan without the trapezoid and rotation options. */
int oracle_scan(const double *u, const double *delta, const double *A, const double *B,
                const double *C, const double *D, const double *z, const double *bias,
                const double *h0, double *y, double *h_last, int64_t batch, int64_t L,
                int64_t d_inner, int64_t d_state, int nthreads, int zoh)
{
    return oracle_scan_ext(u, delta, A, B, C, D, z, bias, h0, y, h_last, batch, L, d_inner,
                           d_state, nthreads, zoh, NULL, NULL, NULL, NULL);
}

/*
 * One recurrent decode step: the body of the time loop above, once, for every
 * (b, d), with the state carried by the caller ("output, h = ssm(token, h)" in
 * the MambaDecoder loop of metaphor-xennon).
 * h: (batch, d_inner, d_state), updated in place.  u, delta, z, y: (batch, d_inner);
 * B, C: (batch, d_state).
 */
int oracle_step_ext(double *h, const double *u, const double *delta, const double *A,
                    const double *B, const double *C, const double *D, const double *z,
                    const double *bias, double *y, int64_t batch, int64_t d_inner,
                    int64_t d_state, int zoh, const double *lam, const double *u_prev,
                    const double *B_prev, const double *theta)
{
    if (!h || !u || !delta || !A || !B || !C || !y || batch < 0 || d_inner < 0 || d_state < 0)
        return -1;
    if ((theta && d_state % 2 != 0) || (lam && zoh))
        return -1;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < d_inner; ++d) {
            const int64_t bd = b * d_inner + d;
            double *hb = h + bd * d_state;
            const double ut = u[bd];
            const double dt = oracle_softplus(delta[bd] + (bias ? bias[d] : 0.0));
            if (theta)
                oracle_rotate(hb, theta + b * (d_state / 2), dt, d_state);
            for (int64_t n = 0; n < d_state; ++n) {
                const double abar = exp(dt * A[d * d_state + n]);
                const double bbar = oracle_bbar(dt, A[d * d_state + n], B[b * d_state + n], zoh);
                if (lam)
                    hb[n] = abar * hb[n] +
                            oracle_trap_input(lam[bd], dt, B[b * d_state + n], ut,
                                              B_prev ? B_prev[b * d_state + n] : 0.0,
                                              u_prev ? u_prev[bd] : 0.0);
                else
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

/* The decode step without the trapezoid and rotation options. */
int oracle_step(double *h, const double *u, const double *delta, const double *A,
                const double *B, const double *C, const double *D, const double *z,
                const double *bias, double *y, int64_t batch, int64_t d_inner, int64_t d_state,
                int zoh)
{
    return oracle_step_ext(h, u, delta, A, B, C, D, z, bias, y, batch, d_inner, d_state, zoh,
                           NULL, NULL, NULL, NULL);
}

/*
 * Gradients of the scan (Euler discretisation), for a loss whose derivatives with
 * respect to the outputs are dy (batch, L, d_inner) and, optionally, dh_last
 * (batch, d_inner, d_state).  Reverse-mode differentiation of the loop above, written
 * out by hand: with mu_t[n] = dLoss/dh_t[n] (total), s_t = sum_n C_t h_t + D u_t,
 * g_t = silu(z_t), ds_t = dy_t g_t,
 *     mu_{L-1} = dh_last + ds_{L-1} C_{L-1};  mu_t = Abar_{t+1} mu_{t+1} + ds_t C_t
 *     dDelta_t = sum_n mu_t[n] (A[n] Abar_t[n] h_{t-1}[n] + B_t[n] u_t)
 *     du_t     = ds_t D + sum_n mu_t[n] Delta_t B_t[n]
 *     dB_t[n]  = sum_d mu_t[n] Delta_t u_t        dC_t[n] = sum_d ds_t h_t[n]
 *     dA[d,n]  = sum_{b,t} mu_t[n] Delta_t Abar_t[n] h_{t-1}[n]
 *     dD[d]    = sum_{b,t} ds_t u_t               dz_t = dy_t s_t silu'(z_t)
 *     ddelta_t = dDelta_t sigmoid(delta_t + bias)  (softplus' = sigmoid)
 *     dbias[d] = sum_{b,t} ddelta_t               dh0 = Abar_0 mu_0
 * The pages name the backward pass (recompute instead of storing the states, "Understanding
 * Mamba" section 7.3; the hnwysp.cn slides, section 4.4) but do not write it out; this is
 * the chain rule applied to the forward definition above, pinned by finite differences.
 * Outputs other than du and ddelta may be NULL.  Threads split the batch rows; the sums
 * over b are added in b order, so the result does not depend on the thread count.
 */
typedef struct {
    const double *u, *delta, *A, *B, *C, *D, *z, *bias, *h0, *dy, *dh_last;
    double *du, *ddelta, *dB, *dC, *dz, *dh0;
    double *dA_part, *dD_part, *dbias_part; /* per batch row: [b][d][n], [b][d], [b][d] */
    int64_t batch, L, Dn, N;
    int64_t b_begin, b_end;
} bwd_job;

static void bwd_rows(const bwd_job *j)
{
    const int64_t L = j->L, Dn = j->Dn, N = j->N;
    double *hs = (double *)malloc((size_t)((L + 1) * N > 0 ? (L + 1) * N : 1) * sizeof(double));
    double *mu = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
    for (int64_t b = j->b_begin; b < j->b_end; ++b) {
        if (j->dB)
            for (int64_t i = 0; i < L * N; ++i)
                j->dB[b * L * N + i] = 0.0;
        if (j->dC)
            for (int64_t i = 0; i < L * N; ++i)
                j->dC[b * L * N + i] = 0.0;
        for (int64_t d = 0; d < Dn; ++d) {
            /* forward: hs[(t + 1) * N + n] = h_t[n], hs[n] = h_{-1}[n] */
            for (int64_t n = 0; n < N; ++n)
                hs[n] = j->h0 ? j->h0[(b * Dn + d) * N + n] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                const int64_t bld = (b * L + t) * Dn + d, bln = (b * L + t) * N;
                const double dt = oracle_softplus(j->delta[bld] + (j->bias ? j->bias[d] : 0.0));
                for (int64_t n = 0; n < N; ++n)
                    hs[(t + 1) * N + n] = exp(dt * j->A[d * N + n]) * hs[t * N + n] +
                                          dt * j->B[bln + n] * j->u[bld];
            }
            /* reverse */
            for (int64_t n = 0; n < N; ++n)
                mu[n] = j->dh_last ? j->dh_last[(b * Dn + d) * N + n] : 0.0;
            double dD_acc = 0.0, dbias_acc = 0.0;
            for (int64_t t = L - 1; t >= 0; --t) {
                const int64_t bld = (b * L + t) * Dn + d, bln = (b * L + t) * N;
                const double v = j->delta[bld] + (j->bias ? j->bias[d] : 0.0);
                const double dt = oracle_softplus(v);
                const double ut = j->u[bld];
                double s = (j->D ? j->D[d] : 0.0) * ut;
                for (int64_t n = 0; n < N; ++n)
                    s += j->C[bln + n] * hs[(t + 1) * N + n];
                double gate = 1.0, dgate = 0.0;
                if (j->z) {
                    const double zt = j->z[bld];
                    const double sig = 1.0 / (1.0 + exp(-zt));
                    gate = zt * sig;
                    dgate = sig * (1.0 + zt * (1.0 - sig));
                }
                const double ds = j->dy[bld] * gate;
                if (j->dz)
                    j->dz[bld] = j->z ? j->dy[bld] * s * dgate : 0.0;
                double ddt = 0.0, du = ds * (j->D ? j->D[d] : 0.0);
                for (int64_t n = 0; n < N; ++n) {
                    mu[n] += ds * j->C[bln + n];                 /* mu_t */
                    const double a = j->A[d * N + n];
                    const double abar = exp(dt * a);
                    const double hprev = hs[t * N + n];
                    ddt += mu[n] * (a * abar * hprev + j->B[bln + n] * ut);
                    du += mu[n] * dt * j->B[bln + n];
                    if (j->dB)
                        j->dB[bln + n] += mu[n] * dt * ut;
                    if (j->dC)
                        j->dC[bln + n] += ds * hs[(t + 1) * N + n];
                    if (j->dA_part)
                        j->dA_part[(b * Dn + d) * N + n] += mu[n] * dt * abar * hprev;
                    mu[n] *= abar;                               /* Abar_t mu_t, for t - 1 */
                }
                dD_acc += ds * ut;
                const double dv = ddt / (1.0 + exp(-v));         /* softplus'(v) = sigmoid(v) */
                j->du[bld] = du;
                j->ddelta[bld] = dv;
                dbias_acc += dv;
            }
            if (j->dh0)
                for (int64_t n = 0; n < N; ++n)
                    j->dh0[(b * Dn + d) * N + n] = mu[n];        /* = Abar_0 mu_0 */
            if (j->dD_part)
                j->dD_part[b * Dn + d] = dD_acc;
            if (j->dbias_part)
                j->dbias_part[b * Dn + d] = dbias_acc;
        }
    }
    free(mu);
    free(hs);
}

static void *bwd_thread(void *arg)
{
    bwd_rows((const bwd_job *)arg);
    return NULL;
}

int oracle_scan_bwd(const double *u, const double *delta, const double *A, const double *B,
                    const double *C, const double *D, const double *z, const double *bias,
                    const double *h0, const double *dy, const double *dh_last, double *du,
                    double *ddelta, double *dA, double *dB, double *dC, double *dD, double *dz,
                    double *dbias, double *dh0, int64_t batch, int64_t L, int64_t d_inner,
                    int64_t d_state, int nthreads)
{
    if (batch < 0 || L < 0 || d_inner < 0 || d_state < 0 || !A)
        return -1;
    if (L > 0 && (!u || !delta || !B || !C || !dy || !du || !ddelta))
        return -1;
    const int64_t Dn = d_inner, N = d_state;
    double *dA_part = (double *)calloc((size_t)(batch * Dn * N > 0 ? batch * Dn * N : 1), sizeof(double));
    double *dD_part = (double *)calloc((size_t)(batch * Dn > 0 ? batch * Dn : 1), sizeof(double));
    double *dbias_part = (double *)calloc((size_t)(batch * Dn > 0 ? batch * Dn : 1), sizeof(double));
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > batch)
        nthreads = (int)(batch > 0 ? batch : 1);
    bwd_job *jobs = (bwd_job *)calloc((size_t)nthreads, sizeof(bwd_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    for (int i = 0; i < nthreads; ++i) {
        bwd_job *j = &jobs[i];
        j->u = u; j->delta = delta; j->A = A; j->B = B; j->C = C; j->D = D; j->z = z;
        j->bias = bias; j->h0 = h0; j->dy = dy; j->dh_last = dh_last;
        j->du = du; j->ddelta = ddelta; j->dB = dB; j->dC = dC; j->dz = dz; j->dh0 = dh0;
        j->dA_part = dA_part; j->dD_part = dD_part; j->dbias_part = dbias_part;
        j->batch = batch; j->L = L; j->Dn = Dn; j->N = N;
        j->b_begin = batch * i / nthreads;
        j->b_end = batch * (i + 1) / nthreads;
    }
    if (L > 0) {
        for (int i = 1; i < nthreads; ++i)
            pthread_create(&tids[i], NULL, bwd_thread, &jobs[i]);
        bwd_rows(&jobs[0]);
        for (int i = 1; i < nthreads; ++i)
            pthread_join(tids[i], NULL);
    } else if (dh0) { /* nothing happened: the initial state's gradient is dh_last */
        for (int64_t i = 0; i < batch * Dn * N; ++i)
            dh0[i] = dh_last ? dh_last[i] : 0.0;
    }
    /* sums over the batch, in b order */
    if (dA)
        for (int64_t i = 0; i < Dn * N; ++i) {
            double s = 0.0;
            for (int64_t b = 0; b < batch; ++b)
                s += dA_part[b * Dn * N + i];
            dA[i] = s;
        }
    if (dD || dbias)
        for (int64_t d = 0; d < Dn; ++d) {
            double sD = 0.0, sb = 0.0;
            for (int64_t b = 0; b < batch; ++b) {
                sD += dD_part[b * Dn + d];
                sb += dbias_part[b * Dn + d];
            }
            if (dD)
                dD[d] = sD;
            if (dbias)
                dbias[d] = sb;
        }
    free(tids);
    free(jobs);
    free(dbias_part);
    free(dD_part);
    free(dA_part);
    return 0;
}

/*
 * Gradients of the scan with the zero-order hold (zoh), the exponential-trapezoidal rule
 * (lam, u_prev, B_prev) and the rotation (theta) -- the forward definition at the top of
 * this file with those options -- for the loss with derivatives dy and dh_last.  The chain
 * rule through each step, written out by hand (the pages give the forward rules only:
 * "Understanding Mamba" section 12 for the zero-order hold, "State space models and the
 * Mamba series" sections 2.1 and 2.2 for the other two).  Per step, with h' the previous
 * state after the rotation and before the decay, a = exp(Delta A), mu = dLoss/dh_t:
 *     dLoss/dh'      = a mu,     dLoss/dh_{t-1} = R^T (a mu)       (R the step's rotation)
 *     dDelta        += sum_n mu A a h'  + (input term)'_Delta  + sum_k theta_k dphi_k
 *     dA[n]         += mu Delta a h'    + (input term)'_A
 * where dphi_k = dLoss/dphi_k = (a mu)_{2k+1} h'_{2k} - (a mu)_{2k} h'_{2k+1} for the pair
 * angle phi_k = Delta theta_k (dR/dphi h' = the pair turned by a further quarter turn), and
 * the input term is Delta B u (Euler), beta B u with beta = expm1(Delta A) / A (zero-order
 * hold: d beta / dDelta = a, d beta / dA = (Delta a - beta) / A, Delta^2 / 2 at A = 0), or
 * (1 - lam) Delta B_{t-1} u_{t-1} + lam Delta B u (trapezoid: its first part also sends
 * gradient to u_{t-1} and B_{t-1} -- to u_prev and B_prev at t = 0 -- and
 * dlam = sum_n mu Delta (B u - B_{t-1} u_{t-1})).  Outputs as oracle_scan_bwd plus dlam
 * (batch, L, d_inner), du_prev (batch, d_inner), dB_prev (batch, d_state), dtheta
 * (batch, L, d_state / 2); each of those may be NULL and is written when its option is on.
 * Sums over channels (dB, dC, dB_prev, dtheta) and over batch rows are taken in index order.
 */
typedef struct {
    const double *u, *delta, *A, *B, *C, *D, *z, *bias, *h0, *dy, *dh_last;
    const double *lam, *u_prev, *B_prev, *theta;
    double *du, *ddelta, *dB, *dC, *dz, *dh0, *dlam, *du_prev, *dB_prev, *dtheta;
    double *dA_part, *dD_part, *dbias_part;
    int64_t batch, L, Dn, N;
    int64_t b_begin, b_end;
    int zoh;
} bwd_ext_job;

static void bwd_ext_rows(const bwd_ext_job *j)
{
    const int64_t L = j->L, Dn = j->Dn, N = j->N, K = N / 2;
    const size_t nn = (size_t)(N > 0 ? N : 1);
    double *hs = (double *)malloc((size_t)(L + 1) * nn * sizeof(double));  /* h_t at t + 1 */
    double *hpre = (double *)malloc((size_t)(L > 0 ? L : 1) * nn * sizeof(double)); /* h' */
    double *mu = (double *)malloc(nn * sizeof(double));
    double *nu = (double *)malloc(nn * sizeof(double));
    double *lbk = (double *)malloc(nn * sizeof(double)); /* trapezoid look-back weights */
    for (int64_t b = j->b_begin; b < j->b_end; ++b) {
        if (j->dB)
            for (int64_t i = 0; i < L * N; ++i)
                j->dB[b * L * N + i] = 0.0;
        if (j->dC)
            for (int64_t i = 0; i < L * N; ++i)
                j->dC[b * L * N + i] = 0.0;
        if (j->dtheta && j->theta)
            for (int64_t i = 0; i < L * K; ++i)
                j->dtheta[b * L * K + i] = 0.0;
        if (j->dB_prev && j->lam)
            for (int64_t n = 0; n < N; ++n)
                j->dB_prev[b * N + n] = 0.0;
        for (int64_t d = 0; d < Dn; ++d) {
            const double bias = j->bias ? j->bias[d] : 0.0;
            const double u_pre = j->u_prev ? j->u_prev[b * Dn + d] : 0.0;
            /* forward, keeping h' and h_t of every step */
            for (int64_t n = 0; n < N; ++n)
                hs[n] = j->h0 ? j->h0[(b * Dn + d) * N + n] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                const int64_t bld = (b * L + t) * Dn + d, bln = (b * L + t) * N;
                const double dt = oracle_softplus(j->delta[bld] + bias);
                double *hp = hpre + t * N;
                for (int64_t n = 0; n < N; ++n)
                    hp[n] = hs[t * N + n];
                if (j->theta)
                    oracle_rotate(hp, j->theta + (b * L + t) * K, dt, N);
                for (int64_t n = 0; n < N; ++n) {
                    const double a = j->A[d * N + n];
                    double in;
                    if (j->lam) {
                        const double bp = t > 0 ? j->B[bln - N + n]
                                                : (j->B_prev ? j->B_prev[b * N + n] : 0.0);
                        const double up = t > 0 ? j->u[bld - Dn] : u_pre;
                        in = oracle_trap_input(j->lam[bld], dt, j->B[bln + n], j->u[bld], bp, up);
                    } else {
                        in = oracle_bbar(dt, a, j->B[bln + n], j->zoh) * j->u[bld];
                    }
                    hs[(t + 1) * N + n] = exp(dt * a) * hp[n] + in;
                }
            }
            /* reverse */
            for (int64_t n = 0; n < N; ++n) {
                mu[n] = j->dh_last ? j->dh_last[(b * Dn + d) * N + n] : 0.0;
                lbk[n] = 0.0;
            }
            double dD_acc = 0.0, dbias_acc = 0.0;
            for (int64_t t = L - 1; t >= 0; --t) {
                const int64_t bld = (b * L + t) * Dn + d, bln = (b * L + t) * N;
                const double v = j->delta[bld] + bias;
                const double dt = oracle_softplus(v);
                const double ut = j->u[bld];
                double s = (j->D ? j->D[d] : 0.0) * ut;
                for (int64_t n = 0; n < N; ++n)
                    s += j->C[bln + n] * hs[(t + 1) * N + n];
                double gate = 1.0, dgate = 0.0;
                if (j->z) {
                    const double zt = j->z[bld];
                    const double sig = 1.0 / (1.0 + exp(-zt));
                    gate = zt * sig;
                    dgate = sig * (1.0 + zt * (1.0 - sig));
                }
                const double ds = j->dy[bld] * gate;
                if (j->dz)
                    j->dz[bld] = j->z ? j->dy[bld] * s * dgate : 0.0;
                double ddt = 0.0, du = ds * (j->D ? j->D[d] : 0.0), dl = 0.0;
                const double lam = j->lam ? j->lam[bld] : 0.0;
                const double up = t > 0 ? j->u[bld - Dn] : u_pre;
                for (int64_t n = 0; n < N; ++n) {
                    const double Bn = j->B[bln + n];
                    /* step t + 1's look-back term read u_t and B_t */
                    if (j->lam) {
                        du += lbk[n] * Bn;
                        if (j->dB)
                            j->dB[bln + n] += lbk[n] * ut;
                    }
                    mu[n] += ds * j->C[bln + n];                 /* mu_t */
                    const double a = j->A[d * N + n];
                    const double abar = exp(dt * a);
                    const double hp = hpre[t * N + n];
                    ddt += mu[n] * a * abar * hp;
                    double dAn = mu[n] * dt * abar * hp;
                    if (j->lam) {
                        const double bp = t > 0 ? j->B[bln - N + n]
                                                : (j->B_prev ? j->B_prev[b * N + n] : 0.0);
                        ddt += mu[n] * ((1.0 - lam) * bp * up + lam * Bn * ut);
                        du += mu[n] * lam * dt * Bn;
                        if (j->dB)
                            j->dB[bln + n] += mu[n] * lam * dt * ut;
                        dl += mu[n] * dt * (Bn * ut - bp * up);
                        lbk[n] = mu[n] * (1.0 - lam) * dt;       /* for step t - 1 */
                    } else if (j->zoh) {
                        const double beta = a != 0.0 ? expm1(dt * a) / a : dt;
                        ddt += mu[n] * Bn * ut * abar;
                        du += mu[n] * beta * Bn;
                        if (j->dB)
                            j->dB[bln + n] += mu[n] * beta * ut;
                        dAn += mu[n] * Bn * ut * (a != 0.0 ? (dt * abar - beta) / a
                                                           : 0.5 * dt * dt);
                    } else {
                        ddt += mu[n] * Bn * ut;
                        du += mu[n] * dt * Bn;
                        if (j->dB)
                            j->dB[bln + n] += mu[n] * dt * ut;
                    }
                    if (j->dC)
                        j->dC[bln + n] += ds * hs[(t + 1) * N + n];
                    if (j->dA_part)
                        j->dA_part[(b * Dn + d) * N + n] += dAn;
                    nu[n] = abar * mu[n];                        /* dLoss/dh' */
                }
                if (j->theta) {
                    const double *th = j->theta + (b * L + t) * K;
                    for (int64_t k = 0; k < K; ++k) {
                        const double *hp = hpre + t * N + 2 * k;
                        const double dphi = nu[2 * k + 1] * hp[0] - nu[2 * k] * hp[1];
                        ddt += th[k] * dphi;
                        if (j->dtheta)
                            j->dtheta[(b * L + t) * K + k] += dt * dphi;
                        const double phi = dt * th[k], c = cos(phi), sn = sin(phi);
                        mu[2 * k] = c * nu[2 * k] + sn * nu[2 * k + 1];       /* R^T nu */
                        mu[2 * k + 1] = -sn * nu[2 * k] + c * nu[2 * k + 1];
                    }
                } else {
                    for (int64_t n = 0; n < N; ++n)
                        mu[n] = nu[n];
                }
                dD_acc += ds * ut;
                const double dv = ddt / (1.0 + exp(-v));
                j->du[bld] = du;
                j->ddelta[bld] = dv;
                if (j->dlam && j->lam)
                    j->dlam[bld] = dl;
                dbias_acc += dv;
            }
            /* the trapezoid's first look-back read u_prev and B_prev */
            if (j->lam) {
                double dup = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double bp = j->B_prev ? j->B_prev[b * N + n] : 0.0;
                    dup += lbk[n] * bp;
                    if (j->dB_prev)
                        j->dB_prev[b * N + n] += lbk[n] * u_pre;
                }
                if (j->du_prev)
                    j->du_prev[b * Dn + d] = dup;
            }
            if (j->dh0)
                for (int64_t n = 0; n < N; ++n)
                    j->dh0[(b * Dn + d) * N + n] = mu[n];
            if (j->dD_part)
                j->dD_part[b * Dn + d] = dD_acc;
            if (j->dbias_part)
                j->dbias_part[b * Dn + d] = dbias_acc;
        }
    }
    free(lbk);
    free(nu);
    free(mu);
    free(hpre);
    free(hs);
}

static void *bwd_ext_thread(void *arg)
{
    bwd_ext_rows((const bwd_ext_job *)arg);
    return NULL;
}

int oracle_scan_bwd_ext(const double *u, const double *delta, const double *A, const double *B,
                        const double *C, const double *D, const double *z, const double *bias,
                        const double *h0, const double *dy, const double *dh_last, int zoh,
                        const double *lam, const double *u_prev, const double *B_prev,
                        const double *theta, double *du, double *ddelta, double *dA,
                        double *dB, double *dC, double *dD, double *dz, double *dbias,
                        double *dh0, double *dlam, double *du_prev, double *dB_prev,
                        double *dtheta, int64_t batch, int64_t L, int64_t d_inner,
                        int64_t d_state, int nthreads)
{
    if (batch < 0 || L < 0 || d_inner < 0 || d_state < 0 || !A)
        return -1;
    if ((theta && d_state % 2 != 0) || (lam && zoh))
        return -1;
    if (L > 0 && (!u || !delta || !B || !C || !dy || !du || !ddelta))
        return -1;
    const int64_t Dn = d_inner, N = d_state;
    double *dA_part = (double *)calloc((size_t)(batch * Dn * N > 0 ? batch * Dn * N : 1), sizeof(double));
    double *dD_part = (double *)calloc((size_t)(batch * Dn > 0 ? batch * Dn : 1), sizeof(double));
    double *dbias_part = (double *)calloc((size_t)(batch * Dn > 0 ? batch * Dn : 1), sizeof(double));
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > batch)
        nthreads = (int)(batch > 0 ? batch : 1);
    bwd_ext_job *jobs = (bwd_ext_job *)calloc((size_t)nthreads, sizeof(bwd_ext_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    for (int i = 0; i < nthreads; ++i) {
        bwd_ext_job *j = &jobs[i];
        j->u = u; j->delta = delta; j->A = A; j->B = B; j->C = C; j->D = D; j->z = z;
        j->bias = bias; j->h0 = h0; j->dy = dy; j->dh_last = dh_last;
        j->lam = lam; j->u_prev = u_prev; j->B_prev = B_prev; j->theta = theta;
        j->du = du; j->ddelta = ddelta; j->dB = dB; j->dC = dC; j->dz = dz; j->dh0 = dh0;
        j->dlam = dlam; j->du_prev = du_prev; j->dB_prev = dB_prev; j->dtheta = dtheta;
        j->dA_part = dA_part; j->dD_part = dD_part; j->dbias_part = dbias_part;
        j->batch = batch; j->L = L; j->Dn = Dn; j->N = N;
        j->b_begin = batch * i / nthreads;
        j->b_end = batch * (i + 1) / nthreads;
        j->zoh = zoh;
    }
    if (L > 0) {
        for (int i = 1; i < nthreads; ++i)
            pthread_create(&tids[i], NULL, bwd_ext_thread, &jobs[i]);
        bwd_ext_rows(&jobs[0]);
        for (int i = 1; i < nthreads; ++i)
            pthread_join(tids[i], NULL);
    } else {
        if (dh0)
            for (int64_t i = 0; i < batch * Dn * N; ++i)
                dh0[i] = dh_last ? dh_last[i] : 0.0;
        if (lam && du_prev)
            for (int64_t i = 0; i < batch * Dn; ++i)
                du_prev[i] = 0.0;
        if (lam && dB_prev)
            for (int64_t i = 0; i < batch * N; ++i)
                dB_prev[i] = 0.0;
    }
    if (dA)
        for (int64_t i = 0; i < Dn * N; ++i) {
            double s = 0.0;
            for (int64_t b = 0; b < batch; ++b)
                s += dA_part[b * Dn * N + i];
            dA[i] = s;
        }
    if (dD || dbias)
        for (int64_t d = 0; d < Dn; ++d) {
            double sD = 0.0, sb = 0.0;
            for (int64_t b = 0; b < batch; ++b) {
                sD += dD_part[b * Dn + d];
                sb += dbias_part[b * Dn + d];
            }
            if (dD)
                dD[d] = sD;
            if (dbias)
                dbias[d] = sb;
        }
    free(tids);
    free(jobs);
    free(dbias_part);
    free(dD_part);
    free(dA_part);
    return 0;
}
