/*
 * Causal depthwise convolution + SiLU oracle: plain, sequential, fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may call this code.  It shares nothing with the HIP library
 * (no headers, helpers or tables) and must never be on the product path.
 *
 * What it computes.  The Mamba block runs its inner activations through a
 * depthwise (one filter per channel) nn.Conv1d with kernel size d_conv = K,
 * padding K - 1 and a bias, keeps the first L outputs and applies SiLU before the
 * selective scan ("Understanding Mamba" (aiattnstudio.link), sections 3.2 and
 * 5.2, MambaBlock.__init__ / forward; the same block in "State Space Models and
 * Mamba" (metaphor-xennon.pages.dev), MambaBlock.forward).  nn.Conv1d computes a
 * cross-correlation, out[t] = sum_k w[k] * in_padded[t + k], and keeping the first
 * L outputs of the K - 1 left-padded input makes it causal:
 *
 *   pre[b,t,d] = bias[d] + sum_{k=0}^{K-1} w[d,k] * xe[b, t - (K-1) + k, d]
 *   u[b,t,d]   = silu(pre[b,t,d]) = pre / (1 + exp(-pre))
 *
 * with xe[b,s,d] = x[b,s,d] for s >= 0.  For -(K-1) <= s < 0, xe is the carried
 * state state_in[b, d, (K-1) + s] (the last K - 1 inputs of the previous segment),
 * or 0 without a state, which is the zero padding of nn.Conv1d.  The state after
 * the call is state_out[b,d,j] = xe[b, L - (K-1) + j, d], j = 0 .. K-2.
 *
 * A decode step is the same computation for one token: the window is the state
 * followed by the new input, and the state shifts by one.
 *
 * Readings: the carried state (a need of recurrent decoding, not spelled out on
 * the pages, which only carry the SSM state) holds raw inputs, oldest first;
 * weights are indexed oldest-to-newest over the window as nn.Conv1d does.  All
 * arithmetic is double precision; compile without -ffast-math.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

static double conv_silu(double p)
{
    return p / (1.0 + exp(-p));
}

/* x: (batch, L, D); w: (D, K); bias: (D) or NULL; state_in: (batch, D, K-1) or NULL;
 * pre, u: (batch, L, D); state_out: (batch, D, K-1) or NULL.  Returns 0, or -1 for
 * invalid sizes. */
int oracle_conv1d_silu(const double *x, const double *w, const double *bias,
                       const double *state_in, double *pre, double *u, double *state_out,
                       int64_t batch, int64_t L, int64_t D, int64_t K)
{
    if (batch < 0 || L < 0 || D < 0 || K < 1 || !w || ((batch * L * D) > 0 && (!x || !pre || !u)))
        return -1;
    const int64_t S = K - 1; /* carried inputs per channel */
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < D; ++d) {
            for (int64_t t = 0; t < L; ++t) {
                double acc = bias ? bias[d] : 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    const int64_t s = t - S + k; /* input time of tap k */
                    double v;
                    if (s >= 0)
                        v = x[(b * L + s) * D + d];
                    else
                        v = state_in ? state_in[(b * D + d) * S + (S + s)] : 0.0;
                    acc += w[d * K + k] * v;
                }
                pre[(b * L + t) * D + d] = acc;
                u[(b * L + t) * D + d] = conv_silu(acc);
            }
            if (state_out) {
                for (int64_t j = 0; j < S; ++j) {
                    const int64_t s = L - S + j;
                    double v;
                    if (s >= 0)
                        v = x[(b * L + s) * D + d];
                    else
                        v = state_in ? state_in[(b * D + d) * S + (S + s)] : 0.0;
                    state_out[(b * D + d) * S + j] = v;
                }
            }
        }
    }
    return 0;
}

/* One decode step.  state: (batch, D, K-1), updated in place; x: (batch, D);
 * pre, u: (batch, D). */
int oracle_conv1d_step(double *state, const double *x, const double *w, const double *bias,
                       double *pre, double *u, int64_t batch, int64_t D, int64_t K)
{
    if (batch < 0 || D < 0 || K < 1 || !w || (batch * D > 0 && (!x || !pre || !u)) ||
        (K > 1 && batch * D > 0 && !state))
        return -1;
    const int64_t S = K - 1;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < D; ++d) {
            double *st = state ? state + (b * D + d) * S : NULL;
            const double xn = x[b * D + d];
            double acc = bias ? bias[d] : 0.0;
            for (int64_t k = 0; k < S; ++k)
                acc += w[d * K + k] * st[k];
            acc += w[d * K + S] * xn;
            pre[b * D + d] = acc;
            u[b * D + d] = conv_silu(acc);
            for (int64_t k = 0; k + 1 < S; ++k)
                st[k] = st[k + 1];
            if (S > 0)
                st[S - 1] = xn;
        }
    }
    return 0;
}
