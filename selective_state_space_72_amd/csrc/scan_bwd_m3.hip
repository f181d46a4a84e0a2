// Backward pass of the scan with the options of the Mamba-3 section of "State space models
// and the Mamba series" (jsqmd.com, sections 2.1 and 2.2): the exponential-trapezoidal input
// term (1 - lam) Delta B_{t-1} u_{t-1} + lam Delta B u and the rotation of each state pair by
// Delta theta before the decay, either of them also with the zero-order hold where the
// forward allows it (rotation), and the Euler or zero-order-hold input term otherwise.
//
// The chain rule through one step (h' the previous state after the rotation, a = exp(Delta
// A), mu = dLoss/dh_t, nu = a mu):
//   dLoss/dh_{t-1} = R^T nu;   dDelta = sum_n (mu A a h' + mu (input term)'_Delta)
//                                       + sum_k theta_k dphi_k,
//   dphi_k = nu_{2k+1} h'_{2k} - nu_{2k} h'_{2k+1} (the pair's angle phi_k = Delta theta_k),
//   dtheta_k = Delta dphi_k (summed over channels),  dA += mu Delta a h' + mu (input)'_A,
// and the trapezoid's look-back part sends mu_t (1 - lam_t) Delta_t to u_{t-1}, B_{t-1} (to
// u_prev, B_prev at t = 0) with dlam_t = sum_n mu Delta (B_t u_t - B_{t-1} u_{t-1}).
//
// Work decomposition: one lane per channel holding all d_state states (the look-back and the
// pair rotation stay inside a lane, no cross-wave sums), one wave per (batch row, 64-channel
// tile).  The wave runs the forward once storing the state every 8 steps, then walks the
// 8-step segments backwards; within a segment, sub-segments of S steps (the states of S
// steps fit the registers) are recomputed from the stored state and their adjoint run.
// Sums over the tile's channels (dB, dC, dtheta) go through an LDS slab (a row per value,
// one lane per channel; each lane then adds one row) into per-tile partials, which a
// second kernel adds in tile order.  This is the correctness-first path of these options:
// a wave per 64 channels gives the large prefill 640 waves (less than one per SIMD).
#include <type_traits>

#include "device_math.h"
#include "scan_common.h"
#include "scan_bwd.h"

namespace mambascan {
namespace {

constexpr int kM3Seg = 8; // steps between stored states

struct M3Args {
    const void *u, *delta, *z, *dy, *B, *C, *lam, *u_prev, *B_prev, *theta;
    const float *A, *D, *bias, *h0, *dh_last;
    void *du, *ddelta, *dz, *dlam, *du_prev;
    float *dh0;
    float *ckpt;       // [unit][segment][n][lane]
    float *part;       // [unit][t][V]: the tile's sums of dB, dC (and dtheta)
    float *bprev_part; // [unit][N]: the tile's sums of dB_prev
    float *dA_part;    // [b][d][n]
    float *dDb_part;   // [b][d][2]: dD, dbias
    int64_t L;
    int32_t Dn, batch, n_seg;
};

template <typename T, int N, bool ZOH, bool TRAP, bool ROT, bool GATED>
__global__ void __launch_bounds__(64) scan_bwd_m3_kernel(M3Args p)
{
    static_assert(!(ZOH && TRAP), "the trapezoid replaces the input term");
    constexpr int S = N <= 16 ? 4 : 2; // steps whose states are kept in registers
    constexpr int SG = kM3Seg / S;      // sub-segments per stored state
    constexpr int K = N / 2;
    constexpr int V = 2 * N + (ROT ? K : 0); // values summed over channels per step
    constexpr int kRow = 68;                 // slab row: 64 lanes + 16 bytes
    __shared__ __attribute__((aligned(16))) float s_v[V > N ? V : N][kRow];

    const int lane = threadIdx.x;
    const int unit = blockIdx.x; // tile * batch + b
    const int b = unit % p.batch, tile = unit / p.batch;
    const int Dn = p.Dn;
    const int d = tile * 64 + lane;
    const bool dvalid = d < Dn;
    const int dc = dvalid ? d : Dn - 1; // tail lanes compute on a valid channel with dy = 0
    const int64_t L = p.L;
    const int64_t row0 = (int64_t)b * L;
    auto ld = [](const void *base, int64_t i) { return load_val((const T *)base, i); };

    float a2[N], an[N], ia[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const float av = p.A[(int64_t)dc * N + n];
        a2[n] = av * kLog2e;
        an[n] = av;
        ia[n] = ZOH ? 1.0f / av : 0.0f;
    }
    const float bias_d = p.bias ? p.bias[dc] : 0.0f;
    const float D_d = p.D ? p.D[dc] : 0.0f;
    const float u_pre = TRAP && p.u_prev ? ld(p.u_prev, (int64_t)b * Dn + dc) : 0.0f;

    // the look-back input (u, B) of step t: the previous step's, or (u_prev, B_prev)
    auto lookback = [&](int64_t t, float &u_lb, float (&b_lb)[N]) {
        if constexpr (TRAP) {
            if (t > 0) {
                u_lb = ld(p.u, (row0 + t - 1) * Dn + dc);
#pragma unroll
                for (int n = 0; n < N; ++n)
                    b_lb[n] = ld(p.B, (row0 + t - 1) * N + n);
            } else {
                u_lb = u_pre;
#pragma unroll
                for (int n = 0; n < N; ++n)
                    b_lb[n] = p.B_prev ? ld(p.B_prev, (int64_t)b * N + n) : 0.0f;
            }
        }
    };
    // one forward step: rotation, decay, input term; the look-back advances to step t
    auto advance = [&](float (&h)[N], int64_t t, float &u_lb, float (&b_lb)[N]) {
        const int64_t bld = (row0 + t) * Dn + dc;
        const float uu = ld(p.u, bld);
        const float dl = softplus_f(ld(p.delta, bld) + bias_d);
        if constexpr (ROT) {
#pragma unroll
            for (int k = 0; k < K; ++k)
                rotate_pair(dl * ld(p.theta, (row0 + t) * K + k), h[2 * k], h[2 * k + 1]);
        }
        const float lm = TRAP ? ld(p.lam, bld) : 0.0f;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const float bn = ld(p.B, (row0 + t) * N + n);
            const float a = decay_exp2(dl, a2[n]);
            float in;
            if constexpr (TRAP)
                in = __builtin_fmaf((1.0f - lm) * dl * u_lb, b_lb[n], lm * dl * uu * bn);
            else if constexpr (ZOH)
                in = zoh_input(dl * an[n], a, dl * uu, uu * ia[n]) * bn;
            else
                in = dl * uu * bn;
            h[n] = __builtin_fmaf(a, h[n], in);
            if constexpr (TRAP)
                b_lb[n] = bn;
        }
        if constexpr (TRAP)
            u_lb = uu;
    };
    // sums over the 64 lanes of NR values per lane (vals), written by lanes < NR to dst[row]
    // (fixed order)
    auto lane_sums = [&](auto NR_, const float (&vals)[decltype(NR_)::value], float *dst) {
        constexpr int NR = decltype(NR_)::value;
#pragma unroll
        for (int r = 0; r < NR; ++r)
            s_v[r][lane] = vals[r];
        for (int r = lane; r < NR; r += 64) {
            const float4 *src = reinterpret_cast<const float4 *>(&s_v[r][0]);
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float4 c = src[i];
                s += (c.x + c.y) + (c.z + c.w);
            }
            dst[r] = s;
        }
    };

    float *ck = p.ckpt + (int64_t)unit * p.n_seg * N * 64;

    // ---- 1. forward: the state entering every 8-step segment ----
    {
        float h[N], b_lb[N], u_lb = 0.0f;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            h[n] = p.h0 ? p.h0[((int64_t)b * Dn + dc) * N + n] : 0.0f;
            b_lb[n] = 0.0f;
        }
        lookback(0, u_lb, b_lb);
        for (int64_t t = 0; t < L; ++t) {
            if (t % kM3Seg == 0) {
#pragma unroll
                for (int n = 0; n < N; ++n)
                    ck[((t / kM3Seg) * N + n) * 64 + lane] = h[n];
            }
            advance(h, t, u_lb, b_lb);
        }
    }

    // ---- 2. segments in reverse ----
    float mu[N], dA[N], lbk[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        mu[n] = dvalid && p.dh_last ? p.dh_last[((int64_t)b * Dn + dc) * N + n] : 0.0f;
        dA[n] = 0.0f;
        lbk[n] = 0.0f; // mu_{t+1} (1 - lam_{t+1}) Delta_{t+1}: the look-back's weights
    }
    float dD_acc = 0.0f, db_acc = 0.0f;
    for (int seg = p.n_seg - 1; seg >= 0; --seg) {
        const int64_t t0 = (int64_t)seg * kM3Seg;
        const int64_t t1 = min(t0 + (int64_t)kM3Seg, L);
        for (int sg = SG - 1; sg >= 0; --sg) {
            const int64_t ts = t0 + (int64_t)sg * S;
            if (ts >= t1)
                continue;
            const int ns = (int)min((int64_t)S, t1 - ts);
            // the state entering ts: the stored one, advanced through [t0, ts)
            float hc[N], b_lb[N], u_lb = 0.0f;
#pragma unroll
            for (int n = 0; n < N; ++n) {
                hc[n] = ck[(seg * N + n) * 64 + lane];
                b_lb[n] = 0.0f;
            }
            lookback(t0, u_lb, b_lb);
            for (int64_t t = t0; t < ts; ++t)
                advance(hc, t, u_lb, b_lb);
            float hin[N], hs[S][N];
#pragma unroll
            for (int n = 0; n < N; ++n)
                hin[n] = hc[n];
#pragma unroll
            for (int s = 0; s < S; ++s) {
                if (s < ns)
                    advance(hc, ts + s, u_lb, b_lb);
#pragma unroll
                for (int n = 0; n < N; ++n)
                    hs[s][n] = hc[n];
            }
            // adjoint, last step first
#pragma unroll
            for (int s = S - 1; s >= 0; --s) {
                if (s >= ns)
                    continue;
                const int64_t t = ts + s;
                const int64_t bld = (row0 + t) * Dn + dc;
                const float uu = ld(p.u, bld);
                const float v = ld(p.delta, bld) + bias_d;
                const float dl = softplus_f(v);
                const float sig = hw_rcp(1.0f + hw_exp2(-v * kLog2e)); // softplus'(v)
                const float dyv = dvalid ? ld(p.dy, bld) : 0.0f;
                float gate = 1.0f, dgate = 0.0f;
                if constexpr (GATED) {
                    const float zz = ld(p.z, bld);
                    const float sz = hw_rcp(1.0f + hw_exp2(-zz * kLog2e));
                    gate = zz * sz;
                    dgate = sz * __builtin_fmaf(zz, 1.0f - sz, 1.0f);
                }
                const float ds = dyv * gate;
                const float lm = TRAP ? ld(p.lam, bld) : 0.0f;
                float up = 0.0f, bp[N];
#pragma unroll
                for (int n = 0; n < N; ++n)
                    bp[n] = 0.0f;
                lookback(t, up, bp);
                // h' : the previous state after the rotation
                float hp[N];
#pragma unroll
                for (int n = 0; n < N; ++n)
                    hp[n] = s == 0 ? hin[n] : hs[s > 0 ? s - 1 : 0][n];
                if constexpr (ROT) {
#pragma unroll
                    for (int k = 0; k < K; ++k)
                        rotate_pair(dl * ld(p.theta, (row0 + t) * K + k), hp[2 * k],
                                    hp[2 * k + 1]);
                }
                float vals[V];
                float sy = D_d * uu, ddt = 0.0f, du = ds * D_d, dlam = 0.0f;
#pragma unroll
                for (int n = 0; n < N; ++n) {
                    const float cn = ld(p.C, (row0 + t) * N + n);
                    sy = __builtin_fmaf(cn, hs[s][n], sy);
                    mu[n] = __builtin_fmaf(ds, cn, mu[n]); // mu_t
                    vals[N + n] = ds * hs[s][n];           // dC
                }
#pragma unroll
                for (int n = 0; n < N; ++n) {
                    const float bn = ld(p.B, (row0 + t) * N + n);
                    const float a = decay_exp2(dl, a2[n]);
                    const float mah = mu[n] * a * hp[n];
                    ddt = __builtin_fmaf(an[n], mah, ddt);
                    dA[n] = __builtin_fmaf(dl, mah, dA[n]);
                    if constexpr (TRAP) {
                        // this step's term, and step t + 1's look-back, which read u_t, B_t
                        ddt += mu[n] * __builtin_fmaf(1.0f - lm, bp[n] * up, lm * bn * uu);
                        du = __builtin_fmaf(__builtin_fmaf(mu[n], lm * dl, lbk[n]), bn, du);
                        vals[n] = __builtin_fmaf(mu[n], lm * dl, lbk[n]) * uu; // dB
                        dlam = __builtin_fmaf(mu[n] * dl, bn * uu - bp[n] * up, dlam);
                        lbk[n] = mu[n] * (1.0f - lm) * dl;
                    } else if constexpr (ZOH) {
                        const float x = dl * an[n];
                        const float beta = zoh_input(x, a, dl, ia[n]);
                        const float psi = __builtin_fmaf(
                            x, __builtin_fmaf(x, __builtin_fmaf(x, __builtin_fmaf(
                                x, 1.0f / 144.0f, 1.0f / 30.0f), 1.0f / 8.0f), 1.0f / 3.0f),
                            0.5f);
                        const float dbA = __builtin_fabsf(x) < 0.0625f ? dl * dl * psi
                                                                       : (dl * a - beta) * ia[n];
                        ddt = __builtin_fmaf(mu[n] * bn * uu, a, ddt);
                        du = __builtin_fmaf(mu[n] * beta, bn, du);
                        vals[n] = mu[n] * beta * uu; // dB
                        dA[n] = __builtin_fmaf(mu[n] * bn * uu, dbA, dA[n]);
                    } else {
                        ddt = __builtin_fmaf(mu[n], bn * uu, ddt);
                        du = __builtin_fmaf(mu[n] * dl, bn, du);
                        vals[n] = mu[n] * dl * uu; // dB
                    }
                    mu[n] *= a; // nu = dLoss/dh'
                }
                if constexpr (ROT) {
#pragma unroll
                    for (int k = 0; k < K; ++k) {
                        const float th = ld(p.theta, (row0 + t) * K + k);
                        const float dphi = mu[2 * k + 1] * hp[2 * k] - mu[2 * k] * hp[2 * k + 1];
                        ddt = __builtin_fmaf(th, dphi, ddt);
                        vals[2 * N + k] = dl * dphi; // dtheta
                        // R^T nu: the pair turned back by the step's angle
                        float sn, cs;
                        sincos_fast(dl * th, sn, cs);
                        const float x0 = mu[2 * k], x1 = mu[2 * k + 1];
                        mu[2 * k] = __builtin_fmaf(cs, x0, sn * x1);
                        mu[2 * k + 1] = __builtin_fmaf(cs, x1, -sn * x0);
                    }
                }
                const float dd = ddt * sig;
                dD_acc = __builtin_fmaf(ds, uu, dD_acc);
                db_acc += dd;
                if (dvalid) {
                    store_val((T *)p.du, bld, du);
                    store_val((T *)p.ddelta, bld, dd);
                    if constexpr (GATED)
                        store_val((T *)p.dz, bld, dyv * sy * dgate);
                    if constexpr (TRAP)
                        if (p.dlam)
                            store_val((T *)p.dlam, bld, dlam);
                }
                lane_sums(std::integral_constant<int, V>{}, vals,
                          p.part + ((int64_t)unit * L + t) * V);
            }
        }
    }

    // ---- 3. per-wave results ----
    if constexpr (TRAP) {
        // the first look-back read u_prev and B_prev
        float bpv[N], dup = 0.0f;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const float bp = p.B_prev ? ld(p.B_prev, (int64_t)b * N + n) : 0.0f;
            dup = __builtin_fmaf(lbk[n], bp, dup);
            bpv[n] = lbk[n] * u_pre;
        }
        if (dvalid && p.du_prev)
            store_val((T *)p.du_prev, (int64_t)b * Dn + d, dup);
        lane_sums(std::integral_constant<int, N>{}, bpv, p.bprev_part + (int64_t)unit * N);
    }
    if (dvalid) {
        const int64_t col = ((int64_t)b * Dn + d) * N;
#pragma unroll
        for (int n = 0; n < N; ++n) {
            p.dA_part[col + n] = dA[n];
            if (p.dh0)
                p.dh0[col + n] = mu[n];
        }
        p.dDb_part[((int64_t)b * Dn + d) * 2 + 0] = dD_acc;
        p.dDb_part[((int64_t)b * Dn + d) * 2 + 1] = db_acc;
    }
}

// dB, dC, dtheta: the tiles' partials added in tile order; dB_prev likewise.
template <typename T>
__global__ void __launch_bounds__(256)
m3_reduce_kernel(const float *__restrict__ part, const float *__restrict__ bprev_part, T *dB,
                 T *dC, T *dtheta, T *dB_prev, int64_t batch, int64_t L, int32_t N, int32_t V,
                 int32_t tiles)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = batch * L * V;
    if (i < total) {
        const int j = (int)(i % V);
        const int64_t bt = i / V;
        const int64_t b = bt / L, t = bt % L;
        float s = 0.0f;
        for (int tile = 0; tile < tiles; ++tile)
            s += part[(((int64_t)tile * batch + b) * L + t) * V + j];
        if (j < N) {
            if (dB)
                store_val(dB, bt * N + j, s);
        } else if (j < 2 * N) {
            if (dC)
                store_val(dC, bt * N + (j - N), s);
        } else if (dtheta) {
            store_val(dtheta, bt * (N / 2) + (j - 2 * N), s);
        }
    } else if (dB_prev && i < total + batch * N) {
        const int64_t k = i - total; // b * N + n
        const int64_t b = k / N, n = k % N;
        float s = 0.0f;
        for (int tile = 0; tile < tiles; ++tile)
            s += bprev_part[((int64_t)tile * batch + b) * N + n];
        store_val(dB_prev, k, s);
    }
}

// dA = sum over the batch rows of dA_part; dD, dbias likewise (fixed order).
__global__ void __launch_bounds__(256)
m3_reduce_params_kernel(const float *__restrict__ dA_part, const float *__restrict__ dDb_part,
                        float *dA, float *dD, float *dbias, int64_t batch, int64_t Dn, int64_t N)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t dn = Dn * N;
    if (i < dn) {
        float s = 0.0f;
        for (int64_t b = 0; b < batch; ++b)
            s += dA_part[b * dn + i];
        if (dA)
            dA[i] = s;
    } else if (i < dn + Dn) {
        const int64_t d = i - dn;
        float sD = 0.0f, sb = 0.0f;
        for (int64_t b = 0; b < batch; ++b) {
            sD += dDb_part[(b * Dn + d) * 2 + 0];
            sb += dDb_part[(b * Dn + d) * 2 + 1];
        }
        if (dD)
            dD[d] = sD;
        if (dbias)
            dbias[d] = sb;
    }
}

template <typename T, int N, bool ZOH, bool TRAP, bool ROT>
hipError_t launch_m3_t(const M3BwdLaunch &q, hipStream_t stream)
{
    const int64_t tiles = (q.d_inner + 63) / 64;
    const int64_t units = tiles * q.batch;
    if (units <= 0 || q.L <= 0)
        return hipSuccess;
    M3Args a{};
    a.u = q.u;
    a.delta = q.delta;
    a.z = q.z;
    a.dy = q.dy;
    a.B = q.B;
    a.C = q.C;
    a.lam = q.lam;
    a.u_prev = q.u_prev;
    a.B_prev = q.B_prev;
    a.theta = q.theta;
    a.A = q.A;
    a.D = q.D;
    a.bias = q.bias;
    a.h0 = q.h0;
    a.dh_last = q.dh_last;
    a.du = q.du;
    a.ddelta = q.ddelta;
    a.dz = q.dz;
    a.dlam = q.dlam;
    a.du_prev = q.du_prev;
    a.dh0 = q.dh0;
    a.ckpt = q.ckpt;
    a.part = q.part;
    a.bprev_part = q.bprev_part;
    a.dA_part = q.dA_part;
    a.dDb_part = q.dDb_part;
    a.L = q.L;
    a.Dn = (int32_t)q.d_inner;
    a.batch = (int32_t)q.batch;
    a.n_seg = (int32_t)((q.L + kM3Seg - 1) / kM3Seg);
    if (q.z)
        hipLaunchKernelGGL((scan_bwd_m3_kernel<T, N, ZOH, TRAP, ROT, true>),
                           dim3((uint32_t)units), dim3(64), 0, stream, a);
    else
        hipLaunchKernelGGL((scan_bwd_m3_kernel<T, N, ZOH, TRAP, ROT, false>),
                           dim3((uint32_t)units), dim3(64), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    constexpr int V = 2 * N + (ROT ? N / 2 : 0);
    const int64_t nred = q.batch * q.L * V + (TRAP ? q.batch * N : 0);
    hipLaunchKernelGGL((m3_reduce_kernel<T>), dim3((uint32_t)((nred + 255) / 256)), dim3(256), 0,
                       stream, q.part, q.bprev_part, (T *)q.dB, (T *)q.dC, (T *)q.dtheta,
                       TRAP ? (T *)q.dB_prev : (T *)nullptr, q.batch, q.L, (int32_t)N,
                       (int32_t)V, (int32_t)tiles);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    const int64_t np = q.d_inner * N + q.d_inner;
    hipLaunchKernelGGL(m3_reduce_params_kernel, dim3((uint32_t)((np + 255) / 256)), dim3(256), 0,
                       stream, q.dA_part, q.dDb_part, q.dA, q.dD, q.dbias, q.batch, q.d_inner,
                       (int64_t)N);
    return hipGetLastError();
}

template <typename T, int N>
hipError_t launch_m3_n(const M3BwdLaunch &q, hipStream_t stream)
{
    const bool trap = q.lam != nullptr, rot = q.theta != nullptr;
    if (trap && rot)
        return launch_m3_t<T, N, false, true, true>(q, stream);
    if (trap)
        return launch_m3_t<T, N, false, true, false>(q, stream);
    if (rot && q.zoh)
        return launch_m3_t<T, N, true, false, true>(q, stream);
    if (rot)
        return launch_m3_t<T, N, false, false, true>(q, stream);
    return hipErrorInvalidValue; // (the other cases run in scan_bwd.hip)
}

} // namespace

size_t m3_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state,
                              bool rot, size_t off[6])
{
    auto al = [](size_t n) { return (n + 255) / 256 * 256; };
    const size_t units = (size_t)batch * (size_t)((d_inner + 63) / 64);
    const size_t n_seg = (size_t)((L + kM3Seg - 1) / kM3Seg);
    const size_t N = (size_t)d_state, V = 2 * N + (rot ? N / 2 : 0), f = sizeof(float);
    size_t sz[5];
    sz[0] = al(units * n_seg * N * 64 * f);           // stored states
    sz[1] = al(units * (size_t)L * V * f);             // dB, dC, dtheta tile partials
    sz[2] = al(units * N * f);                         // dB_prev tile partials
    sz[3] = al((size_t)batch * (size_t)d_inner * N * f); // dA per batch row
    sz[4] = al((size_t)batch * (size_t)d_inner * 2 * f); // dD, dbias per batch row
    off[0] = 0;
    for (int i = 0; i < 5; ++i)
        off[i + 1] = off[i] + sz[i];
    return L > 0 ? off[5] : 0;
}

hipError_t launch_scan_bwd_m3(const M3BwdLaunch &q, hipStream_t stream)
{
#define M3_CASE(N_)                                                \
    if (q.d_state == N_) {                                         \
        if (q.dtype == DType::BF16)                                \
            return launch_m3_n<uint16_t, N_>(q, stream);           \
        return launch_m3_n<float, N_>(q, stream);                  \
    }
    M3_CASE(4)
    M3_CASE(8)
    M3_CASE(16)
    M3_CASE(32)
#undef M3_CASE
    return hipErrorInvalidValue;
}

} // namespace mambascan
