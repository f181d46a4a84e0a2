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
// Work decomposition: a block of four waves per (batch row, 64-channel tile); wave w takes
// channels 16 w .. 16 w + 15 and lane c + 16 g of a wave holds channel c's states
// g N/4 .. (g + 1) N/4 - 1 (whole rotation pairs), so the large prefill runs 2560 waves
// (with the rotation at d_state 4: two waves of 32 channels, two states per lane).  The
// block runs the forward once storing the state every 8 steps, then walks the 8-step
// segments backwards; within a segment, sub-segments of S steps (whose states fit the
// registers) are recomputed from the stored state and their adjoint run.  Per-channel sums
// over the states (dDelta, du, dlam, the readout for dz) join the four lanes of a channel
// with two lane exchanges.  Sums over the tile's channels (dB, dC, dtheta per step and state)
// are added over each lane quad by DPP, written as 16 partials per value to an LDS slab
// (4 quads x 4 waves), and summed there once per sub-segment into per-tile partials, which
// a second kernel adds in tile order.  Every sum runs in a fixed order: results are
// bitwise reproducible.
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
    float *dA_part;    // [span][b][d][n]
    float *dDb_part;   // [span][b][d][2]: dD, dbias
    // sequence split (n_spans > 1; else NULL): the state entering each span and the adjoint
    // entering it from its end, [span][b][d][n]; du of a span's last step before the next
    // span's look-back share, and that share, [span][b][d]; the adjoint span pass's result
    const float *h_in, *mu_in;
    float *du_edge, *du_lb, *mu_loc;
    int64_t L, span_len;
    int32_t Dn, batch, n_seg; // n_seg: segments per block (of its span)
    int32_t n_spans, units;   // units = tiles * batch; block = span * units + unit
};

// NV values of a vector of the activation type at element i (NV consecutive elements, i a
// multiple of NV): one load of 2 NV or 4 NV bytes (the entry point takes the arrays read
// this way 16-byte aligned only).
template <typename T, int NV>
__device__ __forceinline__ void load_vec(const void *base, int64_t i, float (&out)[NV])
{
    if constexpr (std::is_same<T, float>::value) {
        const float *q = (const float *)base + i;
        if constexpr (NV % 4 == 0) {
#pragma unroll
            for (int k = 0; k < NV; k += 4) {
                const float4 v = *reinterpret_cast<const float4 *>(q + k);
                out[k] = v.x; out[k + 1] = v.y; out[k + 2] = v.z; out[k + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int k = 0; k < NV; ++k)
                out[k] = q[k];
        }
    } else {
        const uint16_t *q = (const uint16_t *)base + i;
        if constexpr (NV % 4 == 0) {
#pragma unroll
            for (int k = 0; k < NV; k += 4) {
                const uint2 v = *reinterpret_cast<const uint2 *>(q + k);
                out[k] = __uint_as_float(v.x << 16);
                out[k + 1] = __uint_as_float(v.x & 0xffff0000u);
                out[k + 2] = __uint_as_float(v.y << 16);
                out[k + 3] = __uint_as_float(v.y & 0xffff0000u);
            }
        } else if constexpr (NV == 2) {
            const uint32_t v = *reinterpret_cast<const uint32_t *>(q);
            out[0] = __uint_as_float(v << 16);
            out[1] = __uint_as_float(v & 0xffff0000u);
        } else {
#pragma unroll
            for (int k = 0; k < NV; ++k)
                out[k] = load_val(q, k);
        }
    }
}

// v summed over the lane's quad (lanes 4i .. 4i + 3), every lane of the quad getting the
// same sum: DPP quad_perm [1,0,3,2], then [2,3,0,1].
__device__ __forceinline__ float quad_sum(float v)
{
    const float a = v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1,
                                                                    0xF, 0xF, false));
    return a + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x4E, 0xF, 0xF,
                                                          false));
}

// Groups of states per channel (lanes per channel): four, or two where four would split the
// rotation pairs (d_state 4).
template <int N, bool ROT> constexpr int m3_groups() { return ROT && N < 8 ? 2 : 4; }

// SPLIT: blocks cover the spans of a split sequence (else one block walks the whole sequence:
// the span quantities below are compile-time constants, which keeps the scalar registers of
// the unsplit kernel free).
template <typename T, int N, bool ZOH, bool TRAP, bool ROT, bool GATED, bool SPLIT>
__global__ void __launch_bounds__(256) scan_bwd_m3_kernel(M3Args p)
{
    static_assert(!(ZOH && TRAP), "the trapezoid replaces the input term");
    constexpr int GR = m3_groups<N, ROT>(); // lanes per channel = waves per block
    constexpr int CW = 64 / GR;           // channels per wave
    constexpr int NT = 64 * GR;           // threads per block
    static_assert(N % GR == 0 && (!ROT || (N / GR) % 2 == 0), "states per lane");
    constexpr int NG = N / GR;            // states per lane: n = g NG + j
    constexpr int KG = ROT ? NG / 2 : 1;  // rotation pairs per lane: k = g KG + kk
    constexpr int K = N / 2;
    constexpr int S = NG <= 4 ? 8 : 4;    // steps whose states are kept in registers
    constexpr int SG = kM3Seg / S;        // sub-segments per stored state
    constexpr int V = 2 * N + (ROT ? K : 0); // values summed over channels per step
    constexpr int kQ = 16;                // partials per value: one per 4 channels
    __shared__ __attribute__((aligned(16))) float s_v[S * V][kQ];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane % CW, g = lane / CW;
    const int ch = CW * w + c; // channel within the tile
    const int unit = SPLIT ? blockIdx.x % p.units : blockIdx.x; // tile * batch + b
    const int span = SPLIT ? blockIdx.x / p.units : 0;
    const int b = unit % p.batch, tile = unit / p.batch;
    const int Dn = p.Dn;
    const int d = tile * 64 + ch;
    const bool dvalid = d < Dn;
    const int dc = dvalid ? d : Dn - 1; // tail lanes compute on a valid channel with dy = 0
    const int n0 = g * NG, k0 = g * KG;
    const bool writer = (c & 3) == 0; // the lane that writes its quad's partials
    // the sum over the GR lanes of a channel (every one of them gets it, in the same order)
    auto chan_sum = [](float v) {
        if constexpr (GR == 4) {
            return lane_pair_sum(v);
        } else {
            const uint32_t x = __float_as_uint(v);
            const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
            return __uint_as_float(r[0]) + __uint_as_float(r[1]);
        }
    };
    const int qslot = ch >> 2;
    const int64_t L = p.L;
    const int64_t row0 = (int64_t)b * L;
    const int64_t tb = SPLIT ? (int64_t)span * p.span_len : 0; // this block's steps [tb, te)
    const int64_t te = SPLIT ? min(tb + p.span_len, L) : L;
    const int n_seg = (int)((te - tb + kM3Seg - 1) / kM3Seg);
    const int64_t bd = (int64_t)p.batch * Dn, bdn = bd * N;
    auto ld = [](const void *base, int64_t i) { return load_val((const T *)base, i); };

    float a2[NG], an[NG], ia[NG];
#pragma unroll
    for (int j = 0; j < NG; ++j) {
        const float av = p.A[(int64_t)dc * N + n0 + j];
        a2[j] = av * kLog2e;
        an[j] = av;
        ia[j] = ZOH ? 1.0f / av : 0.0f;
    }
    const float bias_d = p.bias ? p.bias[dc] : 0.0f;
    const float D_d = p.D ? p.D[dc] : 0.0f;
    const float u_pre = TRAP && p.u_prev ? ld(p.u_prev, (int64_t)b * Dn + dc) : 0.0f;
    float bpre[NG];
#pragma unroll
    for (int j = 0; j < NG; ++j)
        bpre[j] = 0.0f;
    if (TRAP && p.B_prev)
        load_vec<T, NG>(p.B_prev, (int64_t)b * N + n0, bpre);

    // the look-back input (u, B of this lane's states) of step t: the previous step's, or
    // (u_prev, B_prev)
    auto lookback = [&](int64_t t, float &u_lb, float (&b_lb)[NG]) {
        if constexpr (TRAP) {
            if (t > 0) {
                u_lb = ld(p.u, (row0 + t - 1) * Dn + dc);
                load_vec<T, NG>(p.B, (row0 + t - 1) * N + n0, b_lb);
            } else {
                u_lb = u_pre;
#pragma unroll
                for (int j = 0; j < NG; ++j)
                    b_lb[j] = bpre[j];
            }
        }
    };
    // one forward step: rotation (its sine and cosine returned), decay, input term; the
    // look-back advances to step t
    auto advance = [&](float (&h)[NG], int64_t t, float &u_lb, float (&b_lb)[NG],
                       float (&sn)[KG], float (&cs)[KG]) {
        const int64_t bld = (row0 + t) * Dn + dc;
        const float uu = ld(p.u, bld);
        const float dl = softplus_act<T>(ld(p.delta, bld) + bias_d);
        if constexpr (ROT) {
            float th[KG];
            load_vec<T, KG>(p.theta, (row0 + t) * K + k0, th);
#pragma unroll
            for (int kk = 0; kk < KG; ++kk) {
                sincos_act<T>(dl * th[kk], sn[kk], cs[kk]);
                turn_pair(sn[kk], cs[kk], h[2 * kk], h[2 * kk + 1]);
            }
        }
        const float lm = TRAP ? ld(p.lam, bld) : 0.0f;
        float bn[NG];
        load_vec<T, NG>(p.B, (row0 + t) * N + n0, bn);
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            const float a = decay_exp2(dl, a2[j]);
            float in;
            if constexpr (TRAP)
                in = __builtin_fmaf((1.0f - lm) * dl * u_lb, b_lb[j], lm * dl * uu * bn[j]);
            else if constexpr (ZOH)
                in = zoh_input(dl * an[j], a, dl * uu, uu * ia[j]) * bn[j];
            else
                in = dl * uu * bn[j];
            h[j] = __builtin_fmaf(a, h[j], in);
            if constexpr (TRAP)
                b_lb[j] = bn[j];
        }
        if constexpr (TRAP)
            u_lb = uu;
    };

    float *ck = p.ckpt + (int64_t)blockIdx.x * p.n_seg * N * 64;

    // ---- 1. forward: the state entering every 8-step segment ----
    {
        float h[NG], b_lb[NG], u_lb = 0.0f, sn[KG], cs[KG];
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            const int64_t hc = ((int64_t)b * Dn + dc) * N + n0 + j;
            h[j] = SPLIT ? p.h_in[span * bdn + hc] : p.h0 ? p.h0[hc] : 0.0f;
            b_lb[j] = 0.0f;
        }
        lookback(tb, u_lb, b_lb);
        for (int seg = 0; seg < n_seg; ++seg) {
            const int64_t t0 = tb + (int64_t)seg * kM3Seg;
#pragma unroll
            for (int j = 0; j < NG; ++j)
                ck[(seg * N + n0 + j) * 64 + ch] = h[j];
            if (t0 + kM3Seg <= te) { // (no branch between the steps: their loads go ahead)
#pragma unroll
                for (int s = 0; s < kM3Seg; ++s)
                    advance(h, t0 + s, u_lb, b_lb, sn, cs);
            } else {
                for (int64_t t = t0; t < te; ++t)
                    advance(h, t, u_lb, b_lb, sn, cs);
            }
        }
    }

    // ---- 2. segments in reverse ----
    float mu[NG], dA[NG], lbk[NG];
#pragma unroll
    for (int j = 0; j < NG; ++j) {
        const int64_t hc = ((int64_t)b * Dn + dc) * N + n0 + j;
        mu[j] = !dvalid     ? 0.0f
                : SPLIT     ? p.mu_in[span * bdn + hc]
                : p.dh_last ? p.dh_last[hc]
                            : 0.0f;
        dA[j] = 0.0f;
        lbk[j] = 0.0f; // mu_{t+1} (1 - lam_{t+1}) Delta_{t+1}: the look-back's weights
    }
    float dD_acc = 0.0f, db_acc = 0.0f;
    // the trapezoid's du of the block's last step waits for the next span's look-back share
    const int64_t t_edge = SPLIT && TRAP && span < p.n_spans - 1 ? te - 1 : -1;
    for (int seg = n_seg - 1; seg >= 0; --seg) {
        const int64_t t0 = tb + (int64_t)seg * kM3Seg;
        const int64_t t1 = min(t0 + (int64_t)kM3Seg, te);
        for (int sg = SG - 1; sg >= 0; --sg) {
            const int64_t ts = t0 + (int64_t)sg * S;
            if (ts >= t1)
                continue; // (uniform over the block)
            const int ns = (int)min((int64_t)S, t1 - ts);
            // the state entering ts: the stored one, advanced through [t0, ts)
            float hc[NG], b_lb[NG], u_lb = 0.0f;
            float rsn[S][KG], rcs[S][KG];
#pragma unroll
            for (int j = 0; j < NG; ++j) {
                hc[j] = ck[(seg * N + n0 + j) * 64 + ch];
                b_lb[j] = 0.0f;
            }
            lookback(t0, u_lb, b_lb);
            for (int64_t t = t0; t < ts; ++t)
                advance(hc, t, u_lb, b_lb, rsn[0], rcs[0]);
            float hin[NG], hs[S][NG];
#pragma unroll
            for (int j = 0; j < NG; ++j)
                hin[j] = hc[j];
#pragma unroll
            for (int s = 0; s < S; ++s) {
                if (s < ns)
                    advance(hc, ts + s, u_lb, b_lb, rsn[s], rcs[s]);
#pragma unroll
                for (int j = 0; j < NG; ++j)
                    hs[s][j] = hc[j];
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
                const float dl = softplus_act<T>(v);
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
                float up = 0.0f, bp[NG], bn[NG], cn[NG];
#pragma unroll
                for (int j = 0; j < NG; ++j)
                    bp[j] = 0.0f;
                lookback(t, up, bp);
                load_vec<T, NG>(p.B, (row0 + t) * N + n0, bn);
                load_vec<T, NG>(p.C, (row0 + t) * N + n0, cn);
                // h' : the previous state after the rotation
                float hp[NG];
#pragma unroll
                for (int j = 0; j < NG; ++j)
                    hp[j] = s == 0 ? hin[j] : hs[s > 0 ? s - 1 : 0][j];
                if constexpr (ROT) {
#pragma unroll
                    for (int kk = 0; kk < KG; ++kk)
                        turn_pair(rsn[s][kk], rcs[s][kk], hp[2 * kk], hp[2 * kk + 1]);
                }
                float vb[NG], vc[NG], vt[KG];
                float sy = 0.0f, ddt = 0.0f, du = 0.0f, dlam = 0.0f;
#pragma unroll
                for (int j = 0; j < NG; ++j) {
                    sy = __builtin_fmaf(cn[j], hs[s][j], sy);
                    mu[j] = __builtin_fmaf(ds, cn[j], mu[j]); // mu_t
                    vc[j] = ds * hs[s][j];                    // dC
                }
                // trapezoid: the step's input term lam Delta B_t u_t + (1 - lam) Delta B_{t-1}
                // u_{t-1} enters dDelta and dlam through sum mu B_t and sum mu B_{t-1} only
                float smb = 0.0f, smp = 0.0f;
                const float ldl = lm * dl, mdl = (1.0f - lm) * dl;
#pragma unroll
                for (int j = 0; j < NG; ++j) {
                    const float a = decay_exp2(dl, a2[j]);
                    const float mah = mu[j] * a * hp[j];
                    ddt = __builtin_fmaf(an[j], mah, ddt);
                    dA[j] = __builtin_fmaf(dl, mah, dA[j]);
                    if constexpr (TRAP) {
                        smb = __builtin_fmaf(mu[j], bn[j], smb);
                        smp = __builtin_fmaf(mu[j], bp[j], smp);
                        // u_t and B_t feed this step's term and step t + 1's look-back
                        const float wgt = __builtin_fmaf(mu[j], ldl, lbk[j]);
                        du = __builtin_fmaf(wgt, bn[j], du);
                        vb[j] = wgt * uu; // dB
                        lbk[j] = mu[j] * mdl;
                    } else if constexpr (ZOH) {
                        const float x = dl * an[j];
                        const float beta = zoh_input(x, a, dl, ia[j]);
                        const float psi = __builtin_fmaf(
                            x, __builtin_fmaf(x, __builtin_fmaf(x, __builtin_fmaf(
                                x, 1.0f / 144.0f, 1.0f / 30.0f), 1.0f / 8.0f), 1.0f / 3.0f),
                            0.5f);
                        const float dbA = __builtin_fabsf(x) < 0.0625f ? dl * dl * psi
                                                                       : (dl * a - beta) * ia[j];
                        ddt = __builtin_fmaf(mu[j] * bn[j] * uu, a, ddt);
                        du = __builtin_fmaf(mu[j] * beta, bn[j], du);
                        vb[j] = mu[j] * beta * uu; // dB
                        dA[j] = __builtin_fmaf(mu[j] * bn[j] * uu, dbA, dA[j]);
                    } else {
                        ddt = __builtin_fmaf(mu[j], bn[j] * uu, ddt);
                        du = __builtin_fmaf(mu[j] * dl, bn[j], du);
                        vb[j] = mu[j] * dl * uu; // dB
                    }
                    mu[j] *= a; // nu = dLoss/dh'
                }
                if constexpr (TRAP) {
                    ddt = __builtin_fmaf((1.0f - lm) * up, smp, __builtin_fmaf(lm * uu, smb, ddt));
                    dlam = dl * __builtin_fmaf(uu, smb, -up * smp);
                }
                if constexpr (ROT) {
                    float th[KG];
                    load_vec<T, KG>(p.theta, (row0 + t) * K + k0, th);
#pragma unroll
                    for (int kk = 0; kk < KG; ++kk) {
                        const float dphi = mu[2 * kk + 1] * hp[2 * kk] - mu[2 * kk] * hp[2 * kk + 1];
                        ddt = __builtin_fmaf(th[kk], dphi, ddt);
                        vt[kk] = dl * dphi; // dtheta
                        // R^T nu: the pair turned back by the step's angle
                        const float x0 = mu[2 * kk], x1 = mu[2 * kk + 1];
                        mu[2 * kk] = __builtin_fmaf(rcs[s][kk], x0, rsn[s][kk] * x1);
                        mu[2 * kk + 1] = __builtin_fmaf(rcs[s][kk], x1, -rsn[s][kk] * x0);
                    }
                }
                // per-channel sums over the four lanes of the channel
                ddt = chan_sum(ddt);
                du = chan_sum(du);
                sy = chan_sum(sy) + D_d * uu;
                if constexpr (TRAP)
                    dlam = chan_sum(dlam);
                const float dd = ddt * sig;
                dD_acc = __builtin_fmaf(ds, uu, dD_acc);
                db_acc += dd;
                if (dvalid && g == 0) {
                    const float duv = __builtin_fmaf(ds, D_d, du);
                    if (t == t_edge)
                        p.du_edge[span * bd + (int64_t)b * Dn + d] = duv;
                    else
                        store_val((T *)p.du, bld, duv);
                    store_val((T *)p.ddelta, bld, dd);
                    if constexpr (GATED)
                        store_val((T *)p.dz, bld, dyv * sy * dgate);
                    if constexpr (TRAP)
                        if (p.dlam)
                            store_val((T *)p.dlam, bld, dlam);
                }
                // sums over the tile's channels: quads by DPP, then the slab
#pragma unroll
                for (int j = 0; j < NG; ++j) {
                    const float sb = quad_sum(vb[j]), sc = quad_sum(vc[j]);
                    if (writer) {
                        s_v[s * V + n0 + j][qslot] = sb;
                        s_v[s * V + N + n0 + j][qslot] = sc;
                    }
                }
                if constexpr (ROT) {
#pragma unroll
                    for (int kk = 0; kk < KG; ++kk) {
                        const float st = quad_sum(vt[kk]);
                        if (writer)
                            s_v[s * V + 2 * N + k0 + kk][qslot] = st;
                    }
                }
            }
            __syncthreads();
            // the sub-segment's per-tile sums, each of the 16 partials in slot order
            for (int e = tid; e < ns * V; e += NT) {
                const float4 *src = reinterpret_cast<const float4 *>(&s_v[e][0]);
                float sum = 0.0f;
#pragma unroll
                for (int i = 0; i < kQ / 4; ++i) {
                    const float4 q = src[i];
                    sum += (q.x + q.y) + (q.z + q.w);
                }
                p.part[((int64_t)unit * L + ts) * V + e] = sum;
            }
            __syncthreads();
        }
    }

    // ---- 3. per-block results ----
    if constexpr (TRAP) {
        // the look-back of the block's first step, which read u and B of the step before it
        // (u_prev and B_prev at t = 0): their shares of du and dB
        float u_s = 0.0f, b_s[NG];
        lookback(tb, u_s, b_s);
        float dup = 0.0f;
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            dup = __builtin_fmaf(lbk[j], b_s[j], dup);
            const float sbp = quad_sum(lbk[j] * u_s);
            if (writer)
                s_v[n0 + j][qslot] = sbp;
        }
        dup = chan_sum(dup);
        if (dvalid && g == 0) {
            if (SPLIT && span > 0)
                p.du_lb[span * bd + (int64_t)b * Dn + d] = dup;
            else if (p.du_prev)
                store_val((T *)p.du_prev, (int64_t)b * Dn + d, dup);
        }
        __syncthreads();
        if (tid < N) {
            const float4 *src = reinterpret_cast<const float4 *>(&s_v[tid][0]);
            float sum = 0.0f;
#pragma unroll
            for (int i = 0; i < kQ / 4; ++i) {
                const float4 q = src[i];
                sum += (q.x + q.y) + (q.z + q.w);
            }
            p.bprev_part[((int64_t)span * p.units + unit) * N + tid] = sum;
        }
    }
    if (dvalid) {
        const int64_t col = ((int64_t)b * Dn + d) * N + n0;
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            p.dA_part[span * bdn + col + j] = dA[j];
            if (p.dh0 && span == 0)
                p.dh0[col + j] = mu[j];
        }
        if (g == 0) {
            p.dDb_part[(span * bd + (int64_t)b * Dn + d) * 2 + 0] = dD_acc;
            p.dDb_part[(span * bd + (int64_t)b * Dn + d) * 2 + 1] = db_acc;
        }
    }
}

// The adjoint span pass of a split sequence: for each span s >= 1, the adjoint of the state
// entering it (dLoss/dh at the step before the span) that the span's own outputs produce,
// walking it backwards from a zero adjoint at its end.  Per step (as the main kernel):
// mu += ds C, mu *= exp(Delta A), the pairs turned back by the step's angle.  The input
// term (Euler, zero-order hold, trapezoid) does not enter this recurrence.
template <typename T, int N, bool ROT, bool GATED>
__global__ void __launch_bounds__(256) m3_adjoint_span_kernel(M3Args p)
{
    constexpr int GR = m3_groups<N, ROT>();
    constexpr int CW = 64 / GR;
    constexpr int NG = N / GR;
    constexpr int KG = ROT ? NG / 2 : 1;
    constexpr int K = N / 2;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int c = lane % CW, g = lane / CW;
    const int unit = blockIdx.x % p.units;
    const int span = 1 + blockIdx.x / p.units;
    const int b = unit % p.batch, tile = unit / p.batch;
    const int Dn = p.Dn;
    const int d = tile * 64 + CW * w + c;
    const bool dvalid = d < Dn;
    const int dc = dvalid ? d : Dn - 1;
    const int n0 = g * NG, k0 = g * KG;
    const int64_t L = p.L, row0 = (int64_t)b * L;
    const int64_t tb = (int64_t)span * p.span_len, te = min(tb + p.span_len, L);
    float a2[NG], mu[NG];
#pragma unroll
    for (int j = 0; j < NG; ++j) {
        a2[j] = p.A[(int64_t)dc * N + n0 + j] * kLog2e;
        mu[j] = 0.0f;
    }
    const float bias_d = p.bias ? p.bias[dc] : 0.0f;
    auto step = [&](int64_t t) {
        const int64_t bld = (row0 + t) * Dn + dc;
        const float dl = softplus_act<T>(load_val((const T *)p.delta, bld) + bias_d);
        float ds = dvalid ? load_val((const T *)p.dy, bld) : 0.0f;
        if constexpr (GATED) {
            const float zz = load_val((const T *)p.z, bld);
            ds *= zz * hw_rcp(1.0f + hw_exp2(-zz * kLog2e));
        }
        float cn[NG];
        load_vec<T, NG>(p.C, (row0 + t) * N + n0, cn);
#pragma unroll
        for (int j = 0; j < NG; ++j)
            mu[j] = __builtin_fmaf(ds, cn[j], mu[j]) * decay_exp2(dl, a2[j]);
        if constexpr (ROT) {
            float th[KG];
            load_vec<T, KG>(p.theta, (row0 + t) * K + k0, th);
#pragma unroll
            for (int kk = 0; kk < KG; ++kk) {
                float sn, cs;
                sincos_act<T>(dl * th[kk], sn, cs);
                const float x0 = mu[2 * kk], x1 = mu[2 * kk + 1];
                mu[2 * kk] = __builtin_fmaf(cs, x0, sn * x1);
                mu[2 * kk + 1] = __builtin_fmaf(cs, x1, -sn * x0);
            }
        }
    };
    int64_t t = te - 1;
    for (; t - kM3Seg + 1 >= tb; t -= kM3Seg) { // whole segments: no branch between the steps
#pragma unroll
        for (int s = 0; s < kM3Seg; ++s)
            step(t - s);
    }
    for (; t >= tb; --t)
        step(t);
    if (dvalid) {
        const int64_t col = ((int64_t)b * Dn + d) * N + n0;
#pragma unroll
        for (int j = 0; j < NG; ++j)
            p.mu_loc[span * (int64_t)p.batch * Dn * N + col + j] = mu[j];
    }
}

// The adjoint entering each span from its end, spans in reverse: mu_in[S - 1] = dh_last,
// mu_in[s - 1] = M_s^T mu_in[s] + mu_loc[s] with M_s the span's forward transition (its
// decays, or each state pair's 2x2 matrix, from the forward span pass).  One thread per state
// (per pair with the rotation).
__global__ void __launch_bounds__(256)
m3_mu_carry_kernel(const float *__restrict__ dec, const float *__restrict__ rot,
                   const float *__restrict__ mu_loc, const float *__restrict__ dh_last,
                   float *__restrict__ mu_in, int64_t columns, int32_t n_spans)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int S = n_spans;
    if (rot) {
        if (i >= columns / 2)
            return;
        const int64_t c = 2 * i;
        float x0 = dh_last ? dh_last[c] : 0.0f, x1 = dh_last ? dh_last[c + 1] : 0.0f;
        mu_in[(int64_t)(S - 1) * columns + c] = x0;
        mu_in[(int64_t)(S - 1) * columns + c + 1] = x1;
        for (int s = S - 1; s >= 1; --s) {
            const float *m = rot + (i * S + s) * 4; // m00, m10, m01, m11
            const float y0 =
                __builtin_fmaf(m[0], x0, __builtin_fmaf(m[1], x1, mu_loc[(int64_t)s * columns + c]));
            const float y1 = __builtin_fmaf(
                m[2], x0, __builtin_fmaf(m[3], x1, mu_loc[(int64_t)s * columns + c + 1]));
            x0 = y0;
            x1 = y1;
            mu_in[(int64_t)(s - 1) * columns + c] = x0;
            mu_in[(int64_t)(s - 1) * columns + c + 1] = x1;
        }
    } else {
        if (i >= columns)
            return;
        float x = dh_last ? dh_last[i] : 0.0f;
        mu_in[(int64_t)(S - 1) * columns + i] = x;
        for (int s = S - 1; s >= 1; --s) {
            x = __builtin_fmaf(dec[i * S + s], x, mu_loc[(int64_t)s * columns + i]);
            mu_in[(int64_t)(s - 1) * columns + i] = x;
        }
    }
}

// du of the step before each span s >= 1: the previous span's own value plus span s's
// look-back share, rounded once.
template <typename T>
__global__ void __launch_bounds__(256)
m3_du_edge_kernel(const float *__restrict__ du_edge, const float *__restrict__ du_lb, T *du,
                  int64_t bd, int64_t L, int32_t Dn, int64_t span_len, int32_t n_spans)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)(n_spans - 1) * bd)
        return;
    const int64_t s = 1 + i / bd, r = i % bd; // r = b * Dn + d
    const int64_t b = r / Dn, dd = r % Dn;
    const int64_t t = s * span_len - 1;
    store_val(du, (b * L + t) * Dn + dd, du_edge[(s - 1) * bd + r] + du_lb[s * bd + r]);
}

// dB, dC, dtheta: the tiles' partials added in tile order, then (dB at the step before a
// span of lb_spans > 1, the trapezoid's) the tiles' look-back shares of that span; dB_prev
// likewise from span 0's shares.
template <typename T>
__global__ void __launch_bounds__(256)
m3_reduce_kernel(const float *__restrict__ part, const float *__restrict__ bprev_part, T *dB,
                 T *dC, T *dtheta, T *dB_prev, int64_t batch, int64_t L, int32_t N, int32_t V,
                 int32_t tiles, int64_t span_len, int32_t lb_spans)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = batch * L * V;
    const int64_t units = (int64_t)tiles * batch;
    if (i < total) {
        const int j = (int)(i % V);
        const int64_t bt = i / V;
        const int64_t b = bt / L, t = bt % L;
        float s = 0.0f;
        for (int tile = 0; tile < tiles; ++tile)
            s += part[(((int64_t)tile * batch + b) * L + t) * V + j];
        if (j < N) {
            if (lb_spans > 1 && (t + 1) % span_len == 0 && t + 1 < L) {
                const int64_t sp = (t + 1) / span_len;
                for (int tile = 0; tile < tiles; ++tile)
                    s += bprev_part[(sp * units + (int64_t)tile * batch + b) * N + j];
            }
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

// dA = sum over the (span, batch row) pairs of dA_part; dD, dbias likewise (fixed order).
__global__ void __launch_bounds__(256)
m3_reduce_params_kernel(const float *__restrict__ dA_part, const float *__restrict__ dDb_part,
                        float *dA, float *dD, float *dbias, int64_t rows, int64_t Dn, int64_t N)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t dn = Dn * N;
    if (i < dn) {
        float s = 0.0f;
        for (int64_t r = 0; r < rows; ++r)
            s += dA_part[r * dn + i];
        if (dA)
            dA[i] = s;
    } else if (i < dn + Dn) {
        const int64_t d = i - dn;
        float sD = 0.0f, sb = 0.0f;
        for (int64_t r = 0; r < rows; ++r) {
            sD += dDb_part[(r * Dn + d) * 2 + 0];
            sb += dDb_part[(r * Dn + d) * 2 + 1];
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
    const int S = q.n_spans;
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
    a.span_len = S > 1 ? q.span_len : q.L;
    a.Dn = (int32_t)q.d_inner;
    a.batch = (int32_t)q.batch;
    a.n_seg = (int32_t)((a.span_len + kM3Seg - 1) / kM3Seg);
    a.n_spans = S;
    a.units = (int32_t)units;
    const dim3 block(64 * m3_groups<N, ROT>());
    hipError_t e;
    if (S > 1) {
        a.h_in = q.h_in;
        a.mu_in = q.mu_in;
        a.mu_loc = q.mu_loc;
        a.du_edge = q.du_edge;
        a.du_lb = q.du_lb;
        // the adjoint span pass (spans 1 .. S - 1), then the adjoint entering every span
        const dim3 grid((uint32_t)(units * (S - 1)));
        if (q.z)
            hipLaunchKernelGGL((m3_adjoint_span_kernel<T, N, ROT, true>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((m3_adjoint_span_kernel<T, N, ROT, false>), grid, block, 0, stream, a);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
        const int64_t columns = q.batch * q.d_inner * N;
        const int64_t threads = ROT ? columns / 2 : columns;
        hipLaunchKernelGGL(m3_mu_carry_kernel, dim3((uint32_t)((threads + 255) / 256)), dim3(256),
                           0, stream, q.ws_decay, ROT ? q.ws_rot : nullptr, q.mu_loc, q.dh_last,
                           q.mu_in, columns, (int32_t)S);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    const dim3 grid((uint32_t)(units * S));
    if (S > 1) {
        if (q.z)
            hipLaunchKernelGGL((scan_bwd_m3_kernel<T, N, ZOH, TRAP, ROT, true, true>), grid, block,
                               0, stream, a);
        else
            hipLaunchKernelGGL((scan_bwd_m3_kernel<T, N, ZOH, TRAP, ROT, false, true>), grid,
                               block, 0, stream, a);
    } else {
        if (q.z)
            hipLaunchKernelGGL((scan_bwd_m3_kernel<T, N, ZOH, TRAP, ROT, true, false>), grid,
                               block, 0, stream, a);
        else
            hipLaunchKernelGGL((scan_bwd_m3_kernel<T, N, ZOH, TRAP, ROT, false, false>), grid,
                               block, 0, stream, a);
    }
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    constexpr int V = 2 * N + (ROT ? N / 2 : 0);
    const int64_t nred = q.batch * q.L * V + (TRAP ? q.batch * N : 0);
    hipLaunchKernelGGL((m3_reduce_kernel<T>), dim3((uint32_t)((nred + 255) / 256)), dim3(256), 0,
                       stream, q.part, q.bprev_part, (T *)q.dB, (T *)q.dC, (T *)q.dtheta,
                       TRAP ? (T *)q.dB_prev : (T *)nullptr, q.batch, q.L, (int32_t)N,
                       (int32_t)V, (int32_t)tiles, a.span_len, TRAP ? (int32_t)S : 1);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    const int64_t np = q.d_inner * N + q.d_inner;
    hipLaunchKernelGGL(m3_reduce_params_kernel, dim3((uint32_t)((np + 255) / 256)), dim3(256), 0,
                       stream, q.dA_part, q.dDb_part, q.dA, q.dD, q.dbias, q.batch * S, q.d_inner,
                       (int64_t)N);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    if (TRAP && S > 1) {
        const int64_t bd = q.batch * q.d_inner;
        const int64_t n = (int64_t)(S - 1) * bd;
        hipLaunchKernelGGL((m3_du_edge_kernel<T>), dim3((uint32_t)((n + 255) / 256)), dim3(256), 0,
                           stream, q.du_edge, q.du_lb, (T *)q.du, bd, q.L, (int32_t)q.d_inner,
                           a.span_len, (int32_t)S);
        e = hipGetLastError();
    }
    return e;
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
                              bool rot, const M3Plan &plan, size_t off[15])
{
    auto al = [](size_t n) { return (n + 255) / 256 * 256; };
    const size_t units = (size_t)batch * (size_t)((d_inner + 63) / 64);
    const size_t S = (size_t)plan.n_spans;
    // segments per block: of the whole sequence, or of one span
    const size_t n_seg = S > 1 ? (size_t)(plan.span_len / kM3Seg)
                               : (size_t)((L + kM3Seg - 1) / kM3Seg);
    const size_t N = (size_t)d_state, V = 2 * N + (rot ? N / 2 : 0), f = sizeof(float);
    const size_t bd = (size_t)batch * (size_t)d_inner, bdn = bd * N;
    size_t sz[14] = {};
    sz[0] = al(S * units * n_seg * N * 64 * f); // stored states
    sz[1] = al(units * (size_t)L * V * f);      // dB, dC, dtheta tile partials
    sz[2] = al(S * units * N * f);              // look-back dB shares (dB_prev at span 0)
    sz[3] = al(S * bdn * f);                    // dA per (span, batch row)
    sz[4] = al(S * bd * 2 * f);                 // dD, dbias per (span, batch row)
    if (S > 1) {
        const size_t rows = (size_t)L + (size_t)plan.fwd_chunk;
        sz[5] = al((size_t)batch * rows * (2 * N + (rot ? N / 2 : 0)) * f);
        sz[6] = sz[7] = sz[8] = al(S * bdn * f);
        sz[9] = rot ? al(2 * S * bdn * f) : 0;
        sz[10] = sz[11] = al(S * bdn * f);
        sz[12] = sz[13] = al(S * bd * f);
    }
    off[0] = 0;
    for (int i = 0; i < 14; ++i)
        off[i + 1] = off[i] + sz[i];
    return L > 0 ? off[14] : 0;
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
