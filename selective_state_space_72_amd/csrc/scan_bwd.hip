// Backward pass of the selective scan (Euler discretisation) for gfx950.
//
// Gradients of the forward operation of scan_kernels.hip with respect to all of its
// inputs, given dy (and optionally the gradient of the final state).  With
// mu_t[n] = dLoss/dh_t[n], s_t = sum_n C_t[n] h_t[n] + D u_t, ds_t = dy_t silu(z_t):
//   mu_t = Abar_{t+1} mu_{t+1} + ds_t C_t          (mu_{L-1} = dh_last + ds_{L-1} C_{L-1})
//   dDelta_t = sum_n mu_t (A Abar_t h_{t-1} + B_t u_t),  du_t = ds_t D + Delta_t sum_n mu_t B_t
//   dB_t[n] = sum_d mu_t Delta_t u_t,  dC_t[n] = sum_d ds_t h_t,  dA = sum mu_t Delta_t Abar_t h_{t-1}
//   dD = sum ds_t u_t,  dz_t = dy_t s_t silu'(z_t),  ddelta_t = dDelta_t sigmoid(delta_t + bias)
//   dh0 = Abar_0 mu_0.
// This is the chain rule applied to the recurrence of "Understanding Mamba"
// (aiattnstudio.link, sections 4.4 and 5.2), whose section 7.3 (and section 4.4 of the
// hnwysp.cn slides) names the approach taken for the states: they are recomputed in the
// backward pass rather than stored for every step.
//
// Work decomposition: the forward scalar kernel's -- one block per (batch row, 64-channel
// tile), lane = channel, wave g owns state indices [g*NQ, (g+1)*NQ).  Each block
//   1. runs the recurrence forward once and stores the state entering every segment of
//      S steps (a checkpoint per lane and state index, in the workspace);
//   2. walks the segments backwards: recomputes the segment's states and decay factors
//      into registers from its checkpoint, then runs the adjoint recurrence mu backwards
//      through it.
// Per (step, channel) quantities (Delta, Delta*u, ds) are computed once and shared
// through LDS, as are B and C (a wave loads its segment's values with one load per lane,
// a segment ahead, and reads them back as broadcasts).  The per-wave partial sums over
// state indices (readout, sum mu B, sum A mu Abar h) are summed across waves through LDS
// in a fixed order.  dB and dC need sums over the block's 64 channels (the lanes), one per
// (step, state index) and wave; each wave writes one partial per (tile, t, n) and a second
// kernel sums the tiles, and dA, dD, dbias over the batch rows and spans.  The sums over
// lanes go either through LDS (LR: every 16 values per lane the wave writes them as rows
// of a slab, each lane adds 16 entries of one row and two lane exchanges join the row's
// four quarters -- about one VALU operation per value) or through a transposed butterfly
// in registers (every exchange halves the values a lane holds, about three operations per
// value, but no LDS).
//
// When the (batch row, tile) units are too few to fill the device, the sequence is split
// into spans that run as separate blocks: the forward span pass and carry give the state
// entering each span, the adjoint span pass below and its reverse carry give the mu
// entering each span from its end, and each block then covers only its span's steps.
// Nothing is accumulated with atomics: results are bitwise reproducible.
#include <type_traits>

#include "device_math.h"
#include "scan_common.h"
#include "scan_bwd.h"

namespace mambascan {
namespace {

constexpr int kRH = 8;  // reverse steps per cross-wave exchange (and per lane reduction)
constexpr int kTCF = 8; // steps per chunk of the checkpointing forward pass

struct BwdArgs {
    const void *u, *delta, *z, *dy, *B, *C;
    const float *A, *D, *bias, *h0, *dh_last;
    void *du, *ddelta, *dz;
    float *dh0;
    float *ckpt;     // [block][segment][n][lane]
    float *dbc_part; // [(block * L + t) * 2N + {n, N + n}]: this tile's dB, dC
    float *dA_part;  // [span][b][d][n]
    float *dDb_part; // [span][b][d][2]: dD, dbias of one (span, batch row)
    const float *h_in;  // [span][b][d][n]: state entering each span (spans > 0), or NULL
    const float *mu_in; // [span][b][d][n]: adjoint entering each span from its end, or NULL
                        // (then dh_last, a single span)
    int64_t L;
    int32_t Dn, batch, n_seg; // n_seg: segments of the whole sequence
    int32_t span_len, n_spans; // span_len: a multiple of the segment length
};

// Value of lane (lane ^ pattern) for the butterfly's partner patterns.  Lane bits 3, 2, 1
// and 0 use DPP row_mirror (l ^ 15 within a row), row_half_mirror (l ^ 7 within 8 lanes),
// quad_perm [3,2,1,0] (l ^ 3) and quad_perm [1,0,3,2] (l ^ 1): each flips the named bit
// and only lower ones, so applied from bit 3 down, partners always hold the same value
// indices.  Bits 4 and 5 use lane shuffles.
template <int BIT>
__device__ __forceinline__ float partner(float v)
{
    const int x = __builtin_bit_cast(int, v);
    if constexpr (BIT == 3)
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, true));
    else if constexpr (BIT == 2)
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, true));
    else if constexpr (BIT == 1)
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x1B, 0xF, 0xF, true));
    else if constexpr (BIT == 0)
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, true));
    else if constexpr (BIT == 4)
        return __shfl_xor(v, 16);
    else
        return __shfl_xor(v, 32);
}

// One butterfly exchange: lanes whose bit BIT is clear keep value index `lo`, the others
// `hi`; each adds its partner's copy of the index it keeps.
template <int BIT>
__device__ __forceinline__ float halve(float lo, float hi, int lane)
{
    const bool up = (lane >> BIT) & 1;
    const float keep = up ? hi : lo;
    const float send = up ? lo : hi;
    return keep + partner<BIT>(send);
}

template <typename T>
__device__ __forceinline__ T zero_val()
{
    return T(0);
}

// AB: keep the segment's decay factors in registers (else recompute them in the adjoint
// sweep, one more exp per element, to save S * NQ registers).  WPE: waves per SIMD the
// register allocation targets.  LR: the dB/dC lane sums through an LDS slab per wave (16
// rows of 64 lanes; else the register butterfly).  CKE: the checkpoints hold every segment's
// entering state already (written by the forward scan): no forward pass here, and a later
// span's entering state is its first checkpoint.  ZOH: the zero-order-hold input term
// beta B u, beta = expm1(Delta A) / A (d beta / dDelta = Abar, d beta / dA = Delta^2 psi(Delta
// A) with psi(x) = (x e^x - e^x + 1) / x^2), which needs one more per-wave partial sum per
// step (sum Abar mu B, for dDelta).
template <typename T, int N, int NW, int S, bool AB, int WPE, bool LR, bool GATED, bool CKE,
          bool ZOH = false>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(WPE)))
scan_bwd_kernel(BwdArgs p)
{
    static_assert(!(ZOH && CKE), "the forward stores checkpoints for the Euler rule only");
    constexpr int NPL = ZOH ? 4 : 3; // per-wave partial sums per (step, channel)
    constexpr int NQ = N / NW;     // state indices per lane
    constexpr int BCW = 2 * NQ;    // B then C per step; also dB/dC values per step
    constexpr int RH = kRH;
    constexpr int NH = S / RH;     // reverse parts per segment
    constexpr int KP = S / NW;     // a segment's (step, channel) items per lane
    constexpr int KF = kTCF / NW;  // a forward chunk's items per lane
    constexpr int KE = RH / NW;    // a reverse part's items per lane
    static_assert(NQ >= 1 && N % NW == 0 && S % RH == 0 && RH % NW == 0 && kTCF % NW == 0 &&
                  S % kTCF == 0, "bad variant");
    static_assert(BCW == 2 || BCW == 4 || BCW == 8, "butterfly handles 2 to 8 values per step");
    static_assert(S * BCW <= 64 && kTCF * NQ <= 64, "one lane load per B/C value");

    __shared__ float4 s_in[S][64];       // Delta, Delta*u, ds (and u: ZOH) per (step, channel)
    // readout, sum mu B (ZOH: sum mu beta B), sum A mu Abar h (and ZOH: sum Abar mu B)
    __shared__ float s_p[NPL][RH][NW][64];
    __shared__ float s_bc[NW][S * BCW];  // this segment's B, C per wave: [step][B(NQ), C(NQ)]
    // LR: per wave 16 rows (a group of 16 / BCW steps' values) of 64 lanes, padded by 16
    // bytes so that the row reads below (16 consecutive lanes of one row per lane, rows
    // lane % 16) fall in distinct banks
    constexpr int kRow = 68;
    __shared__ float s_r[LR ? NW : 1][LR ? 16 * kRow : 1];

    const int lane = threadIdx.x & 63;
    const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tiles = (p.Dn + 63) / 64;
    const int units = tiles * p.batch;
    const int unit = blockIdx.x % units;    // = tile * batch + b
    const int span = blockIdx.x / units;
    const int b = unit % p.batch;
    const int tile = unit / p.batch;
    const int Dn = p.Dn;
    const int d = tile * 64 + lane;
    const bool dvalid = d < Dn;
    const int dc = dvalid ? d : Dn - 1; // tail lanes compute on a valid channel with dy = 0
    const int n0 = g * NQ;
    const int64_t L = p.L;

    // this block's steps [t_begin, t_end) = segments [seg_lo, seg_hi)
    const int64_t t_begin = (int64_t)span * p.span_len;
    const int64_t t_end = min(t_begin + (int64_t)p.span_len, L);
    const int seg_lo = (int)(t_begin / S);
    const int seg_hi = (int)((t_end + S - 1) / S);

    float a2[NQ], an[NQ], ia[NQ], h[NQ], hstart[NQ];
    const int64_t col_c = ((int64_t)b * Dn + dc) * N + n0;       // (b, dc, n0)
    const int64_t span_col = (int64_t)span * p.batch * Dn * N;   // span offset of [span][b][d][n]
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const float av = p.A[(int64_t)dc * N + n0 + q];
        a2[q] = av * kLog2e;
        an[q] = av;
        ia[q] = ZOH ? 1.0f / av : 0.0f;
        if (span == 0)
            h[q] = p.h0 ? p.h0[col_c + q] : 0.0f;
        else if constexpr (CKE) // unused: the span's first segment reads its checkpoint
            h[q] = 0.0f;
        else
            h[q] = p.h_in[span_col + col_c + q];
        hstart[q] = h[q];
    }
    const float bias_d = p.bias ? p.bias[dc] : 0.0f;
    const float D_d = p.D ? p.D[dc] : 0.0f;

    const int64_t row0 = (int64_t)b * L * Dn; // element offset of (b, 0, 0)
    const T *ub = (const T *)p.u + row0 + dc;
    const T *db = (const T *)p.delta + row0 + dc;
    const T *zb = GATED ? (const T *)p.z + row0 + dc : nullptr;
    const T *gb = (const T *)p.dy + row0 + dc;
    float *ck = p.ckpt + (int64_t)unit * p.n_seg * N * 64; // [global segment][n][lane]

    // One B/C value per lane: for a segment, lane l < S*BCW holds step l / BCW, value
    // l % BCW (B for the first NQ, then C) of this wave's state indices; for a forward
    // chunk, lane l < kTCF*NQ holds B of step l / NQ, state n0 + l % NQ.  The prefetch
    // loads here and in rfetch are unconditional, from rows clamped into the sequence
    // (steps past its end and lanes past the values are never used; the tail lanes' dy is
    // masked where it is used): a load inside a branch makes the compiler wait for every
    // outstanding memory operation where the branch joins (measured 4 % / 8 % faster for
    // the backward without / with stored checkpoints at the large prefill).  They return
    // the raw element, widened where it is stored to LDS: widening at the load made the
    // compiler wait for it, and for every load issued before it, right after the issue
    // (9 % / 5 % faster).
    const int r_step = lane / BCW, r_i = lane % BCW;
    const T *r_src = (const T *)(r_i < NQ ? p.B : p.C) + (int64_t)b * L * N + n0 + r_i % NQ;
    auto bc_fetch = [&](int64_t t0) -> T { return r_src[min(t0 + r_step, L - 1) * N]; };
    const int f_step = lane / NQ, f_q = lane % NQ;
    const T *f_src = (const T *)p.B + (int64_t)b * L * N + n0 + f_q;
    auto b_fetch = [&](int64_t t0) -> T { return f_src[min(t0 + f_step, L - 1) * N]; };

    // ---- 1. forward pass: checkpoints at the start of segments seg_lo+1 .. seg_hi-1 ----
    if constexpr (!CKE) {
        // (Delta, Delta*u) and B of two chunks, alternating; aliases s_p
        float2 *s_f = reinterpret_cast<float2 *>(&s_p[0][0][0][0]);   // [2][kTCF][64]
        float *s_fb = reinterpret_cast<float *>(&s_p[2][0][0][0]);    // [2][NW][kTCF * NQ]
        const int64_t LF = (int64_t)(seg_hi - 1) * S;                   // whole segments only
        T fu[KF], fd[KF];
        T fb = 0;
        auto ffetch = [&](int64_t t0) {
#pragma unroll
            for (int k = 0; k < KF; ++k) {
                const int64_t t = t0 + g + k * NW;
                fu[k] = ub[t * Dn];
                fd[k] = db[t * Dn];
            }
            fb = b_fetch(t0);
        };
        if (LF > t_begin)
            ffetch(t_begin);
        int par = 0;
        for (int64_t t0 = t_begin; t0 < LF; t0 += kTCF) {
            // wave priorities per phase (see the segment below): the chunk's updates 2,
            // its prologue 0
            __builtin_amdgcn_s_setprio(0);
#pragma unroll
            for (int k = 0; k < KF; ++k) {
                const int tl = g + k * NW;
                const float dl = softplus_act<T>(widen(fd[k]) + bias_d);
                // (Delta, Delta u); ZOH: (Delta, u)
                s_f[(par * kTCF + tl) * 64 + lane] =
                    make_float2(dl, ZOH ? widen(fu[k]) : dl * widen(fu[k]));
            }
            if (lane < kTCF * NQ)
                s_fb[(par * NW + g) * (kTCF * NQ) + lane] = widen(fb);
            if (t0 + kTCF < LF)
                ffetch(t0 + kTCF);
            __syncthreads();
            const float *bs = s_fb + (par * NW + g) * (kTCF * NQ);
            __builtin_amdgcn_s_setprio(2);
#pragma unroll
            for (int tl = 0; tl < kTCF; ++tl) {
                const float2 w = s_f[(par * kTCF + tl) * 64 + lane];
#pragma unroll
                for (int i = 0; i < NQ; ++i) {
                    const float a = decay_exp2(w.x, a2[i]);
                    const float bu = ZOH ? zoh_input(w.x * an[i], a, w.x * w.y, w.y * ia[i]) : w.y;
                    h[i] = __builtin_fmaf(a, h[i], bu * bs[tl * NQ + i]);
                }
            }
            if ((t0 + kTCF) % S == 0) {
                const int64_t seg = (t0 + kTCF) / S;
#pragma unroll
                for (int i = 0; i < NQ; ++i)
                    ck[(seg * N + n0 + i) * 64 + lane] = h[i];
            }
            par ^= 1;
        }
        __syncthreads(); // s_f and s_fb alias s_p
    }

    // ---- 2. segments in reverse ----
    float mu[NQ], dA[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        if (!dvalid)
            mu[q] = 0.0f;
        else if (p.mu_in)
            mu[q] = p.mu_in[span_col + col_c + q];
        else
            mu[q] = p.dh_last ? p.dh_last[col_c + q] : 0.0f;
        dA[q] = 0.0f;
    }
    float dD_acc = 0.0f, db_acc = 0.0f;

    // inputs of the next segment to process, loaded one segment ahead
    T ru[KP], rd[KP], rz[KP], rg[KP];
    T bcv = 0;
    float hnext[NQ];
    auto rfetch = [&](int seg) {
        const int64_t t0 = (int64_t)seg * S;
#pragma unroll
        for (int k = 0; k < KP; ++k) {
            const int64_t t = t0 + g + k * NW;
            const int64_t tc = min(t, L - 1);
            ru[k] = ub[tc * Dn];
            rd[k] = db[tc * Dn];
            if (GATED)
                rz[k] = zb[tc * Dn];
            rg[k] = gb[tc * Dn];
        }
        bcv = bc_fetch(t0);
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            hnext[q] = (CKE ? seg == 0 : seg == seg_lo)
                           ? hstart[q] : ck[((int64_t)seg * N + n0 + q) * 64 + lane];
    };
    if (seg_hi > seg_lo)
        rfetch(seg_hi - 1);

    // One segment: t0 its first step; PARTIAL when it has fewer than S steps (the last).
    auto segment = [&](auto PARTIAL_, int seg) {
        constexpr bool PARTIAL = decltype(PARTIAL_)::value;
        const int64_t t0 = (int64_t)seg * S;
        const int nt = PARTIAL ? (int)(L - t0) : S;

        // prologue: per (step, channel) values, kept by this lane for the epilogue
        // Wave priorities per phase (the SIMD issues the ready wave of highest priority):
        // adjoint 3, epilogue 2, recompute 1, prologue 0.  Measured at the large prefill
        // (three blocks of four waves per CU): 2.98 / 2.25 ms (own / stored checkpoints)
        // against 3.33 / 2.62 ms with equal priorities; results unchanged.
        __builtin_amdgcn_s_setprio(0);
        float e_u[KP], e_dl[KP], e_sig[KP], e_ds[KP], e_dyg[KP];
#pragma unroll
        for (int k = 0; k < KP; ++k) {
            const int tl = g + k * NW;
            const float uu = widen(ru[k]);
            const float v = widen(rd[k]) + bias_d;
            const float dl = softplus_act<T>(v);
            const float dyv = dvalid ? widen(rg[k]) : 0.0f; // tail lanes: no gradient
            float gate = 1.0f, dgate = 0.0f;
            if (GATED) {
                const float zz = widen(rz[k]);
                const float sz = hw_rcp(1.0f + hw_exp2(-zz * kLog2e));
                gate = zz * sz;
                dgate = sz * __builtin_fmaf(zz, 1.0f - sz, 1.0f);
            }
            const float ds = dyv * gate;
            e_u[k] = uu;
            e_dl[k] = dl;
            e_sig[k] = hw_rcp(1.0f + hw_exp2(-v * kLog2e)); // softplus'(v)
            e_ds[k] = ds;
            e_dyg[k] = dyv * dgate;
            s_in[tl][lane] = make_float4(dl, dl * uu, ds, ZOH ? uu : 0.0f);
        }
        if (lane < S * BCW)
            s_bc[g][lane] = widen(bcv);
        float hin[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            hin[q] = hnext[q];
        if (seg > seg_lo)
            rfetch(seg - 1);
        __syncthreads();

        // recompute the segment's states and decay factors
        __builtin_amdgcn_s_setprio(1);
        float hs[S][NQ], ab[AB ? S : 1][NQ];
        {
            float hc[NQ];
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                hc[q] = hin[q];
#pragma unroll
            for (int T_ = 0; T_ < S; ++T_) {
                if (!PARTIAL || T_ < nt) {
                    const float4 w = s_in[T_][lane];
#pragma unroll
                    for (int q = 0; q < NQ; ++q) {
                        const float a = decay_exp2(w.x, a2[q]);
                        const float bu = ZOH ? zoh_input(w.x * an[q], a, w.y, w.w * ia[q]) : w.y;
                        hc[q] = __builtin_fmaf(a, hc[q], bu * s_bc[g][T_ * BCW + q]);
                        if constexpr (AB)
                            ab[T_][q] = a;
                        hs[T_][q] = hc[q];
                    }
                }
            }
        }

        // (re-read Delta, B, C from LDS below rather than keeping the recompute's copies live)
        asm volatile("" ::: "memory");

        // adjoint recurrence, last part first
#pragma unroll
        for (int part = NH - 1; part >= 0; --part) {
            __builtin_amdgcn_s_setprio(3);
            float pend[BCW], r1[4][BCW], r2[2][BCW], r3[BCW];
#pragma unroll
            for (int tl = RH - 1; tl >= 0; --tl) {
                const int T_ = part * RH + tl;
                float xv[BCW];
                float yp = 0.0f, p1 = 0.0f, p2 = 0.0f, p3 = 0.0f;
#pragma unroll
                for (int i = 0; i < BCW; ++i)
                    xv[i] = 0.0f;
                if (!PARTIAL || T_ < nt) {
                    const float4 w = s_in[T_][lane]; // Delta, Delta*u, ds
#pragma unroll
                    for (int q = 0; q < NQ; ++q) {
                        const float bq = s_bc[g][T_ * BCW + q];
                        const float cq = s_bc[g][T_ * BCW + NQ + q];
                        yp = __builtin_fmaf(cq, hs[T_][q], yp);
                        mu[q] = __builtin_fmaf(w.z, cq, mu[q]); // mu_t
                        xv[NQ + q] = w.z * hs[T_][q];           // dC
                        const float hp = T_ == 0 ? hin[q] : hs[T_ > 0 ? T_ - 1 : 0][q];
                        const float abq = AB ? ab[AB ? T_ : 0][q] : decay_exp2(w.x, a2[q]);
                        const float m2 = mu[q] * abq;           // Abar_t mu_t
                        const float qv = m2 * hp;
                        p2 = __builtin_fmaf(an[q], qv, p2);
                        if constexpr (ZOH) {
                            // beta = Delta phi(x) and d beta / dA = Delta^2 psi(x), x = Delta A:
                            // series below |x| = 1/16, else from Abar (as the forward)
                            const float x = w.x * an[q];
                            const float beta = zoh_input(x, abq, w.x, ia[q]);
                            const float psi = __builtin_fmaf(
                                x, __builtin_fmaf(x, __builtin_fmaf(x, __builtin_fmaf(
                                    x, 1.0f / 144.0f, 1.0f / 30.0f), 1.0f / 8.0f), 1.0f / 3.0f),
                                0.5f);
                            const float dbA = __builtin_fabsf(x) < 0.0625f
                                                  ? w.x * w.x * psi
                                                  : (w.x * abq - beta) * ia[q];
                            const float mb = mu[q] * bq;
                            p1 = __builtin_fmaf(mb, beta, p1);  // sum mu beta B
                            p3 = __builtin_fmaf(m2, bq, p3);    // sum Abar mu B
                            xv[q] = mu[q] * beta * w.w;         // dB
                            dA[q] = __builtin_fmaf(w.x, qv, __builtin_fmaf(mb * w.w, dbA, dA[q]));
                        } else {
                            p1 = __builtin_fmaf(mu[q], bq, p1);
                            xv[q] = mu[q] * w.y;                // dB
                            dA[q] = __builtin_fmaf(w.x, qv, dA[q]);
                        }
                        mu[q] = m2;
                    }
                }
                s_p[0][tl][g][lane] = yp;
                s_p[1][tl][g][lane] = p1;
                s_p[2][tl][g][lane] = p2;
                if constexpr (ZOH)
                    s_p[ZOH ? 3 : 0][tl][g][lane] = p3;

                if constexpr (LR) {
                    // rows (tl % GS) * BCW + i of the slab; after the group's first step
                    // (the loop runs backwards) lane l sums row l % 16 over lanes
                    // 16 (l / 16) .. + 15, and the four quarters are joined across lanes
                    // (lane permutes: no LDS round trip)
                    constexpr int GS = 16 / BCW;
                    float *slab = &s_r[LR ? g : 0][0];
#pragma unroll
                    for (int i = 0; i < BCW; ++i)
                        slab[((tl % GS) * BCW + i) * kRow + lane] = xv[i];
                    if (tl % GS == 0) {
                        const float4 *src = reinterpret_cast<const float4 *>(
                            slab + (lane & 15) * kRow + (lane >> 4) * 16);
                        const float4 c0 = src[0], c1 = src[1], c2 = src[2], c3 = src[3];
                        float v = ((c0.x + c0.y) + (c0.z + c0.w)) + ((c1.x + c1.y) + (c1.z + c1.w));
                        v += ((c2.x + c2.y) + (c2.z + c2.w)) + ((c3.x + c3.y) + (c3.z + c3.w));
                        v = lane_pair_sum(v);
                        const int o = lane & 15, j = o % BCW;
                        const int64_t t = t0 + part * RH + tl + o / BCW;
                        if (lane < 16 && (!PARTIAL || t < L)) {
                            const int kind = j / NQ, q = j % NQ;
                            p.dbc_part[((int64_t)unit * L + t) * (2 * N) + kind * N + n0 + q] = v;
                        }
                    }
                } else if (tl & 1) {
                    // butterfly over the steps of this part: step bit 0, 1, 2 on lane bit 3, 2, 1
#pragma unroll
                    for (int i = 0; i < BCW; ++i)
                        pend[i] = xv[i];
                } else {
                    const int m = tl >> 1;
#pragma unroll
                    for (int i = 0; i < BCW; ++i)
                        r1[m][i] = halve<3>(xv[i], pend[i], lane);
                    if ((m & 1) == 0) {
#pragma unroll
                        for (int i = 0; i < BCW; ++i)
                            r2[m >> 1][i] = halve<2>(r1[m][i], r1[m + 1][i], lane);
                        if (m == 0) {
#pragma unroll
                            for (int i = 0; i < BCW; ++i)
                                r3[i] = halve<1>(r2[0][i], r2[1][i], lane);
                        }
                    }
                }
            }
            // value bits (kind, state) on lane bits 0, 4, 5; the remaining lane bits sum
            if constexpr (!LR) {
            float v;
            if constexpr (BCW == 2) {
                v = halve<0>(r3[0], r3[1], lane);
                v += partner<4>(v);
                v += partner<5>(v);
            } else if constexpr (BCW == 4) {
                const float s0 = halve<0>(r3[0], r3[1], lane);
                const float s1 = halve<0>(r3[2], r3[3], lane);
                v = halve<4>(s0, s1, lane);
                v += partner<5>(v);
            } else {
                float s1[4], s2[2];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    s1[i] = halve<0>(r3[2 * i], r3[2 * i + 1], lane);
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    s2[i] = halve<4>(s1[2 * i], s1[2 * i + 1], lane);
                v = halve<5>(s2[0], s2[1], lane);
            }
            {
                const int tlo = ((lane >> 3) & 1) | (((lane >> 2) & 1) << 1) | (((lane >> 1) & 1) << 2);
                int j = lane & 1;
                bool writer;
                if constexpr (BCW == 2) {
                    writer = (lane >> 4) == 0;
                } else if constexpr (BCW == 4) {
                    j |= ((lane >> 4) & 1) << 1;
                    writer = (lane >> 5) == 0;
                } else {
                    j |= ((lane >> 4) & 1) << 1;
                    j |= ((lane >> 5) & 1) << 2;
                    writer = true;
                }
                const int64_t t = t0 + part * RH + tlo;
                if (writer && (!PARTIAL || t < L)) {
                    const int kind = j / NQ, q = j % NQ;
                    p.dbc_part[((int64_t)unit * L + t) * (2 * N) + kind * N + n0 + q] = v;
                }
            }
            }
            __syncthreads();

            // epilogue of this part: sums over waves, per (step, channel) gradients
            __builtin_amdgcn_s_setprio(2);
#pragma unroll
            for (int k = part * KE; k < (part + 1) * KE; ++k) {
                const int tl = g + k * NW;
                const int lt = tl - part * RH;
                float Y = s_p[0][lt][0][lane], P1 = s_p[1][lt][0][lane], P2 = s_p[2][lt][0][lane];
                float P3 = ZOH ? s_p[ZOH ? 3 : 0][lt][0][lane] : 0.0f;
#pragma unroll
                for (int w = 1; w < NW; ++w) {
                    Y += s_p[0][lt][w][lane];
                    P1 += s_p[1][lt][w][lane];
                    P2 += s_p[2][lt][w][lane];
                    if constexpr (ZOH)
                        P3 += s_p[ZOH ? 3 : 0][lt][w][lane];
                }
                if (!PARTIAL || tl < nt) {
                    const int64_t t = t0 + tl;
                    // dDelta = sum mu (A Abar h' + B u) (Euler), sum Abar mu (A h' + B u) (ZOH);
                    // du = ds D + Delta sum mu B (Euler), ds D + sum mu beta B (ZOH)
                    const float ddt = __builtin_fmaf(e_u[k], ZOH ? P3 : P1, P2);
                    const float dd = ddt * e_sig[k];
                    const float duv = __builtin_fmaf(e_ds[k], D_d, ZOH ? P1 : e_dl[k] * P1);
                    dD_acc = __builtin_fmaf(e_ds[k], e_u[k], dD_acc);
                    db_acc += dd;
                    if (dvalid) {
                        const int64_t o = row0 + t * Dn + d;
                        store_val((T *)p.du, o, duv);
                        store_val((T *)p.ddelta, o, dd);
                        if (GATED)
                            store_val((T *)p.dz, o, e_dyg[k] * __builtin_fmaf(D_d, e_u[k], Y));
                    }
                }
            }
            if (part > 0)
                __syncthreads(); // the next part rewrites s_p
        }
    };

    int seg = seg_hi - 1;
    if (seg >= seg_lo && L - (int64_t)seg * S < S) {
        segment(std::true_type{}, seg);
        --seg;
    }
    for (; seg >= seg_lo; --seg)
        segment(std::false_type{}, seg);

    // ---- 3. per-block results ----
    if (dvalid) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            p.dA_part[span_col + col_c + q] = dA[q];
            if (p.dh0 && span == 0)
                p.dh0[col_c + q] = mu[q]; // Abar_0 mu_0
        }
    }
    __syncthreads();
    s_p[0][0][g][lane] = dD_acc;
    s_p[1][0][g][lane] = db_acc;
    __syncthreads();
    if (g == 0 && dvalid) {
        float sD = s_p[0][0][0][lane], sb = s_p[1][0][0][lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) {
            sD += s_p[0][0][w][lane];
            sb += s_p[1][0][w][lane];
        }
        const int64_t o = (((int64_t)span * p.batch + b) * Dn + d) * 2;
        p.dDb_part[o + 0] = sD;
        p.dDb_part[o + 1] = sb;
    }
}

// Adjoint summaries of spans 1 .. n_spans-1 (a longer sequence is split into spans so
// that more blocks share the work): over span k, the recurrence mu <- Abar_t (mu +
// ds_t C_t) run from the span's last step to its first is affine in the mu entering at
// the end, mu_out = dec_k mu_in + loc_k, with dec_k = exp(A sum_{t in k} Delta_t) and
// loc_k the result for mu_in = 0.  Layout of dec and loc: [span][b][d][n].  Same block
// shape as the main kernel; (Delta, ds) and C are exchanged through LDS per chunk.
struct MuSumArgs {
    const void *delta, *z, *dy, *C;
    const float *A, *bias;
    float *dec, *loc;
    int64_t L;
    int32_t Dn, batch, span_len;
};

template <typename T, int N, int NW, bool GATED>
__global__ void __launch_bounds__(64 * NW)
scan_bwd_musum_kernel(MuSumArgs p)
{
    constexpr int NQ = N / NW;
    constexpr int KF = kTCF / NW;
    __shared__ float2 s_m[2][kTCF][64];          // Delta, ds per (step, channel)
    __shared__ float s_c[2][NW][kTCF * NQ];      // C of the chunk per wave

    const int lane = threadIdx.x & 63;
    const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tiles = (p.Dn + 63) / 64;
    const int units = tiles * p.batch;
    const int unit = blockIdx.x % units;
    const int span = 1 + blockIdx.x / units;    // spans 1 .. n_spans-1
    const int b = unit % p.batch;
    const int tile = unit / p.batch;
    const int Dn = p.Dn;
    const int d = tile * 64 + lane;
    const bool dvalid = d < Dn;
    const int dc = dvalid ? d : Dn - 1;
    const int n0 = g * NQ;
    const int64_t L = p.L;
    const int64_t t_begin = (int64_t)span * p.span_len;
    const int64_t t_end = min(t_begin + (int64_t)p.span_len, L);

    float a2[NQ], mu[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        a2[q] = p.A[(int64_t)dc * N + n0 + q] * kLog2e;
        mu[q] = 0.0f;
    }
    const float bias_d = p.bias ? p.bias[dc] : 0.0f;
    const int64_t row0 = (int64_t)b * L * Dn;
    const T *db = (const T *)p.delta + row0 + dc;
    const T *zb = GATED ? (const T *)p.z + row0 + dc : nullptr;
    const T *gb = (const T *)p.dy + row0 + dc;
    const int f_step = lane / NQ, f_q = lane % NQ;
    const T *c_src = (const T *)p.C + (int64_t)b * L * N + n0 + f_q;

    T rd[KF], rz[KF], rg[KF];
    float cv = 0.0f;
    auto fetch = [&](int64_t t0) {
#pragma unroll
        for (int k = 0; k < KF; ++k) {
            const int64_t t = t0 + g + k * NW;
            rd[k] = rz[k] = rg[k] = zero_val<T>();
            if (t < t_end) {
                rd[k] = db[t * Dn];
                if (GATED)
                    rz[k] = zb[t * Dn];
                if (dvalid)
                    rg[k] = gb[t * Dn];
            }
        }
        const int64_t tc = t0 + f_step;
        cv = (lane < kTCF * NQ && tc < t_end) ? load_val(c_src, tc * N) : 0.0f;
    };

    float sum_dt = 0.0f;
    // chunks from the last (possibly partial) one backwards
    const int64_t last0 = t_begin + (t_end - t_begin - 1) / kTCF * kTCF;
    if (t_end > t_begin)
        fetch(last0);
    int par = 0;
    for (int64_t t0 = last0; t0 >= t_begin; t0 -= kTCF) {
#pragma unroll
        for (int k = 0; k < KF; ++k) {
            const int tl = g + k * NW;
            const float v = widen(rd[k]) + bias_d;
            float gate = 1.0f;
            if (GATED) {
                const float zz = widen(rz[k]);
                gate = zz * hw_rcp(1.0f + hw_exp2(-zz * kLog2e));
            }
            s_m[par][tl][lane] = make_float2(softplus_act<T>(v), widen(rg[k]) * gate);
        }
        if (lane < kTCF * NQ)
            s_c[par][g][lane] = cv;
        if (t0 - kTCF >= t_begin)
            fetch(t0 - kTCF);
        __syncthreads();
        const int nt = (int)min((int64_t)kTCF, t_end - t0);
#pragma unroll
        for (int tl = kTCF - 1; tl >= 0; --tl) {
            if (tl < nt) {
                const float2 w = s_m[par][tl][lane];
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    mu[q] = __builtin_fmaf(w.y, s_c[par][g][tl * NQ + q], mu[q]);
                    mu[q] *= decay_exp2(w.x, a2[q]);
                }
                sum_dt += w.x;
            }
        }
        par ^= 1;
    }
    if (dvalid) {
        const int64_t o = (((int64_t)span * p.batch + b) * Dn + d) * N + n0;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            p.dec[o + q] = hw_exp2(a2[q] * sum_dt);
            p.loc[o + q] = mu[q];
        }
    }
}

// mu entering every span from its end: mu_in[n_spans-1] = dh_last (or 0), then
// mu_in[k-1] = dec[k] mu_in[k] + loc[k].  One thread per (b, d, n) column.
__global__ void __launch_bounds__(256)
bwd_mu_carry_kernel(const float *__restrict__ dec, const float *__restrict__ loc,
                    const float *__restrict__ dh_last, float *__restrict__ mu_in,
                    int64_t columns, int32_t n_spans)
{
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= columns)
        return;
    float g = dh_last ? dh_last[c] : 0.0f;
    for (int k = n_spans - 1; k >= 0; --k) {
        mu_in[(int64_t)k * columns + c] = g;
        if (k > 0)
            g = __builtin_fmaf(dec[(int64_t)k * columns + c], g, loc[(int64_t)k * columns + c]);
    }
}

// dB, dC: sums of the tiles' partials (fixed tile order), rounded to the input dtype.
template <typename T>
__global__ void __launch_bounds__(256)
bwd_reduce_bc_kernel(const float *__restrict__ part, T *dB, T *dC, int64_t batch, int64_t L,
                     int32_t N, int32_t tiles)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; // (b * L + t) * 2N + j
    const int64_t total = batch * L * 2 * N;
    if (i >= total)
        return;
    const int j = (int)(i % (2 * N));
    const int64_t bt = i / (2 * N);
    const int64_t b = bt / L, t = bt % L;
    // (unrolled: the loads are issued ahead, the sums stay in tile order)
    float s = 0.0f;
#pragma unroll 8
    for (int tile = 0; tile < tiles; ++tile)
        s += part[(((int64_t)tile * batch + b) * L + t) * (2 * N) + j];
    if (j < N) {
        if (dB)
            store_val(dB, bt * N + j, s);
    } else if (dC) {
        store_val(dC, bt * N + (j - N), s);
    }
}

// dA = sum over the (span, batch row) rows of dA_part; dD, dbias likewise (fixed order).
__global__ void __launch_bounds__(256)
bwd_reduce_params_kernel(const float *__restrict__ dA_part, const float *__restrict__ dDb_part,
                         float *dA, float *dD, float *dbias, int64_t batch, int64_t Dn, int64_t N)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t dn = Dn * N;
    if (i < dn) {
        if (dA) {
            float s = 0.0f;
            for (int64_t b = 0; b < batch; ++b)
                s += dA_part[b * dn + i];
            dA[i] = s;
        }
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

// (d_state, waves, segment length, decay factors in registers, waves per SIMD targeted).
// d_state 16: 4 waves of 4 state indices with the decay factors recomputed fit three
// blocks per compute unit (167 VGPRs, 33 KB LDS), so the 640 blocks of an 8 x 5120 grid
// are all resident: 4.01 ms against 4.50 ms for 8 waves of 2 state indices with stored
// decay factors (119 VGPRs but 58 KB LDS: two blocks per CU) at 8 x 4096 x 5120.
#define MAMBA_BWD_VARIANTS(X)        \
    X(4, 4, 8, true, 4, false)       \
    X(8, 8, 8, true, 4, false)       \
    X(16, 4, 8, false, 3, true)      \
    X(32, 8, 8, true, 2, false)

template <typename T, int N, int NW, int S, bool AB, int WPE, bool LR>
hipError_t launch_bwd_t(const BwdLaunch &q, hipStream_t stream)
{
    const int64_t tiles = (q.d_inner + 63) / 64;
    const int64_t units = tiles * q.batch;
    if (units <= 0 || q.L <= 0)
        return hipSuccess;
    const bool gated = q.z != nullptr;
    hipError_t e;
    if (q.n_spans > 1) {
        // adjoint summaries of spans 1 .. n_spans-1, then the reverse carry
        MuSumArgs m{};
        m.delta = q.delta;
        m.z = q.z;
        m.dy = q.dy;
        m.C = q.C;
        m.A = q.A;
        m.bias = q.bias;
        m.dec = q.mu_dec;
        m.loc = q.mu_loc;
        m.L = q.L;
        m.Dn = (int32_t)q.d_inner;
        m.batch = (int32_t)q.batch;
        m.span_len = (int32_t)q.span_len;
        const dim3 grid((uint32_t)(units * (q.n_spans - 1)));
        if (gated)
            hipLaunchKernelGGL((scan_bwd_musum_kernel<T, N, NW, true>), grid, dim3(64 * NW), 0,
                               stream, m);
        else
            hipLaunchKernelGGL((scan_bwd_musum_kernel<T, N, NW, false>), grid, dim3(64 * NW), 0,
                               stream, m);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
        const int64_t cols = q.batch * q.d_inner * N;
        hipLaunchKernelGGL(bwd_mu_carry_kernel, dim3((uint32_t)((cols + 255) / 256)), dim3(256),
                           0, stream, q.mu_dec, q.mu_loc, q.dh_last, q.mu_in, cols,
                           (int32_t)q.n_spans);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }

    BwdArgs a{};
    a.u = q.u;
    a.delta = q.delta;
    a.z = q.z;
    a.dy = q.dy;
    a.B = q.B;
    a.C = q.C;
    a.A = q.A;
    a.D = q.D;
    a.bias = q.bias;
    a.h0 = q.h0;
    a.dh_last = q.dh_last;
    a.du = q.du;
    a.ddelta = q.ddelta;
    a.dz = q.dz;
    a.dh0 = q.dh0;
    a.ckpt = q.ckpt;
    a.dbc_part = q.dbc_part;
    a.dA_part = q.dA_part;
    a.dDb_part = q.dDb_part;
    a.h_in = q.n_spans > 1 ? q.h_in : nullptr;
    a.mu_in = q.n_spans > 1 ? q.mu_in : nullptr;
    a.L = q.L;
    a.Dn = (int32_t)q.d_inner;
    a.batch = (int32_t)q.batch;
    a.n_seg = (int32_t)((q.L + S - 1) / S);
    a.n_spans = (int32_t)q.n_spans;
    a.span_len = (int32_t)(q.n_spans > 1 ? q.span_len : (q.L + S - 1) / S * S);
    const dim3 grid((uint32_t)(units * q.n_spans));
    if (q.zoh) {
        // The zero-order hold's extra per-element terms hold more registers: decay factors
        // recomputed, two waves per SIMD, and the LDS slab for the lane sums (its registers
        // would spill with the butterfly)
        constexpr bool LRZ = true;
        if (gated)
            hipLaunchKernelGGL((scan_bwd_kernel<T, N, NW, S, false, 2, LRZ, true, false, true>),
                               grid, dim3(64 * NW), 0, stream, a);
        else
            hipLaunchKernelGGL((scan_bwd_kernel<T, N, NW, S, false, 2, LRZ, false, false, true>),
                               grid, dim3(64 * NW), 0, stream, a);
    } else if (q.ck_ext) {
        if (gated)
            hipLaunchKernelGGL((scan_bwd_kernel<T, N, NW, S, AB, WPE, LR, true, true>), grid,
                               dim3(64 * NW), 0, stream, a);
        else
            hipLaunchKernelGGL((scan_bwd_kernel<T, N, NW, S, AB, WPE, LR, false, true>), grid,
                               dim3(64 * NW), 0, stream, a);
    } else if (gated) {
        hipLaunchKernelGGL((scan_bwd_kernel<T, N, NW, S, AB, WPE, LR, true, false>), grid, dim3(64 * NW), 0,
                           stream, a);
    } else {
        hipLaunchKernelGGL((scan_bwd_kernel<T, N, NW, S, AB, WPE, LR, false, false>), grid, dim3(64 * NW), 0,
                           stream, a);
    }
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    const int64_t nbc = q.batch * q.L * 2 * N;
    if (q.dB || q.dC)
        hipLaunchKernelGGL((bwd_reduce_bc_kernel<T>), dim3((uint32_t)((nbc + 255) / 256)),
                           dim3(256), 0, stream, q.dbc_part, (T *)q.dB, (T *)q.dC, q.batch,
                           q.L, (int32_t)N, (int32_t)tiles);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    const int64_t np = q.d_inner * N + q.d_inner;
    if (q.dA || q.dD || q.dbias)
        hipLaunchKernelGGL(bwd_reduce_params_kernel, dim3((uint32_t)((np + 255) / 256)),
                           dim3(256), 0, stream, q.dA_part, q.dDb_part, q.dA, q.dD, q.dbias,
                           q.batch * q.n_spans, q.d_inner, (int64_t)N);
    return hipGetLastError();
}

} // namespace

bool bwd_variant(int64_t d_state, int *waves, int *seg_len)
{
#define X(N_, W_, S_, AB_, WPE_, LR_)      \
    if (d_state == N_) {              \
        *waves = W_;                  \
        *seg_len = S_;                \
        return true;                  \
    }
    MAMBA_BWD_VARIANTS(X)
#undef X
    return false;
}

hipError_t launch_scan_bwd(const BwdLaunch &q, hipStream_t stream)
{
#define X(N_, W_, S_, AB_, WPE_, LR_)                                             \
    if (q.d_state == N_) {                                                  \
        if (q.dtype == DType::BF16)                                         \
            return launch_bwd_t<uint16_t, N_, W_, S_, AB_, WPE_, LR_>(q, stream); \
        return launch_bwd_t<float, N_, W_, S_, AB_, WPE_, LR_>(q, stream);        \
    }
    MAMBA_BWD_VARIANTS(X)
#undef X
    return hipErrorInvalidValue;
}

} // namespace mambascan
