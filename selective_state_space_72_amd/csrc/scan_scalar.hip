// Chunked selective-scan kernel for gfx950 with B and C delivered through SGPRs.
//
// Operation as in scan_kernels.hip (the selective scan of "Understanding Mamba",
// aiattnstudio.link, sections 4.4 and 5.2).  Work decomposition as the block kernel
// there -- one block is 64 consecutive channels (the 64 lanes of every wave), wave g owns
// the state indices [g*NQ, (g+1)*NQ) -- but B_t and C_t, which are uniform across a
// wave, never pass through LDS or the vector register file's broadcast paths:
//   * a staging kernel first rewrites B and C as fp32 in a layout where the values one
//     wave needs for one chunk of TC steps are contiguous: bcp[b][g][t][B(NQ), C(NQ)];
//   * the scan kernel fetches a chunk's values with a few wide scalar loads, issued
//     while the chunk's prologue computes, so the inner update uses SGPR operands:
//     v_mul (Delta*A'), v_exp_f32, v_mul (Delta*u * B), v_fmac (recurrence), v_fmac
//     (readout) -- all plain single-cycle-issue VALU forms, no DPP, no LDS reads for B/C.
//   * LDS carries only what must cross waves: Delta and Delta*u per (step, channel),
//     read once per chunk into registers, and the partial readouts, summed in a fixed
//     order in the epilogue (bitwise deterministic).
#include <type_traits>

#include "device_math.h"
#include "relay.h"
#include "scan_common.h"

namespace mambascan {
namespace {

typedef const __attribute__((address_space(4))) float *cfloat_ptr;

template <int I0, int I1, typename F>
__device__ __forceinline__ void for_c(F &&f)
{
    if constexpr (I0 < I1) {
        f(std::integral_constant<int, I0>{});
        for_c<I0 + 1, I1>(f);
    }
}

// bcp[((b * NW + g) * Lp + t) * BCW + {q, NQ + q}] = {B, C}[b, t, g * NQ + q] (0 past L;
// rows (b, t) of B and C start sB and sC elements apart),
// BCW = 2 NQ; with rotation rates (ROT) also bcp[... + 2 NQ + q / 2] = theta[b, t, (g NQ + q)
// / 2] for even q (divided by 2 pi for bf16 activations), BCW = 2 NQ + NQ / 2.  One thread per (b, g, t), t fastest, writes the BCW
// contiguous values of its row, so consecutive threads write consecutive rows.  Also zeroes
// the relay hand-off flags and fault word (n_sync words) for the scan launch that follows on
// the same stream.
template <typename T, int N, int NW, bool ROT>
__global__ void __launch_bounds__(256)
stage_bc_kernel(const T *__restrict__ Bm, const T *__restrict__ Cm, const T *__restrict__ th,
                float *__restrict__ bcp, int64_t L, int64_t Lp, int64_t total,
                uint32_t *__restrict__ sync, int32_t n_sync, int64_t sB, int64_t sC)
{
    constexpr int NQ = N / NW;
    constexpr int BCW = 2 * NQ + (ROT ? NQ / 2 : 0);
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; // over batch * NW * Lp
    if (i < n_sync)
        sync[i] = 0u;
    if (i >= total)
        return;
    const int64_t t = i % Lp;
    const int64_t bg = i / Lp; // b * NW + g
    const int g = (int)(bg % NW);
    const int64_t b = bg / NW;
    const int n0 = g * NQ;
    float v[BCW];
#pragma unroll
    for (int k = 0; k < BCW; ++k)
        v[k] = 0.0f;
    if (t < L) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            v[q] = load_val(Bm, (b * L + t) * sB + n0 + q);
            v[NQ + q] = load_val(Cm, (b * L + t) * sC + n0 + q);
        }
        if constexpr (ROT) {
#pragma unroll
            for (int k = 0; k < NQ / 2; ++k)
                v[2 * NQ + k] = load_val(th, (b * L + t) * (N / 2) + n0 / 2 + k) *
                                (sizeof(T) == 2 ? kInv2Pi : 1.0f); // see sincos_staged
        }
    }
    float *dst = bcp + i * BCW;
#pragma unroll
    for (int k = 0; k < BCW; ++k)
        dst[k] = v[k];
}

// Activations of one (batch row, span) are read and written through buffer resources
// based at the span's first time step: the lane's channel is a 32-bit vector offset and
// the step a 32-bit scalar offset, so an access needs no 64-bit vector address
// arithmetic.  The planner keeps a span's bytes (span length x d_inner x element size)
// below 2^31.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000; // gfx9 raw-buffer descriptor word 3

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ uint16_t buf_load(rsrc_t r, uint32_t vo, uint32_t so, uint16_t *)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, vo, so, 0);
}
__device__ __forceinline__ float buf_load(rsrc_t r, uint32_t vo, uint32_t so, float *)
{
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, vo, so, 0));
}
__device__ __forceinline__ void buf_store(float v, rsrc_t r, uint32_t vo, uint32_t so, uint16_t *)
{
    // round to nearest even, as store_val
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, static_cast<__bf16>(v)),
                                          r, vo, so, 0);
}
__device__ __forceinline__ void buf_store(float v, rsrc_t r, uint32_t vo, uint32_t so, float *)
{
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, vo, so, 0);
}

// Inputs of the Mamba-3 options: trapezoid mixing coefficients lam (as u), the input
// before t = 0 (u_prev (B,D), B_prev (B,N); NULL = 0) and B itself for the look-back at
// a span's or relay part's first step.  Also the checkpoint output of the CK variants.
struct Mamba3Args {
    const void *lam, *u_prev, *B_prev, *Bm;
    float *ck;       // checkpoints for the backward pass (CK variants)
    int32_t ck_nseg; // 8-step segments of the whole sequence
    float *rot_m;    // span pass with the rotation: each pair's 2x2 transition over the span
    int32_t su, sd, sz, sB; // row strides (elements) of u, delta, z, B; the planner keeps a
                            // span of rows below 2^31 bytes
};

// DISC: 0 Euler, 1 zero-order hold, 2 exponential-trapezoidal; ROT: rotation of state pairs;
// CK: also store the state entering every 8-step segment (the backward pass's checkpoints).
template <typename T, int N, int NW, int TC, int PD, bool FULL, bool GATED, int DISC, bool ROT,
          bool CK = false>
__global__ void __launch_bounds__(64 * NW)
scan_scalar_kernel(const T *__restrict__ u, const T *__restrict__ delta,
                   const T *__restrict__ z, const float *__restrict__ bcp,
                   const float *__restrict__ A, const float *__restrict__ Dv,
                   const float *__restrict__ bias, const float *h_init, int64_t h_init_stride,
                   T *__restrict__ y, float *h_last, float *__restrict__ ws_decay,
                   float *__restrict__ ws_hloc, int64_t L, int64_t Lp, int32_t Dn,
                   int64_t span_len, int32_t n_spans, int32_t first_span, int32_t tiles,
                   int32_t batch, RelayArgs relay, Mamba3Args m3)
{
    constexpr bool ZOH = DISC == 1, TRAP = DISC == 2;
    constexpr int NQ = N / NW;                 // state indices per lane
    constexpr int KPL = (TC + NW - 1) / NW;    // prologue/epilogue channel-steps per lane
    constexpr int BCW = 2 * NQ + (ROT ? NQ / 2 : 0); // B, C (and theta) per step, in bcp
    constexpr bool gated = FULL && GATED;
    static_assert(NQ >= 1 && N % NW == 0, "bad variant");
    static_assert(!ROT || NQ % 2 == 0, "rotation needs whole state pairs per wave");
    static_assert(PD % 2 == 0, "ring slots double as chunk parity");

    // Double-buffered by chunk parity so that one barrier per chunk suffices: chunk c's
    // prologue writes s_dw[c&1]; after the barrier every wave finishes chunk c-1 from
    // s_yp[(c-1)&1] and scans chunk c into s_yp[c&1].
    // (Delta, Delta*u) per (step, channel); with the zero-order hold also u; with the
    // trapezoid (Delta, lam Delta u, (1 - lam) Delta, u)
    typedef typename std::conditional<ZOH || TRAP, float4, float2>::type DW;
    __shared__ DW s_dw[2][TC][64];
    __shared__ float s_yp[FULL ? 2 : 1][TC][NW][64]; // partial readouts per (step, wave, channel)
    __shared__ float s_sdt[FULL ? 1 : NW][64];       // span pass: the waves' sums of Delta

    const int lane = threadIdx.x & 63;
    const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // Work unit of this block.  Without relay: blockIdx -> (batch row fastest, tile, span);
    // consecutive blocks go to different XCDs, so with 8 batch rows on 8 XCDs each XCD's L2
    // holds the staged B/C of one row only.  With relay the grid is ordered
    // [part 0 of each relayed unit][whole units][part 1 ...]...[part k-1 ...]: workgroups
    // are dispatched in index order, round-robin over the compute units, so the parts land
    // on different compute units from the whole units' last round, and a part only waits
    // for the previous part of its unit, which has a smaller index and therefore already
    // holds a slot (its wait is bounded all the same).
    int b, tile, span, part = -1, r_unit = 0;
    int64_t t_begin, t_end;
    const bool relayed = FULL && relay.parts > 1;
    if (relayed) {
        const int v = blockIdx.x;
        const int nu = relay.units, nr = relay.tiles;
        int unit;
        if (v < nr) {
            unit = nu - nr + v;
            part = 0;
        } else if (v < nu) {
            unit = v - nr;
        } else {
            part = 1 + (v - nu) / nr;
            unit = nu - nr + (v - nu) % nr;
        }
        r_unit = unit - (nu - nr);
        b = unit % batch;
        tile = unit / batch;
        span = 0;
        t_begin = part < 0 ? 0 : (int64_t)part * relay.len;
        t_end = part < 0 ? L : min(t_begin + (int64_t)relay.len, L);
    } else {
        int bid = blockIdx.x;
        b = bid % batch;
        bid /= batch;
        tile = bid % tiles;
        span = first_span + bid / tiles;
        t_begin = (int64_t)span * span_len;
        t_end = min(t_begin + span_len, L);
    }
    const int d = tile * 64 + lane;
    const bool dvalid = d < Dn;
    const int dc = dvalid ? d : Dn - 1; // tail lanes compute on a valid channel, store nothing
    const int n0 = g * NQ;

    const int64_t col0 = ((int64_t)b * Dn + dc) * N + n0;
    float a2[NQ], h[NQ], ia[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const float av = A[(int64_t)dc * N + n0 + q];
        a2[q] = av * kLog2e; // exp(Delta*A) = exp2(Delta*A*log2 e)
        ia[q] = ZOH ? 1.0f / av : 0.0f;
        h[q] = h_init ? h_init[span * h_init_stride + col0 + q] : 0.0f;
    }
    if (relayed && part > 0) {
        // the previous part's final state: wait for its flag, then read it
        const int slot = r_unit * (relay.parts - 1) + part - 1;
        if (relay_receive(relay.sync + slot, relay.fault, relay.max_polls)) {
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                h[q] = relay.state[((int64_t)slot * N + n0 + q) * 64 + lane];
        } else {
            // the hand-off never came (counted in relay.fault): a NaN state makes every
            // output of this part and of the unit's final state NaN instead of wrong
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                h[q] = __builtin_nanf("");
        }
    }
    const float bias_d = bias ? bias[dc] : 0.0f;
    const float D_d = Dv ? Dv[dc] : 0.0f;

    // trapezoid look-back: the input (u, B) of the step before this span's first step
    float u_lb = 0.0f, b_lb[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q)
        b_lb[q] = 0.0f;
    if constexpr (TRAP) {
        if (t_begin > 0) {
            u_lb = load_val(u, ((int64_t)b * L + t_begin - 1) * m3.su + dc);
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                b_lb[q] = load_val((const T *)m3.Bm,
                                   ((int64_t)b * L + t_begin - 1) * m3.sB + n0 + q);
        } else {
            if (m3.u_prev)
                u_lb = load_val((const T *)m3.u_prev, (int64_t)b * Dn + dc);
            if (m3.B_prev) {
#pragma unroll
                for (int q = 0; q < NQ; ++q)
                    b_lb[q] = load_val((const T *)m3.B_prev, (int64_t)b * N + n0 + q);
            }
        }
    }

    // bytes per time step of one batch row (y, lam: d_inner elements; u, delta, z: their row
    // strides); span bytes stay below 2^31 (planner)
    const uint32_t step_bytes = (uint32_t)Dn * (uint32_t)sizeof(T);
    const uint32_t step_u = (uint32_t)m3.su * (uint32_t)sizeof(T);
    const uint32_t step_d = (uint32_t)m3.sd * (uint32_t)sizeof(T);
    const uint32_t step_z = (uint32_t)m3.sz * (uint32_t)sizeof(T);
    const uint32_t vo_in = (uint32_t)dc * (uint32_t)sizeof(T);
    const uint32_t vo_out = (uint32_t)d * (uint32_t)sizeof(T);
    const int64_t row0 = (int64_t)b * L + t_begin; // row (b, t_begin)
    const int64_t span0 = row0 * step_bytes;       // its byte offset in y (and lam)
    // local time: 0 .. n_loc - 1 within this span (32-bit, as are all loop quantities)
    const int n_loc = (int)(t_end - t_begin);
    const uint32_t span_bytes = (uint32_t)n_loc * step_bytes;
    const rsrc_t r_u = make_rsrc(reinterpret_cast<const char *>(u) + row0 * step_u,
                                 (uint32_t)n_loc * step_u);
    const rsrc_t r_d = make_rsrc(reinterpret_cast<const char *>(delta) + row0 * step_d,
                                 (uint32_t)n_loc * step_d);
    const rsrc_t r_z = gated ? make_rsrc(reinterpret_cast<const char *>(z) + row0 * step_z,
                                         (uint32_t)n_loc * step_z)
                             : r_u;
    const rsrc_t r_l = TRAP ? make_rsrc(reinterpret_cast<const char *>(m3.lam) + span0,
                                        span_bytes)
                            : r_u;
    const rsrc_t r_y = FULL ? make_rsrc(reinterpret_cast<const char *>(y) + span0, span_bytes)
                            : r_u;
    // this wave's (t, B/C) rows from the span's first step
    const float *bc_span = bcp + (((int64_t)b * NW + g) * Lp + t_begin) * BCW;

    // raw inputs of PD chunks in flight: u, delta, z for this lane's KPL channel-steps
    // (zeroed so that the prologue may process the unloaded steps of a last, partial chunk:
    // their values are computed and never used)
    T ru[PD][KPL] = {}, rd[PD][KPL] = {}, rz[PD][KPL] = {}, rl[PD][KPL] = {};
    auto fetch = [&](auto BUF, int t0) {
        constexpr int j = decltype(BUF)::value;
#pragma unroll
        for (int k = 0; k < KPL; ++k) {
            const int tl = g + k * NW;
            const int t = t0 + tl;
            if (tl < TC && t < n_loc) { // wave-uniform
                ru[j][k] = buf_load(r_u, vo_in, (uint32_t)t * step_u, (T *)nullptr);
                rd[j][k] = buf_load(r_d, vo_in, (uint32_t)t * step_d, (T *)nullptr);
                if (gated)
                    rz[j][k] = buf_load(r_z, vo_in, (uint32_t)t * step_z, (T *)nullptr);
                if (TRAP)
                    rl[j][k] = buf_load(r_l, vo_in, (uint32_t)t * step_bytes, (T *)nullptr);
            }
        }
    };

    // B/C of one chunk in scalar registers.  Chunk c + 1's values are requested as soon
    // as chunk c's recurrence has consumed chunk c's, so their latency overlaps the next
    // prologue and the barrier (whose LDS wait drains them anyway).
    float bcs[TC][BCW];
    auto load_bc = [&](int t0) {
        const cfloat_ptr q = (cfloat_ptr)(bc_span + (int64_t)t0 * BCW);
#pragma unroll
        for (int tl = 0; tl < TC; ++tl)
#pragma unroll
            for (int i = 0; i < BCW; ++i)
                bcs[tl][i] = (FULL || i < NQ || (ROT && i >= 2 * NQ)) ? q[tl * BCW + i] : 0.0f;
    };

    // span pass: sum of Delta over the span, the waves' shares of the steps (each step is
    // added once, by the lane that computes its Delta; joined over the waves at the end)
    float sum_dt = 0.0f;
    // span pass with the rotation: the transition of each state pair over the span, a 2x2
    // matrix (rotations and unequal decays within a pair do not commute), columns
    // (m00, m10) and (m01, m11) of pair k at rm[4k ..]
    constexpr bool RM = ROT && !FULL;
    float rm[RM ? 2 * NQ : 1];
    if constexpr (RM) {
#pragma unroll
        for (int k = 0; k < NQ / 2; ++k) {
            rm[4 * k] = 1.0f;
            rm[4 * k + 1] = 0.0f;
            rm[4 * k + 2] = 0.0f;
            rm[4 * k + 3] = 1.0f;
        }
    }
    // pending epilogue (the previous chunk): this lane's D*u, gate, first step, valid steps
    float e_du[KPL], e_gz[KPL];
    int e_t0 = -1;
    int e_nt = 0;
#pragma unroll
    for (int k = 0; k < KPL; ++k) {
        e_du[k] = 0.0f;
        e_gz[k] = 1.0f;
    }

    // fixed-order sum of the pending chunk's partial readouts (LDS reads only)
    auto epilogue_sum = [&](auto PAR, float (&s)[KPL]) {
        constexpr int pp = FULL ? decltype(PAR)::value : 0; // s_yp has one slot when !FULL
#pragma unroll
        for (int k = 0; k < KPL; ++k) {
            const int tl = g + k * NW;
            s[k] = 0.0f;
            if (FULL && tl < TC) {
                s[k] = s_yp[pp][tl][0][lane];
#pragma unroll
                for (int w = 1; w < NW; ++w)
                    s[k] += s_yp[pp][tl][w][lane];
            }
        }
    };
    // D*u, gate and store of the pending chunk
    auto epilogue_store = [&](const float (&s)[KPL]) {
        if (FULL && e_t0 >= 0 && dvalid) {
#pragma unroll
            for (int k = 0; k < KPL; ++k) {
                const int tl = g + k * NW;
                if (tl < e_nt)
                    buf_store((s[k] + e_du[k]) * e_gz[k], r_y, vo_out,
                              (uint32_t)(e_t0 + tl) * step_bytes, (T *)nullptr);
            }
        }
    };

    auto chunk = [&](auto BUF, int t0) {
        constexpr int j = decltype(BUF)::value; // ring slot; its low bit is the chunk parity
        constexpr int pp = j & 1;
        const int nt = min(TC, n_loc - t0);

        // ---- prologue: Delta and Delta*u once per (t, d) ----
        // Wave priorities per phase (the SIMD issues the ready wave of highest priority):
        // the chunk's decay exps 3, its recurrence 1, the prologue up to the barrier 0.
        // Measured at the large prefill, six waves of three blocks per SIMD: 650 us against
        // 705 us with equal priorities (705 with the exps alone not raised, 675 with the
        // prologue alone lowered); results unchanged.
        __builtin_amdgcn_s_setprio(0);
        // (steps tl >= nt of a partial chunk are computed from stale registers and ignored)
        float du[KPL], gz[KPL];
#pragma unroll
        for (int k = 0; k < KPL; ++k) {
            const int tl = g + k * NW;
            const float uu = widen(ru[j][k]);
            const float dl = softplus_act<T>(widen(rd[j][k]) + bias_d);
            du[k] = FULL ? D_d * uu : 0.0f;
            gz[k] = gated ? silu_f(widen(rz[j][k])) : 1.0f;
            if (!FULL && tl < nt)
                sum_dt += dl;
            if (tl < TC) {
                if constexpr (ZOH) {
                    s_dw[pp][tl][lane] = make_float4(dl, dl * uu, uu, 0.0f);
                } else if constexpr (TRAP) {
                    const float lm = widen(rl[j][k]);
                    s_dw[pp][tl][lane] = make_float4(dl, lm * dl * uu, (1.0f - lm) * dl, uu);
                } else {
                    s_dw[pp][tl][lane] = make_float2(dl, dl * uu);
                }
            }
        }
        if (t0 + PD * TC < n_loc)
            fetch(BUF, t0 + PD * TC);
        __syncthreads();

        // LDS reads: the previous chunk's partial readouts and this chunk's (Delta, Delta*u)
        float es[KPL];
        epilogue_sum(std::integral_constant<int, pp ^ 1>{}, es);
        DW dw[TC];
#pragma unroll
        for (int tl = 0; tl < TC; ++tl)
            dw[tl] = s_dw[pp][tl][lane];
        epilogue_store(es);
        __builtin_amdgcn_s_setprio(3);

        // ---- recurrence over the chunk ----
        // The chunk's decay factors first: issued back to back, the exps leave the VALU
        // free of the switches between exp and FMA forms inside each step (measured 5 %
        // faster at the large prefill; the values are the same).
        // (the zero-order hold keeps the exp2 arguments for its input term)
        float ag[TC][NQ], xg[ZOH ? TC : 1][ZOH ? NQ : 1];
#pragma unroll
        for (int tl = 0; tl < TC; ++tl)
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const float xa = __builtin_fmaf(dw[tl].x, a2[q], kExp2Shift);
                if constexpr (ZOH)
                    xg[ZOH ? tl : 0][ZOH ? q : 0] = xa;
                ag[tl][q] = hw_exp2(xa); // decay_exp2(dw[tl].x, a2[q])
            }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
        auto step = [&](int tl) {
            float yp = 0.0f;
            if constexpr (ROT) {
                // rotate each state pair by Delta * theta before the decay
#pragma unroll
                for (int k = 0; k < NQ / 2; ++k) {
                    if constexpr (RM) { // the same turn of the pair's transition columns
                        float sn, cs;
                        sincos_staged<T>(dw[tl].x * bcs[tl][2 * NQ + k], sn, cs);
                        turn_pair(sn, cs, h[2 * k], h[2 * k + 1]);
                        turn_pair(sn, cs, rm[4 * k], rm[4 * k + 1]);
                        turn_pair(sn, cs, rm[4 * k + 2], rm[4 * k + 3]);
                    } else {
                        float sn, cs;
                        sincos_staged<T>(dw[tl].x * bcs[tl][2 * NQ + k], sn, cs);
                        turn_pair(sn, cs, h[2 * k], h[2 * k + 1]);
                    }
                }
            }
            // trapezoid: (1 - lam) Delta u_{t-1}, from the previous step (or the carry)
            float p_lb = 0.0f;
            if constexpr (TRAP)
                p_lb = dw[tl].z * (tl == 0 ? u_lb : dw[tl > 0 ? tl - 1 : 0].w);
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const float a = ag[tl][q];
                if constexpr (RM) { // row q % 2 of pair q / 2 decays with state q
                    rm[4 * (q / 2) + (q & 1)] *= a;
                    rm[4 * (q / 2) + 2 + (q & 1)] *= a;
                }
                float bu = dw[tl].y; // Bbar u / B: Euler Delta u (trapezoid: lam Delta u)
                if constexpr (ZOH)
                    bu = zoh_input_b2(xg[ZOH ? tl : 0][ZOH ? q : 0], a, dw[tl].y, dw[tl].z * ia[q]);
                if constexpr (TRAP) {
                    const float bp = tl == 0 ? b_lb[q] : bcs[tl > 0 ? tl - 1 : 0][q];
                    h[q] = __builtin_fmaf(a, h[q], __builtin_fmaf(p_lb, bp, bu * bcs[tl][q]));
                } else {
                    h[q] = __builtin_fmaf(a, h[q], bu * bcs[tl][q]);
                }
                if (FULL)
                    yp = __builtin_fmaf(bcs[tl][NQ + q], h[q], yp);
            }
            if (FULL)
                s_yp[FULL ? pp : 0][tl][g][lane] = yp;
            if constexpr (CK) {
                // the state after absolute step tn - 1 enters segment tn / 8 (every lane,
                // tail lanes included: they hold a valid channel's finite state).  Spans and
                // relay parts start at multiples of the chunk, so with chunks of a multiple
                // of 8 steps the boundaries are known steps of the chunk.
                const int64_t tn = t_begin + t0 + tl + 1;
                if ((TC % 8 == 0 ? (tl & 7) == 7 : (tn & 7) == 0) && tn < L) {
                    float *ckp = m3.ck + ((((int64_t)tile * batch + b) * m3.ck_nseg + (tn >> 3)) * N +
                                          n0) * 64 + lane;
#pragma unroll
                    for (int q = 0; q < NQ; ++q)
                        ckp[q * 64] = h[q];
                }
            }
        };
        if (nt == TC) {
#pragma unroll
            for (int tl = 0; tl < TC; ++tl)
                step(tl);
        } else {
#pragma unroll
            for (int tl = 0; tl < TC; ++tl)
                if (tl < nt)
                    step(tl);
        }
        if constexpr (TRAP) {
            // look-back of the next chunk's first step (only a full chunk has a next one)
            u_lb = dw[TC - 1].w;
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                b_lb[q] = bcs[TC - 1][q];
        }
        __builtin_amdgcn_sched_barrier(0);
        if (t0 + TC < n_loc)
            load_bc(t0 + TC);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < KPL; ++k) {
            e_du[k] = du[k];
            e_gz[k] = gz[k];
        }
        e_t0 = t0;
        e_nt = nt;
    };

    for_c<0, PD>([&](auto BUF) {
        const int t0 = decltype(BUF)::value * TC;
        if (t0 < n_loc)
            fetch(BUF, t0);
    });
    if (n_loc > 0)
        load_bc(0);
    int last_parity = 0;
    for (int t0 = 0; t0 < n_loc; t0 += PD * TC) {
        for_c<0, PD>([&](auto BUF) {
            const int tc = t0 + decltype(BUF)::value * TC; // block-uniform
            if (tc < n_loc) {
                chunk(BUF, tc);
                last_parity = decltype(BUF)::value & 1;
            }
        });
    }
    if (FULL) {
        __syncthreads();
        float es[KPL];
        if (last_parity == 0)
            epilogue_sum(std::integral_constant<int, 0>{}, es);
        else
            epilogue_sum(std::integral_constant<int, 1>{}, es);
        epilogue_store(es);
    }

    if (relayed && part >= 0 && part < relay.parts - 1) {
        // hand the final state to the next part (every lane: the slot is dense)
        const int slot = r_unit * (relay.parts - 1) + part;
        if (relay.withhold && part == 0)
            return; // failure test: the next part's wait gives up
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            relay.state[((int64_t)slot * N + n0 + q) * 64 + lane] = h[q];
        relay_signal(relay.sync + slot);
        return;
    }
    if constexpr (!FULL) {
        // the span's sum of Delta: the waves' shares in wave order
        s_sdt[g][lane] = sum_dt;
        __syncthreads();
        sum_dt = s_sdt[0][lane];
#pragma unroll
        for (int w = 1; w < NW; ++w)
            sum_dt += s_sdt[w][lane];
    }
    if (!dvalid)
        return;
    const int64_t col = ((int64_t)b * Dn + d) * N + n0;
    if (FULL) {
        if (h_last && span == n_spans - 1) {
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                h_last[col + q] = h[q];
        }
    } else {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            ws_decay[(col + q) * n_spans + span] = hw_exp2(a2[q] * sum_dt);
            ws_hloc[(col + q) * n_spans + span] = h[q];
        }
        if constexpr (RM) {
#pragma unroll
            for (int k = 0; k < NQ / 2; ++k)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    m3.rot_m[((col / 2 + k) * n_spans + span) * 4 + j] = rm[4 * k + j];
        }
    }
}

// (d_state, waves, chunk, prefetch depth): variants whose chunk of B/C (chunk * 2 *
// d_state / waves floats) fits the scalar register file without spilling.
#define MAMBA_SCALAR_VARIANTS(X) \
    X(4, 4, 8, 2)                \
    X(8, 8, 8, 2)                \
    X(16, 8, 4, 2)               \
    X(16, 8, 8, 2)               \
    X(32, 8, 4, 2)

template <typename T, int N, int NW, int TC, int PD, bool FULL, bool GATED, int DISC, bool ROT,
          bool CK = false>
hipError_t launch_scalar_variant(const ScanLaunch &p, hipStream_t stream)
{
    const int32_t tiles = (int32_t)((p.d_inner + 63) / 64);
    int64_t blocks = (int64_t)tiles * p.batch * p.launch_spans;
    RelayArgs relay{};
    relay.parts = 1;
    if (FULL && p.relay_parts > 1) {
        relay.sync = p.relay_sync;
        relay.fault = p.relay_sync + (int64_t)p.relay_tiles * (p.relay_parts - 1);
        relay.max_polls = p.relay_max_polls;
        relay.withhold = p.relay_withhold ? 1 : 0;
        relay.state = p.relay_state;
        relay.tiles = p.relay_tiles;
        relay.parts = p.relay_parts;
        relay.units = (int32_t)(tiles * p.batch);
        relay.len = (int32_t)p.relay_len;
        blocks = (int64_t)relay.units + (int64_t)relay.tiles * (relay.parts - 1);
    }
    if (blocks <= 0)
        return hipSuccess;
    Mamba3Args m3{p.lam,    p.u_prev,  p.B_prev,  p.B,       p.ckpt, (int32_t)((p.L + 7) / 8),
                  p.ws_rot, (int32_t)p.su, (int32_t)p.sd, (int32_t)p.sz, (int32_t)p.sB};
    hipLaunchKernelGGL((scan_scalar_kernel<T, N, NW, TC, PD, FULL, GATED, DISC, ROT, CK>),
                       dim3((uint32_t)blocks), dim3(64 * NW), 0, stream, (const T *)p.u,
                       (const T *)p.delta, (const T *)p.z, p.bc_staged, p.A, p.D, p.bias,
                       p.h_init, p.h_init_span_stride, (T *)p.y, p.h_last, p.ws_decay,
                       p.ws_hloc, p.L, p.staged_rows, (int32_t)p.d_inner, p.span_len,
                       p.n_spans, p.first_span, tiles, (int32_t)p.batch, relay, m3);
    return hipGetLastError();
}

template <typename T, int N, int NW>
hipError_t launch_stage(const ScanLaunch &p, hipStream_t stream)
{
    const int64_t total = p.batch * NW * p.staged_rows; // one thread per (b, wave, t)
    // hand-off flags and the fault word after them
    const int32_t n_sync = p.relay_parts > 1 ? p.relay_tiles * (p.relay_parts - 1) + 1 : 0;
    const int64_t blocks = (max(total, (int64_t)n_sync) + 255) / 256;
    if (blocks <= 0)
        return hipSuccess;
    if (p.rot) {
        if constexpr ((N / NW) % 2 == 0)
            hipLaunchKernelGGL((stage_bc_kernel<T, N, NW, true>), dim3((uint32_t)blocks),
                               dim3(256), 0, stream, (const T *)p.B, (const T *)p.C,
                               (const T *)p.theta, p.bc_staged, p.L, p.staged_rows, total,
                               p.relay_sync, n_sync, p.sB, p.sC);
        else
            return hipErrorInvalidValue;
    } else {
        hipLaunchKernelGGL((stage_bc_kernel<T, N, NW, false>), dim3((uint32_t)blocks), dim3(256),
                           0, stream, (const T *)p.B, (const T *)p.C, (const T *)nullptr,
                           p.bc_staged, p.L, p.staged_rows, total, p.relay_sync, n_sync, p.sB,
                           p.sC);
    }
    return hipGetLastError();
}

// Rotation is compiled for variants whose waves hold whole state pairs; its span pass also
// gives each pair's 2x2 transition over the span (ws_rot) for the carry.
template <typename T, int N, int NW, int TC, int PD, bool FULL, int DISC>
hipError_t launch_scalar_disc(const ScanLaunch &p, hipStream_t stream)
{
    const bool g = FULL && p.z != nullptr;
    if (p.ckpt) {
        // checkpoints: Euler without rotation, written by the full-output pass
        if constexpr (FULL && DISC == 0)
            return g ? launch_scalar_variant<T, N, NW, TC, PD, FULL, true, 0, false, true>(p, stream)
                     : launch_scalar_variant<T, N, NW, TC, PD, FULL, false, 0, false, true>(p, stream);
        else
            return hipErrorInvalidValue;
    }
    if (p.rot) {
        // the span pass needs the pairs' transitions (ws_rot) for the carry
        if constexpr ((N / NW) % 2 == 0) {
            if (!FULL && !p.ws_rot)
                return hipErrorInvalidValue;
            return g ? launch_scalar_variant<T, N, NW, TC, PD, FULL, true, DISC, true>(p, stream)
                     : launch_scalar_variant<T, N, NW, TC, PD, FULL, false, DISC, true>(p, stream);
        } else {
            return hipErrorInvalidValue;
        }
    }
    return g ? launch_scalar_variant<T, N, NW, TC, PD, FULL, true, DISC, false>(p, stream)
             : launch_scalar_variant<T, N, NW, TC, PD, FULL, false, DISC, false>(p, stream);
}

template <typename T, int N, int NW, int TC, int PD, bool FULL>
hipError_t launch_scalar_opts(const ScanLaunch &p, hipStream_t stream)
{
    if (p.trap)
        return launch_scalar_disc<T, N, NW, TC, PD, FULL, 2>(p, stream);
    if (p.zoh)
        return launch_scalar_disc<T, N, NW, TC, PD, FULL, 1>(p, stream);
    return launch_scalar_disc<T, N, NW, TC, PD, FULL, 0>(p, stream);
}

template <bool FULL>
hipError_t launch_scalar_any(const ScanLaunch &p, hipStream_t stream)
{
#define X(N_, W_, C_, P_)                                                   \
    if (p.d_state == N_ && p.waves == W_ && p.chunk == C_) {                \
        if (p.dtype == DType::BF16)                                         \
            return launch_scalar_opts<uint16_t, N_, W_, C_, P_, FULL>(p, stream); \
        return launch_scalar_opts<float, N_, W_, C_, P_, FULL>(p, stream);  \
    }
    MAMBA_SCALAR_VARIANTS(X)
#undef X
    return hipErrorInvalidValue;
}

} // namespace

bool scalar_variant_supported(int64_t d_state, int waves, int chunk)
{
#define X(N_, W_, C_, P_)                                        \
    if (d_state == N_ && waves == W_ && chunk == C_) return true;
    MAMBA_SCALAR_VARIANTS(X)
#undef X
    return false;
}

hipError_t launch_stage_bc(const ScanLaunch &p, hipStream_t stream)
{
#define X(N_, W_, C_, P_)                                               \
    if (p.d_state == N_ && p.waves == W_) {                             \
        if (p.dtype == DType::BF16)                                     \
            return launch_stage<uint16_t, N_, W_>(p, stream);           \
        return launch_stage<float, N_, W_>(p, stream);                  \
    }
    MAMBA_SCALAR_VARIANTS(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_scalar_full(const ScanLaunch &p, hipStream_t stream)
{
    return launch_scalar_any<true>(p, stream);
}

hipError_t launch_scalar_end(const ScanLaunch &p, hipStream_t stream)
{
    return launch_scalar_any<false>(p, stream);
}

} // namespace mambascan
