// Barrier-free selective-scan kernel for gfx950: every wavefront scans 16 channels on its
// own, with no s_barrier anywhere.
//
// Same operation as scan_kernels.hip (the selective scan of "Understanding Mamba",
// aiattnstudio.link, sections 4.4 and 5.2), laid out on the four 16-lane DPP rows of a
// wave64:
//   * lane (row r, column c) owns channel d = 16 * group + c and the state indices
//     n in [r * NQ, (r + 1) * NQ), NQ = N / 4.  The 16 channels of a wave are therefore
//     present in every row, each row holding a different quarter of their states.
//   * B_t[n] and C_t[n] depend on the row only.  Each lane loads one value of a 4-step
//     block of B (and of C) -- row r's 16 lanes hold B[t0..t0+3][r*NQ .. r*NQ+NQ) -- and
//     the update takes the value it needs with a DPP row_newbcast broadcast folded into
//     the multiply (v_mul_f32_dpp): B and C cost no extra instructions and no LDS.
//   * time advances in blocks of 4 steps.  Lane (r, c) computes Delta = softplus(delta +
//     bias) and Delta * u for step t0 + r of channel c (once per channel-step), and the
//     four rows exchange them through a 512-byte wave-private LDS area (one 8-byte write,
//     two 16-byte reads).  The partial readouts of the four rows are exchanged the same
//     way so that lane (r, c) ends up with the complete y of step t0 + r, adds D u,
//     applies the gate and stores it.
//   * with no barriers, waves never wait for each other; the inputs of a block are
//     requested PF blocks ahead into a ring of registers.
// Spans for long sequences (END / FULL modes) work as in scan_kernels.hip.
#include <type_traits>

#include "device_math.h"
#include "scan_common.h"

namespace mambascan {
namespace {

template <int I0, int I1, typename F>
__device__ __forceinline__ void unroll_for(F &&f)
{
    if constexpr (I0 < I1) {
        f(std::integral_constant<int, I0>{});
        unroll_for<I0 + 1, I1>(f);
    }
}

// Value of `v` in lane K of the caller's 16-lane row (DPP row_newbcast).  Used as the
// first operand of a multiply, the broadcast is folded into v_mul_f32_dpp.
template <int K>
__device__ __forceinline__ float row_bcast(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + K, 0xF, 0xF, true));
}

// Orders this wave's LDS accesses around a cross-lane exchange (no other wave takes part).
__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T, int N, int PF, bool FULL>
__global__ void __launch_bounds__(256)
scan_rows_kernel(const T *__restrict__ u, const T *__restrict__ delta, const T *__restrict__ z,
                 const T *__restrict__ Bm, const T *__restrict__ Cm,
                 const float *__restrict__ A, const float *__restrict__ Dv,
                 const float *__restrict__ bias, const float *h_init, int64_t h_init_stride,
                 T *__restrict__ y, float *h_last, float *__restrict__ ws_decay,
                 float *__restrict__ ws_hloc, int64_t L, int32_t Dn, int64_t span_len,
                 int32_t n_spans, int32_t first_span, int32_t tiles, int32_t batch)
{
    constexpr int NQ = N / 4;                  // state indices per lane
    constexpr int BCV = (4 * NQ + 15) / 16;    // B (and C) registers per 4-step block
    static_assert(N % 4 == 0 && NQ >= 1, "d_state must be a multiple of 4");

    __shared__ float2 s_dw[4][16][4];                   // [wave][channel][step]
    __shared__ float s_y[FULL ? 4 : 1][16][4][5];       // [wave][channel][step][row] (+pad)

    const int lane = threadIdx.x & 63;
    const int r = lane >> 4;  // row: state group, and the step of the block this lane stages
    const int c = lane & 15;  // channel within the wave
    const int wv = threadIdx.x >> 6;

    int bid = blockIdx.x;
    const int tile = bid % tiles; // 64 channels per block, 16 per wave
    bid /= tiles;
    const int b = bid % batch;
    const int span = first_span + bid / batch;

    const int64_t t_begin = (int64_t)span * span_len;
    const int64_t t_end = min(t_begin + span_len, L);
    const int d = tile * 64 + wv * 16 + c;
    const bool dvalid = d < Dn;
    const int dc = dvalid ? d : Dn - 1;
    const int n0 = r * NQ;

    const int64_t col0 = ((int64_t)b * Dn + dc) * N + n0;
    float a2[NQ], h[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        a2[q] = A[(int64_t)dc * N + n0 + q] * kLog2e;
        h[q] = h_init ? h_init[span * h_init_stride + col0 + q] : 0.0f;
    }
    const float bias_d = bias ? bias[dc] : 0.0f;
    const float D_d = Dv ? Dv[dc] : 0.0f;
    const bool gated = FULL && z != nullptr;
    const int64_t row_b = (int64_t)b * L;

    // Addresses: a wave-uniform base pointer per 4-step block (scalar arithmetic) plus a
    // fixed 32-bit offset per lane.  Lane (r, c) reads u/delta/z at step t0 + r of its
    // channel; B/C register v holds element e = 16 v + c of this row's (4 steps x NQ
    // states) block: step e / NQ, state r * NQ + e % NQ.
    const int off_x = r * Dn + dc;
    int off_bc[BCV];
#pragma unroll
    for (int v = 0; v < BCV; ++v) {
        const int e = 16 * v + c;
        off_bc[v] = (e / NQ) * N + n0 + e % NQ;
    }
    const T *u_b = u + row_b * Dn, *delta_b = delta + row_b * Dn;
    const T *z_b = z ? z + row_b * Dn : nullptr;
    const T *B_b = Bm + row_b * N, *C_b = Cm + row_b * N;

    T ru[PF], rd[PF], rz[PF], rb[PF][BCV], rc[PF][BCV];
    // GUARD: the block may cross the span end (per-lane guards); otherwise it is whole.
    auto fetch = [&](auto BUF, auto GUARD, int64_t t0) {
        constexpr int j = decltype(BUF)::value;
        constexpr bool guarded = decltype(GUARD)::value;
        const int64_t ox = t0 * Dn, obc = t0 * N; // uniform
        if (!guarded || t0 + r < t_end) {
            ru[j] = u_b[ox + off_x];
            rd[j] = delta_b[ox + off_x];
            if (gated)
                rz[j] = z_b[ox + off_x];
        }
#pragma unroll
        for (int v = 0; v < BCV; ++v) {
            const int e = 16 * v + c;
            if (e < 4 * NQ && (!guarded || t0 + e / NQ < t_end)) {
                rb[j][v] = B_b[obc + off_bc[v]];
                if (FULL)
                    rc[j][v] = C_b[obc + off_bc[v]];
            }
        }
    };

    float sum_dt = 0.0f;
    auto block = [&](auto BUF, auto GUARD, int64_t t0) {
        constexpr int j = decltype(BUF)::value;
        constexpr bool guarded = decltype(GUARD)::value;
        const int nt = guarded ? (int)min((int64_t)4, t_end - t0) : 4; // valid steps

        // ---- this lane's channel-step: Delta, Delta*u, D*u, gate ----
        float dl = 0.0f, w = 0.0f, du = 0.0f, gz = 1.0f;
        if (!guarded || r < nt) {
            const float uu = widen(ru[j]);
            dl = softplus_act<T>(widen(rd[j]) + bias_d);
            w = dl * uu;
            if (FULL) {
                du = D_d * uu;
                if (gated)
                    gz = silu_f(widen(rz[j]));
            }
        }
        float bv[BCV], cv[BCV];
#pragma unroll
        for (int v = 0; v < BCV; ++v) {
            bv[v] = widen(rb[j][v]);
            cv[v] = FULL ? widen(rc[j][v]) : 0.0f;
        }
        if (!guarded)
            fetch(BUF, std::false_type{}, t0 + 4 * PF);
        else if (t0 + 4 * PF < t_end)
            fetch(BUF, std::true_type{}, t0 + 4 * PF);

        // ---- all-gather (Delta, Delta*u) of the block's 4 steps within the wave ----
        s_dw[wv][c][r] = make_float2(dl, w);
        wave_sync();
        const float4 x01 = *reinterpret_cast<const float4 *>(&s_dw[wv][c][0]);
        const float4 x23 = *reinterpret_cast<const float4 *>(&s_dw[wv][c][2]);
        const float dls[4] = {x01.x, x01.z, x23.x, x23.z};
        const float ws[4] = {x01.y, x01.w, x23.y, x23.w};

        // ---- recurrence: 4 steps x NQ states; B and C via row broadcasts ----
        float yp[4];
        auto step = [&](auto S) {
            constexpr int s = decltype(S)::value;
            float acc = 0.0f;
            unroll_for<0, NQ>([&](auto Q) {
                constexpr int q = decltype(Q)::value;
                constexpr int e = s * NQ + q;
                const float a = decay_exp2(dls[s], a2[q]);
                h[q] = __builtin_fmaf(a, h[q], row_bcast<e % 16>(bv[e / 16]) * ws[s]);
                if (FULL) {
                    const float p = row_bcast<e % 16>(cv[e / 16]) * h[q];
                    acc = q == 0 ? p : acc + p;
                }
            });
            yp[s] = acc;
            if (!FULL)
                sum_dt += dls[s];
        };
        if (!guarded || nt == 4) { // straight-line code for whole blocks
            unroll_for<0, 4>(step);
        } else {
            unroll_for<0, 4>([&](auto S) {
                if (decltype(S)::value < nt)
                    step(S);
                else
                    yp[decltype(S)::value] = 0.0f;
            });
        }

        // ---- reduce-scatter of the readout: lane (r, c) collects step t0 + r ----
        if (FULL) {
            wave_sync(); // the previous block's reads of s_y are done
#pragma unroll
            for (int i = 0; i < 4; ++i)
                s_y[wv][c][i][r] = yp[i];
            wave_sync();
            if ((!guarded || r < nt) && dvalid) {
                const float *py = &s_y[wv][c][r][0];
                const float tot = ((py[0] + py[1]) + py[2]) + py[3];
                store_val(y + (row_b + t0) * Dn, off_x - dc + d, (tot + du) * gz);
            }
        }
        wave_sync(); // s_dw is rewritten by the next block
    };

    // prime the ring, then whole rounds of PF blocks whose refills are whole too, then
    // the guarded tail
    unroll_for<0, PF>([&](auto BUF) {
        const int64_t t0 = t_begin + 4 * decltype(BUF)::value;
        if (t0 < t_end)
            fetch(BUF, std::true_type{}, t0);
    });
    int64_t t0 = t_begin;
    for (; t0 + 8 * PF <= t_end; t0 += 4 * PF) {
        unroll_for<0, PF>([&](auto BUF) {
            block(BUF, std::false_type{}, t0 + 4 * decltype(BUF)::value);
        });
    }
    for (; t0 < t_end; t0 += 4 * PF) {
        unroll_for<0, PF>([&](auto BUF) {
            const int64_t tb = t0 + 4 * decltype(BUF)::value;
            if (tb < t_end)
                block(BUF, std::true_type{}, tb);
        });
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
    }
}

constexpr int kRowsPrefetch = 4; // blocks of 4 steps in flight

template <typename T, int N, bool FULL>
hipError_t launch_rows_variant(const ScanLaunch &p, hipStream_t stream)
{
    const int32_t tiles = (int32_t)((p.d_inner + 63) / 64);
    const int64_t blocks = (int64_t)tiles * p.batch * p.launch_spans;
    if (blocks <= 0)
        return hipSuccess;
    hipLaunchKernelGGL((scan_rows_kernel<T, N, kRowsPrefetch, FULL>), dim3((uint32_t)blocks),
                       dim3(256), 0, stream, (const T *)p.u, (const T *)p.delta,
                       (const T *)p.z, (const T *)p.B, (const T *)p.C, p.A, p.D, p.bias,
                       p.h_init, p.h_init_span_stride, (T *)p.y, p.h_last, p.ws_decay,
                       p.ws_hloc, p.L, (int32_t)p.d_inner, p.span_len, p.n_spans,
                       p.first_span, tiles, (int32_t)p.batch);
    return hipGetLastError();
}

template <bool FULL>
hipError_t launch_rows_any(const ScanLaunch &p, hipStream_t stream)
{
#define ROWS_CASE(N_)                                                      \
    if (p.d_state == N_) {                                                 \
        if (p.dtype == DType::BF16)                                        \
            return launch_rows_variant<uint16_t, N_, FULL>(p, stream);     \
        return launch_rows_variant<float, N_, FULL>(p, stream);            \
    }
    ROWS_CASE(4)
    ROWS_CASE(8)
    ROWS_CASE(16)
    ROWS_CASE(32)
    ROWS_CASE(64)
#undef ROWS_CASE
    return hipErrorInvalidValue;
}

} // namespace

hipError_t launch_rows_full(const ScanLaunch &p, hipStream_t stream)
{
    return launch_rows_any<true>(p, stream);
}

hipError_t launch_rows_end(const ScanLaunch &p, hipStream_t stream)
{
    return launch_rows_any<false>(p, stream);
}

} // namespace mambascan
