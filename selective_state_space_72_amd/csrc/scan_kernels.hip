// Chunked selective-scan kernels for gfx950 (MI355X).
//
// Operation: Delta_t = softplus(delta_t + bias_d), h_t[n] = exp(Delta_t A[d,n]) h_{t-1}[n]
// + Delta_t B_t[n] u_t, y_t = (sum_n C_t[n] h_t[n] + D_d u_t) * silu(z_t): the selective
// scan of "Understanding Mamba" (aiattnstudio.link) sections 4.4 and 5.2, fused into one
// pass so that nothing of shape (batch, L, d_inner, d_state) touches HBM -- the kernel
// fusion the hnwysp.cn Mamba slides describe in section 3.3, re-designed for CDNA4.
//
// Work decomposition (one block = 64 consecutive channels of one batch row):
//   * lane l of every wave owns channel d = 64*tile + l; wave g owns the state indices
//     n in [g*NQ, (g+1)*NQ), NQ = N / NW.  Because n is uniform across a wave, B_t[n] and
//     C_t[n] are the same for all its lanes: the inner update costs one multiply
//     (Delta*A), one v_exp_f32, one multiply (Delta*u*B), one FMA (recurrence) and one
//     FMA (readout) per (t, d, n), with h held in VGPRs.
//   * time advances in chunks of TC steps.  A chunk starts with a prologue in which the
//     block's lanes compute Delta and Delta*u once per (t, d) -- the expensive softplus is
//     never repeated per n -- and stage them in LDS together with the chunk's B and C
//     rows (widened to fp32 once, shared by all 64 channels of the block); the inputs of
//     the next chunk are requested right after, so their latency hides behind the
//     recurrence.
//   * every wave writes its partial readout sum_{n in its group} C h to LDS; the epilogue
//     adds the NW partials in a fixed order (bitwise deterministic), adds D*u, applies the
//     gate and stores y with coalesced 2-byte (bf16) or 4-byte stores.
//   * the state stays in registers across chunks (unbounded L).  For long sequences with
//     few channels the sequence is split into spans (the segment scan of the hnwysp.cn
//     slides, section 3.2): an END launch computes each span's zero-initial end state and
//     total decay exp(A * sum Delta); the carry kernel combines spans with the associative
//     map (a, b) o (a', b') = (a a', a' b + b'); a FULL launch rescans each span from its
//     true carry-in and emits y.
#include <type_traits>

#include "device_math.h"
#include "scan_common.h"

namespace mambascan {

// Compile-time loop: f(integral_constant<int, I>) for I in [I0, I1).
template <int I0, int I1, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I0 < I1) {
        f(std::integral_constant<int, I0>{});
        static_for<I0 + 1, I1>(f);
    }
}

template <typename T, int N, int NW, int TC, int PD, bool FULL>
__global__ void __launch_bounds__(64 * NW)
scan_chunk_kernel(const T *__restrict__ u, const T *__restrict__ delta, const T *__restrict__ z,
                  const T *__restrict__ Bm, const T *__restrict__ Cm,
                  const float *__restrict__ A, const float *__restrict__ Dv,
                  const float *__restrict__ bias, const float *h_init, int64_t h_init_stride,
                  T *__restrict__ y, float *h_last, float *__restrict__ ws_decay,
                  float *__restrict__ ws_hloc, int64_t L, int32_t Dn, int64_t span_len,
                  int32_t n_spans, int32_t first_span, int32_t tiles, int32_t batch)
{
    constexpr int NQ = N / NW;   // state indices per lane
    constexpr int KPL = TC / NW; // prologue/epilogue channel-steps per lane per chunk
    // PD: chunks of input in flight (prefetch depth)
    constexpr int NT = 64 * NW;  // threads per block
    constexpr int PBC = (TC * N + NT - 1) / NT; // B (and C) values staged per thread per chunk
    constexpr int BCW = FULL ? 2 * NQ : NQ;     // floats per (step, wave) in s_bc
    static_assert(NQ >= 1 && N % NW == 0 && TC % NW == 0, "bad variant");

    __shared__ float2 s_dw[TC][64];                          // (Delta, Delta*u)
    __shared__ float s_yp[FULL ? TC : 1][NW][64];            // partial readouts
    __shared__ __attribute__((aligned(16))) float s_bc[TC][NW][BCW]; // B (then C) per wave group

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int g = __builtin_amdgcn_readfirstlane(tid >> 6);

    int bid = blockIdx.x;
    const int tile = bid % tiles;
    bid /= tiles;
    const int b = bid % batch;
    const int span = first_span + bid / batch;

    const int64_t t_begin = (int64_t)span * span_len;
    const int64_t t_end = min(t_begin + span_len, L);
    const int d = tile * 64 + lane;
    const bool dvalid = d < Dn;
    const int dc = dvalid ? d : Dn - 1; // tail lanes compute on a valid channel, store nothing
    const int n0 = g * NQ;

    const int64_t col0 = ((int64_t)b * Dn + dc) * N + n0; // state column of (b, dc, n0)
    float a2[NQ], h[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        a2[q] = A[(int64_t)dc * N + n0 + q] * kLog2e; // exp(Delta*A) = exp2(Delta*A*log2 e)
        h[q] = h_init ? h_init[span * h_init_stride + col0 + q] : 0.0f;
    }
    const float bias_d = bias ? bias[dc] : 0.0f;
    const float D_d = Dv ? Dv[dc] : 0.0f;
    const bool gated = FULL && z != nullptr;

    const int64_t row_b = (int64_t)b * L; // row (b, t=0) of the (B, L, *) tensors

    // Inputs of a chunk, requested PD chunks ahead into a ring of register buffers: u,
    // delta, z for KPL (t, d) pairs per lane (coalesced rows of 64 channels) and PBC
    // entries of the chunk's B and C rows, which are contiguous (TC * N values each).
    T ru[PD][KPL], rd[PD][KPL], rz[PD][KPL], rb[PD][PBC], rc[PD][PBC];
    auto fetch = [&](auto BUF, int64_t t0) {
        constexpr int j = decltype(BUF)::value;
#pragma unroll
        for (int k = 0; k < KPL; ++k) {
            const int64_t t = t0 + g + k * NW; // wave-uniform
            if (t < t_end) {
                const int64_t i = (row_b + t) * Dn + dc;
                ru[j][k] = u[i];
                rd[j][k] = delta[i];
                if (gated)
                    rz[j][k] = z[i];
            }
        }
#pragma unroll
        for (int k = 0; k < PBC; ++k) {
            const int e = tid + k * NT; // element of the chunk's (TC, N) block
            if (e < TC * N && t0 + e / N < t_end) {
                const int64_t i = (row_b + t0) * N + e;
                rb[j][k] = Bm[i];
                if (FULL)
                    rc[j][k] = Cm[i];
            }
        }
    };

    float sum_dt = 0.0f;
    auto chunk = [&](auto BUF, int64_t t0) {
        constexpr int j = decltype(BUF)::value;
        const int nt = (int)min((int64_t)TC, t_end - t0);

        // ---- prologue: Delta and Delta*u once per (t, d); B and C widened to fp32 ----
        float du[KPL], gz[KPL];
#pragma unroll
        for (int k = 0; k < KPL; ++k) {
            const int tl = g + k * NW;
            float dl = 0.0f, w = 0.0f;
            du[k] = 0.0f;
            gz[k] = 1.0f;
            if (tl < nt) {
                const float uu = widen(ru[j][k]);
                dl = softplus_act<T>(widen(rd[j][k]) + bias_d);
                w = dl * uu;
                if (FULL) {
                    du[k] = D_d * uu;
                    if (gated)
                        gz[k] = silu_f(widen(rz[j][k]));
                }
            }
            s_dw[tl][lane] = make_float2(dl, w);
        }
#pragma unroll
        for (int k = 0; k < PBC; ++k) {
            const int e = tid + k * NT;
            if (e < TC * N) {
                const int tl = e / N, n = e % N;
                const bool ok = tl < nt;
                s_bc[tl][n / NQ][n % NQ] = ok ? widen(rb[j][k]) : 0.0f;
                if (FULL)
                    s_bc[tl][n / NQ][NQ + n % NQ] = ok ? widen(rc[j][k]) : 0.0f;
            }
        }
        if (t0 + PD * TC < t_end)
            fetch(BUF, t0 + PD * TC); // this buffer is free again: refill it PD chunks ahead
        __syncthreads();

        // ---- recurrence over the chunk ----
        // B_t and C_t of this wave's state indices come from one wave-uniform (broadcast)
        // LDS read per step; Delta and Delta*u from one per-lane read.
        auto step = [&](int tl) {
            const float2 dw = s_dw[tl][lane];
            float bc[BCW];
#pragma unroll
            for (int i = 0; i < BCW; ++i)
                bc[i] = s_bc[tl][g][i];
            float yp = 0.0f;
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const float a = decay_exp2(dw.x, a2[q]);
                h[q] = __builtin_fmaf(a, h[q], dw.y * bc[q]);
                if (FULL)
                    yp = __builtin_fmaf(bc[NQ + q], h[q], yp);
            }
            if (FULL)
                s_yp[tl][g][lane] = yp;
            else
                sum_dt += dw.x;
        };
        if (nt == TC) {
#pragma unroll
            for (int tl = 0; tl < TC; ++tl)
                step(tl);
        } else {
            for (int tl = 0; tl < nt; ++tl)
                step(tl);
        }
        __syncthreads();

        // ---- epilogue: fixed-order sum of the partial readouts, D*u, gate, store ----
        if (FULL) {
#pragma unroll
            for (int k = 0; k < KPL; ++k) {
                const int tl = g + k * NW;
                if (tl < nt && dvalid) {
                    float s = s_yp[tl][0][lane];
#pragma unroll
                    for (int w = 1; w < NW; ++w)
                        s += s_yp[tl][w][lane];
                    store_val(y, (row_b + t0 + tl) * Dn + d, (s + du[k]) * gz[k]);
                }
            }
        }
    };

    static_for<0, PD>([&](auto BUF) {
        const int64_t t0 = t_begin + decltype(BUF)::value * TC;
        if (t0 < t_end)
            fetch(BUF, t0);
    });
    for (int64_t t0 = t_begin; t0 < t_end; t0 += PD * TC) {
        static_for<0, PD>([&](auto BUF) {
            const int64_t tc = t0 + decltype(BUF)::value * TC; // block-uniform
            if (tc < t_end)
                chunk(BUF, tc);
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
        // span summary: total decay exp(A * sum_t Delta_t) and the end state from zero
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            ws_decay[(col + q) * n_spans + span] = hw_exp2(a2[q] * sum_dt);
            ws_hloc[(col + q) * n_spans + span] = h[q];
        }
    }
}

// ---------------------------------------------------------------------------
// variant table
// ---------------------------------------------------------------------------

// (d_state, waves, chunk, prefetch depth)
#define MAMBA_SCAN_VARIANTS(X) \
    X(4, 4, 16, 2)             \
    X(8, 4, 16, 2)             \
    X(8, 8, 8, 3)              \
    X(16, 4, 16, 2)            \
    X(16, 4, 32, 2)            \
    X(16, 8, 8, 3)             \
    X(16, 8, 16, 2)            \
    X(32, 4, 16, 2)            \
    X(32, 8, 8, 3)             \
    X(32, 8, 16, 2)            \
    X(64, 8, 8, 3)             \
    X(64, 8, 16, 2)

bool scan_variant_supported(int64_t d_state, int waves, int chunk)
{
#define X(N_, W_, C_, P_)                                        \
    if (d_state == N_ && waves == W_ && chunk == C_) return true;
    MAMBA_SCAN_VARIANTS(X)
#undef X
    return false;
}

// Defaults: 8 waves (d_state/8 state indices per lane) where d_state allows it, so a
// block holds 512 lanes; 16-step chunks.  Every default is in the variant table.
int default_waves(int64_t d_state) { return d_state >= 16 ? 8 : 4; }

int default_chunk(int64_t d_state, int waves)
{
    (void)d_state;
    (void)waves;
    return 16;
}

template <typename T, int N, int NW, int TC, int PD, bool FULL>
static hipError_t launch_variant(const ScanLaunch &p, hipStream_t stream)
{
    const int32_t tiles = (int32_t)((p.d_inner + 63) / 64);
    const int64_t blocks = (int64_t)tiles * p.batch * p.launch_spans;
    if (blocks <= 0)
        return hipSuccess;
    hipLaunchKernelGGL((scan_chunk_kernel<T, N, NW, TC, PD, FULL>), dim3((uint32_t)blocks),
                       dim3(64 * NW), 0, stream, (const T *)p.u, (const T *)p.delta,
                       (const T *)p.z, (const T *)p.B, (const T *)p.C, p.A, p.D, p.bias,
                       p.h_init, p.h_init_span_stride, (T *)p.y, p.h_last, p.ws_decay,
                       p.ws_hloc, p.L, (int32_t)p.d_inner, p.span_len, p.n_spans,
                       p.first_span, tiles, (int32_t)p.batch);
    return hipGetLastError();
}

template <bool FULL>
static hipError_t launch_any(const ScanLaunch &p, hipStream_t stream)
{
#define X(N_, W_, C_, P_)                                                                \
    if (p.d_state == N_ && p.waves == W_ && p.chunk == C_) {                             \
        if (p.dtype == DType::BF16)                                                      \
            return launch_variant<uint16_t, N_, W_, C_, P_, FULL>(p, stream);            \
        return launch_variant<float, N_, W_, C_, P_, FULL>(p, stream);                   \
    }
    MAMBA_SCAN_VARIANTS(X)
#undef X
    return hipErrorInvalidValue;
}

hipError_t launch_scan_full(const ScanLaunch &p, hipStream_t stream)
{
    return launch_any<true>(p, stream);
}

hipError_t launch_scan_end(const ScanLaunch &p, hipStream_t stream)
{
    return launch_any<false>(p, stream);
}

// ---------------------------------------------------------------------------
// carry pass: wavefront-level inclusive scan of (decay, end state) pairs over spans
// ---------------------------------------------------------------------------

// Value of `v` held by the lane `off` positions lower in the same row of 16 lanes (DPP
// row_shr); lanes without a source get `v` back, which the caller masks out.
template <int OFF>
__device__ __forceinline__ float row_shr(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v),
                                                      0x110 + OFF, 0xF, 0xF, false));
}

// Value held OFF lanes lower.  Segments of up to 16 lanes sit inside one DPP row, so
// row_shr reaches every source that matters; wider segments cross rows (ds_bpermute).
template <int SEG, int OFF>
__device__ __forceinline__ float lane_up(float v)
{
    if constexpr (SEG <= 16)
        return row_shr<OFF>(v);
    else
        return __shfl_up(v, OFF, 64);
}

// A block carries 64 consecutive state columns; each wave scans 64/SEG of them at a time,
// lane = (column, span).  Span s (< n_spans-1) contributes the map x -> decay_s * x + hloc_s;
// the inclusive composition over spans 0..s applied to h0 is the state entering span s+1.
// The results go through LDS so that the block writes each span's 64 columns as one
// contiguous run (h_in is [span][column]).
template <int SEG>
__global__ void __launch_bounds__(256)
carry_kernel(const float *__restrict__ decay, const float *__restrict__ hloc,
             const float *__restrict__ h0, float *__restrict__ h_in, int64_t columns,
             int32_t n_spans)
{
    constexpr int CPW = 64 / SEG; // columns per wave and round
    __shared__ float tile[SEG][65];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int64_t c0 = (int64_t)blockIdx.x * 64;
    const int s = lane % SEG;
    const int nmaps = n_spans - 1; // spans whose summary is needed
    // rounds per wave; every round's loads are issued before the first scan
    constexpr int R = 16 / CPW > 0 ? 16 / CPW : 1;
    float a[R], bb[R], x0[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int cl = (r * 4 + w) * CPW + lane / SEG; // local column
        const int64_t col = c0 + (cl < 64 ? cl : 63);
        const int64_t c = col < columns ? col : columns - 1;
        a[r] = 1.0f; // identity map
        bb[r] = 0.0f;
        if (s < nmaps) {
            a[r] = decay[c * n_spans + s];
            bb[r] = hloc[c * n_spans + s];
        }
        x0[r] = h0 ? h0[c] : 0.0f;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int cl = (r * 4 + w) * CPW + lane / SEG;
        float ar = a[r], br = bb[r];
        auto combine = [&](float ap, float bp, int off) {
            if (s >= off) { // (prefix up to s-off) then (own segment)
                br = __builtin_fmaf(ar, bp, br);
                ar = ar * ap;
            }
        };
        if constexpr (SEG > 1) { const float ap = lane_up<SEG, 1>(ar), bp = lane_up<SEG, 1>(br); combine(ap, bp, 1); }
        if constexpr (SEG > 2) { const float ap = lane_up<SEG, 2>(ar), bp = lane_up<SEG, 2>(br); combine(ap, bp, 2); }
        if constexpr (SEG > 4) { const float ap = lane_up<SEG, 4>(ar), bp = lane_up<SEG, 4>(br); combine(ap, bp, 4); }
        if constexpr (SEG > 8) { const float ap = lane_up<SEG, 8>(ar), bp = lane_up<SEG, 8>(br); combine(ap, bp, 8); }
        if constexpr (SEG > 16) { const float ap = lane_up<SEG, 16>(ar), bp = lane_up<SEG, 16>(br); combine(ap, bp, 16); }
        if constexpr (SEG > 32) { const float ap = lane_up<SEG, 32>(ar), bp = lane_up<SEG, 32>(br); combine(ap, bp, 32); }
        if (cl < 64)
            tile[s][cl] = __builtin_fmaf(ar, x0[r], br);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * (nmaps + 1); i += 256) {
        const int sp = i >> 6, j = i & 63;
        const int64_t col = c0 + j;
        if (col >= columns)
            continue;
        // span 0 enters with h0; span sp + 1 with the composition over spans 0..sp
        h_in[(int64_t)sp * columns + col] =
            sp == 0 ? (h0 ? h0[col] : 0.0f) : tile[sp - 1][j];
    }
}

// Carry with the pair rotation: a span maps a state pair x to M x + b with M its 2x2
// transition (rotations and unequal decays within a pair do not commute, so the scalar
// decays do not compose); one thread per pair walks the spans in order.
__global__ void __launch_bounds__(256)
carry_rot_kernel(const float *__restrict__ rot, const float *__restrict__ hloc,
                 const float *__restrict__ h0, float *__restrict__ h_in, int64_t columns,
                 int32_t n_spans)
{
    const int64_t pr = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; // state pair
    if (pr >= columns / 2)
        return;
    const int64_t c = 2 * pr;
    float x0 = h0 ? h0[c] : 0.0f, x1 = h0 ? h0[c + 1] : 0.0f;
    h_in[c] = x0;
    h_in[c + 1] = x1;
    for (int s = 0; s < n_spans - 1; ++s) {
        const float *m = rot + (pr * n_spans + s) * 4; // m00, m10, m01, m11
        const float y0 = __builtin_fmaf(m[0], x0, __builtin_fmaf(m[2], x1, hloc[c * n_spans + s]));
        const float y1 =
            __builtin_fmaf(m[1], x0, __builtin_fmaf(m[3], x1, hloc[(c + 1) * n_spans + s]));
        x0 = y0;
        x1 = y1;
        h_in[(int64_t)(s + 1) * columns + c] = x0;
        h_in[(int64_t)(s + 1) * columns + c + 1] = x1;
    }
}

hipError_t launch_carry(const CarryLaunch &p, hipStream_t stream)
{
    if (p.ws_rot) {
        const int64_t pairs = p.columns / 2;
        if (pairs <= 0)
            return hipSuccess;
        hipLaunchKernelGGL(carry_rot_kernel, dim3((uint32_t)((pairs + 255) / 256)), dim3(256), 0,
                           stream, p.ws_rot, p.ws_hloc, p.h0, p.h_in, p.columns, p.n_spans);
        return hipGetLastError();
    }
    const int nmaps = p.n_spans - 1;
    int seg = 1;
    while (seg < nmaps)
        seg <<= 1;
    if (seg > 64)
        return hipErrorInvalidValue;
    const int64_t blocks = (p.columns + 63) / 64;
    if (blocks <= 0)
        return hipSuccess;
#define CARRY_CASE(S_)                                                                    \
    case S_:                                                                             \
        hipLaunchKernelGGL((carry_kernel<S_>), dim3((uint32_t)blocks), dim3(256), 0,      \
                           stream, p.ws_decay, p.ws_hloc, p.h0, p.h_in, p.columns,        \
                           p.n_spans);                                                   \
        break;
    switch (seg) {
        CARRY_CASE(1)
        CARRY_CASE(2)
        CARRY_CASE(4)
        CARRY_CASE(8)
        CARRY_CASE(16)
        CARRY_CASE(32)
        CARRY_CASE(64)
    default:
        return hipErrorInvalidValue;
    }
#undef CARRY_CASE
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// empty sequence: h_last = h0 (or zeros)
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(256)
copy_state_kernel(float *__restrict__ dst, const float *__restrict__ src, int64_t count)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count)
        dst[i] = src ? src[i] : 0.0f;
}

hipError_t launch_copy_state(float *dst, const float *src, int64_t count, hipStream_t stream)
{
    if (count <= 0 || dst == src)
        return hipSuccess;
    const int64_t blocks = (count + 255) / 256;
    hipLaunchKernelGGL(copy_state_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, dst,
                       src, count);
    return hipGetLastError();
}

} // namespace mambascan
