// Single-token recurrent state update (decode) for gfx950.
//
// One step of h[n] = exp(Delta A[d,n]) h[n] + Delta B[n] u, y = (sum_n C[n] h[n] + D u)
// * silu(z), Delta = softplus(delta + bias), on a persistent fp32 state of shape
// (batch, d_inner, d_state) -- the constant-memory token loop "output, h = ssm(token, h)"
// of "State Space Models and Mamba" (metaphor-xennon.pages.dev, MambaDecoder).
//
// The step is bound by the state's read-modify-write (8 bytes per state element), so the
// layout is chosen for it: each lane owns 4 consecutive state indices of one channel and
// moves them with one 16-byte load and one 16-byte store, consecutive lanes covering
// consecutive addresses.  The N/4 lanes of a channel each compute the per-channel softplus
// and gate (spare VALU in a memory-bound kernel) and combine their partial readouts with a
// butterfly over N/4 lanes in a fixed order; the first lane of the channel stores y.  The
// state is loaded and stored non-temporally: a model's per-layer states together exceed
// the last-level cache, so a layer's state arrives from HBM on every token, and streaming
// it past the caches measured 10 % faster there (and 12 % slower when the one state is
// chained back to back from a warm cache, which a multi-layer decoder never sees).
//
// Options (the Mamba-3 section of "State space models and the Mamba series", jsqmd.com,
// sections 2.1 and 2.2): the exponential-trapezoidal input term (1 - lam) Delta
// B_prev u_prev + lam Delta B u, with the previous token's u and B supplied by the caller,
// and the rotation of each state pair (2k, 2k+1) by Delta theta[k] before the decay (the
// pairs of a lane's 4 states are its own).
#include "device_math.h"
#include "scan_common.h"

namespace mambascan {

struct StepExt {
    const void *lam, *u_prev, *B_prev, *theta; // (B,D), (B,D), (B,N), (B,N/2); rows of this launch
    int64_t su, sd, sz, sB, sC; // elements between batch rows of u, delta, z, B, C
};

// DISC: 0 Euler, 1 zero-order hold, 2 exponential-trapezoidal; ROT: pair rotation.
// GEN: d_state nr below the compiled N (a size without kernels of its own): the lanes of N
// are kept, state indices >= nr are skipped (their h, A, B, C read as 0, -1, 0, 0 and
// nothing stored), and the state moves with 4-byte accesses (rows of nr floats need not be
// 16-byte aligned).
template <typename T, int N, int DISC, bool ROT, bool GEN>
__global__ void __launch_bounds__(256)
state_update_kernel(float *__restrict__ h, const T *__restrict__ u, const T *__restrict__ delta,
                    const T *__restrict__ z, const T *__restrict__ Bm, const T *__restrict__ Cm,
                    const float *__restrict__ A, const float *__restrict__ Dv,
                    const float *__restrict__ bias, T *__restrict__ y, int32_t Dn, StepExt ext,
                    int32_t n_real)
{
    constexpr bool ZOH = DISC == 1, TRAP = DISC == 2;
    constexpr int LPC = N / 4; // lanes per channel
    static_assert(N % 4 == 0 && LPC <= 64, "bad d_state");
    const int nr = GEN ? n_real : N; // row length of h, A, B, C (and B_prev, 2 x theta)
    const int b = blockIdx.y;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; // (d, q) within row b
    const bool valid = i < (int64_t)Dn * LPC;
    const int d = valid ? (int)(i / LPC) : Dn - 1;
    const int q = (int)(i % LPC);

    const int64_t c = (int64_t)b * Dn + d; // channel index
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    f32x4 *hp = reinterpret_cast<f32x4 *>(h + c * nr) + q;
    float hin[4], ain[4];
    bool kv[4]; // state index 4q + k exists
#pragma unroll
    for (int k = 0; k < 4; ++k)
        kv[k] = !GEN || 4 * q + k < nr;
    if constexpr (GEN) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            hin[k] = kv[k] ? h[c * nr + 4 * q + k] : 0.0f;
            ain[k] = kv[k] ? A[(int64_t)d * nr + 4 * q + k] : -1.0f;
        }
    } else {
        const f32x4 hv = __builtin_nontemporal_load(hp);
        const float4 av = reinterpret_cast<const float4 *>(A + (int64_t)d * N)[q];
        hin[0] = hv.x, hin[1] = hv.y, hin[2] = hv.z, hin[3] = hv.w;
        ain[0] = av.x, ain[1] = av.y, ain[2] = av.z, ain[3] = av.w;
    }

    const float uu = load_val(u, b * ext.su + d);
    const float dl = softplus_act<T>(load_val(delta, b * ext.sd + d) + (bias ? bias[d] : 0.0f));
    const float w = dl * uu;
    const int64_t bn = (int64_t)b * nr + 4 * q;                 // B_prev, theta rows
    const int64_t bB = (int64_t)b * ext.sB + 4 * q, bC = (int64_t)b * ext.sC + 4 * q;

    float hn[4];
    if constexpr (ROT) { // (nr even: a pair exists whole or not at all)
#pragma unroll
        for (int k = 0; k < 4; k += 2)
            if (kv[k])
                rotate_pair_act<T>(dl * load_val((const T *)ext.theta, ((int64_t)b * nr + 4 * q + k) / 2),
                            hin[k], hin[k + 1]);
    }
    float lm = 1.0f, p_lb = 0.0f;
    if constexpr (TRAP) {
        lm = load_val((const T *)ext.lam, c);
        p_lb = (1.0f - lm) * dl * (ext.u_prev ? load_val((const T *)ext.u_prev, c) : 0.0f);
    }
    float yp = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float a = decay_exp2(dl, ain[k] * kLog2e);
        float bu = w; // Bbar u / B: Euler Delta u, or the zero-order hold
        if constexpr (ZOH)
            bu = zoh_input(dl * ain[k], a, w, uu / ain[k]);
        const float bk = kv[k] ? load_val(Bm, bB + k) : 0.0f;
        const float ck = kv[k] ? load_val(Cm, bC + k) : 0.0f;
        if constexpr (TRAP) {
            const float bp = ext.B_prev && kv[k] ? load_val((const T *)ext.B_prev, bn + k) : 0.0f;
            hn[k] = __builtin_fmaf(a, hin[k], __builtin_fmaf(p_lb, bp, lm * w * bk));
        } else {
            hn[k] = __builtin_fmaf(a, hin[k], bu * bk);
        }
        yp = __builtin_fmaf(ck, hn[k], yp);
    }
#pragma unroll
    for (int m = 1; m < LPC; m <<= 1)
        yp += __shfl_xor(yp, m, 64);

    if (!valid)
        return;
    if constexpr (GEN) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (kv[k])
                h[c * nr + 4 * q + k] = hn[k];
    } else {
        const f32x4 ho = {hn[0], hn[1], hn[2], hn[3]};
        __builtin_nontemporal_store(ho, hp);
    }
    if (q == 0) {
        float yv = yp + (Dv ? Dv[d] : 0.0f) * uu;
        if (z)
            yv *= silu_f(load_val(z, b * ext.sz + d));
        store_val(y, c, yv);
    }
}

template <typename T, int N, int DISC, bool ROT>
static hipError_t launch_step(const StepLaunch &p, hipStream_t stream)
{
    constexpr int LPC = N / 4;
    const bool gen = p.d_state != N;
    const int64_t nr = p.d_state;
    const int64_t lanes = p.d_inner * LPC;
    const uint32_t gx = (uint32_t)((lanes + 255) / 256);
    // gridDim.y is limited; walk the batch in slices of at most 65535 rows
    for (int64_t b0 = 0; b0 < p.batch; b0 += 65535) {
        const int64_t nb = p.batch - b0 < 65535 ? p.batch - b0 : 65535;
        const int64_t off_bd = b0 * p.d_inner, off_bn = b0 * nr;
        StepExt ext{};
        ext.su = p.su;
        ext.sd = p.sd;
        ext.sz = p.sz;
        ext.sB = p.sB;
        ext.sC = p.sC;
        ext.lam = p.lam ? (const T *)p.lam + off_bd : nullptr;
        ext.u_prev = p.u_prev ? (const T *)p.u_prev + off_bd : nullptr;
        ext.B_prev = p.B_prev ? (const T *)p.B_prev + off_bn : nullptr;
        ext.theta = p.theta ? (const T *)p.theta + b0 * (nr / 2) : nullptr;
        if (gen)
            hipLaunchKernelGGL((state_update_kernel<T, N, DISC, ROT, true>),
                               dim3(gx, (uint32_t)nb), dim3(256), 0, stream,
                               p.h + off_bd * nr, (const T *)p.u + b0 * p.su,
                               (const T *)p.delta + b0 * p.sd,
                               p.z ? (const T *)p.z + b0 * p.sz : nullptr,
                               (const T *)p.B + b0 * p.sB, (const T *)p.C + b0 * p.sC, p.A, p.D,
                               p.bias, (T *)p.y + off_bd, (int32_t)p.d_inner, ext, (int32_t)nr);
        else
            hipLaunchKernelGGL((state_update_kernel<T, N, DISC, ROT, false>),
                               dim3(gx, (uint32_t)nb), dim3(256), 0, stream,
                               p.h + off_bd * nr, (const T *)p.u + b0 * p.su,
                               (const T *)p.delta + b0 * p.sd,
                               p.z ? (const T *)p.z + b0 * p.sz : nullptr,
                               (const T *)p.B + b0 * p.sB, (const T *)p.C + b0 * p.sC, p.A, p.D,
                               p.bias, (T *)p.y + off_bd, (int32_t)p.d_inner, ext, (int32_t)nr);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

template <typename T, int N>
static hipError_t launch_step_opts(const StepLaunch &p, hipStream_t stream)
{
    const int disc = p.trap ? 2 : p.zoh ? 1 : 0;
    if (p.rot) {
        switch (disc) {
        case 2: return launch_step<T, N, 2, true>(p, stream);
        case 1: return launch_step<T, N, 1, true>(p, stream);
        default: return launch_step<T, N, 0, true>(p, stream);
        }
    }
    switch (disc) {
    case 2: return launch_step<T, N, 2, false>(p, stream);
    case 1: return launch_step<T, N, 1, false>(p, stream);
    default: return launch_step<T, N, 0, false>(p, stream);
    }
}

hipError_t launch_state_update(const StepLaunch &p, hipStream_t stream)
{
    if (p.batch <= 0 || p.d_inner <= 0)
        return hipSuccess;
    // a d_state without kernels of its own runs in the next compiled size's lanes
    int64_t np = 4;
    while (np < p.d_state)
        np *= 2;
#define STEP_CASE(N_)                                                   \
    if (np == N_) {                                                     \
        if (p.dtype == DType::BF16)                                     \
            return launch_step_opts<uint16_t, N_>(p, stream);           \
        return launch_step_opts<float, N_>(p, stream);                  \
    }
    STEP_CASE(4)
    STEP_CASE(8)
    STEP_CASE(16)
    STEP_CASE(32)
    STEP_CASE(64)
#undef STEP_CASE
    return hipErrorInvalidValue;
}

} // namespace mambascan
