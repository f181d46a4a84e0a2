// Single-token state update (recurrent decoding) of the Mamba-2 SSD for gfx950.
//
// One step of the SSD recurrence ("Understanding Mamba" (aiattnstudio.link) section 6 and
// "State space models and the Mamba series" (jsqmd.com) section 1.2): per batch row b and
// head h, with Delta = softplus(dt[b,h] + dt_bias[h]) and abar = exp(Delta A[h]) shared by
// the head's P channels and all N state indices,
//   H[p,n] <- abar H[p,n] + Delta B[b,n] x[b,h*P+p],
//   y[b,h*P+p] = (sum_n C[b,n] H[p,n] + D[h] x[b,h*P+p]) * silu(z[b,h*P+p]),
// on the persistent fp32 state (batch, H * P, N) -- the token loop of the recurrent form,
// the chunked scan (ssd.hip) being its parallel form over a sequence.
//
// The step is bound by the state's read-modify-write (8 bytes per state element): each lane
// owns 4 consecutive state indices of one channel and moves them with one 16-byte
// non-temporal load and store (consecutive lanes, consecutive addresses; a model's layers
// together hold more state than the last-level cache, so it is streamed past the caches as
// in the Mamba-1 decode step).  The decay is one exp per lane, the scalar A being shared by
// the lane's four states.  The N/4 lanes of a channel combine their partial readouts with a
// butterfly in a fixed order; the first of them writes y.
#include "device_math.h"
#include "ssd.h"

namespace mambascan {
namespace {

template <typename T, int N>
__global__ void __launch_bounds__(256)
ssd_step_kernel(float *__restrict__ h, const T *__restrict__ x, const T *__restrict__ dt,
                const T *__restrict__ z, const T *__restrict__ Bm, const T *__restrict__ Cm,
                const float *__restrict__ A, const float *__restrict__ Dv,
                const float *__restrict__ bias, T *__restrict__ y, int32_t H, int32_t P)
{
    constexpr int LPC = N / 4; // lanes per channel
    static_assert(N % 4 == 0 && LPC <= 64 && (LPC & (LPC - 1)) == 0, "bad d_state");
    const int b = blockIdx.y;
    const int64_t Dn = (int64_t)H * P;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; // (channel, q) of row b
    const bool valid = i < Dn * LPC;
    const int64_t d = valid ? i / LPC : Dn - 1;
    const int q = (int)(i % LPC);
    const int hd = (int)(d / P);

    const int64_t c = (int64_t)b * Dn + d; // channel index
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    f32x4 *hp = reinterpret_cast<f32x4 *>(h + c * N) + q;
    const f32x4 hv = __builtin_nontemporal_load(hp);

    const float xv = load_val(x, c);
    const float dl = softplus_act<T>(load_val(dt, (int64_t)b * H + hd) + (bias ? bias[hd] : 0.0f));
    const float a = decay_exp2(dl, A[hd] * kLog2e);
    const float w = dl * xv;
    const int64_t bn = (int64_t)b * N + 4 * q;

    float hn[4];
    const float hin[4] = {hv.x, hv.y, hv.z, hv.w};
    float yp = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        hn[k] = __builtin_fmaf(a, hin[k], w * load_val(Bm, bn + k));
        yp = __builtin_fmaf(load_val(Cm, bn + k), hn[k], yp);
    }
#pragma unroll
    for (int m = 1; m < LPC; m <<= 1)
        yp += __shfl_xor(yp, m, 64);

    if (!valid)
        return;
    const f32x4 ho = {hn[0], hn[1], hn[2], hn[3]};
    __builtin_nontemporal_store(ho, hp);
    if (q == 0) {
        float yv = yp + (Dv ? Dv[hd] : 0.0f) * xv;
        if (z)
            yv *= silu_f(load_val(z, c));
        store_val(y, c, yv);
    }
}

template <typename T, int N>
hipError_t launch_step_t(const SsdStepLaunch &p, hipStream_t stream)
{
    constexpr int LPC = N / 4;
    const int64_t lanes = p.n_heads * p.head_dim * LPC;
    const uint32_t gx = (uint32_t)((lanes + 255) / 256);
    // gridDim.y is limited; walk the batch in slices of at most 65535 rows
    for (int64_t b0 = 0; b0 < p.batch; b0 += 65535) {
        const int64_t nb = p.batch - b0 < 65535 ? p.batch - b0 : 65535;
        const int64_t off_bd = b0 * p.n_heads * p.head_dim;
        hipLaunchKernelGGL((ssd_step_kernel<T, N>), dim3(gx, (uint32_t)nb), dim3(256), 0, stream,
                           p.h + off_bd * N, (const T *)p.x + off_bd,
                           (const T *)p.dt + b0 * p.n_heads,
                           p.z ? (const T *)p.z + off_bd : nullptr, (const T *)p.B + b0 * N,
                           (const T *)p.C + b0 * N, p.A, p.D, p.dt_bias, (T *)p.y + off_bd,
                           (int32_t)p.n_heads, (int32_t)p.head_dim);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

} // namespace

hipError_t launch_ssd_step(const SsdStepLaunch &p, hipStream_t stream)
{
    if (p.batch <= 0 || p.n_heads <= 0)
        return hipSuccess;
    const bool bf = p.dtype == DType::BF16;
    switch (p.d_state) {
    case 64: return bf ? launch_step_t<uint16_t, 64>(p, stream) : launch_step_t<float, 64>(p, stream);
    case 128: return bf ? launch_step_t<uint16_t, 128>(p, stream) : launch_step_t<float, 128>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace mambascan
