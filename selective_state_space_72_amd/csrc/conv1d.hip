// Causal depthwise convolution + SiLU for gfx950 (the Mamba block's conv1d, which
// produces the scan's input u).
//
// Operation ("Understanding Mamba", aiattnstudio.link, sections 3.2 and 5.2: a
// depthwise nn.Conv1d with kernel K, padding K - 1 and a bias, first L outputs, then
// SiLU):  u[b,t,d] = silu(bias[d] + sum_k w[d,k] * xe[b, t-(K-1)+k, d]), where xe is x
// for t >= 0 and the carried state (the previous segment's last K - 1 inputs) before.
//
// The prefill is bound by HBM traffic (2 bytes read and 2 written per channel-step in
// bf16), so the layout is chosen for streaming: a lane owns V consecutive channels
// (one 8-byte load of 4 bf16 values, or 16 bytes of fp32) and walks a span of time
// steps, keeping the last K - 1 inputs in registers, so every input is read once plus
// K - 1 rows of overlap per span.  Several rows are requested together before any is
// used.  The block of the first span of each channel group also writes the outgoing
// state, which it can read from x at any time: with state_in == state_out, the only
// reader of the old state is the same thread, before it writes.
#include "device_math.h"
#include "scan_common.h"

namespace mambascan {
namespace {

template <typename T, int V> struct Vec;
template <> struct Vec<uint16_t, 1> { typedef uint16_t type; };
template <> struct Vec<uint16_t, 4> { typedef ushort4 type; };
template <> struct Vec<float, 1> { typedef float type; };
template <> struct Vec<float, 4> { typedef float4 type; };

// V consecutive values moved as one access of V * sizeof(T) bytes
template <typename T, int V>
__device__ __forceinline__ void vload(const T *p, float (&out)[V])
{
    if constexpr (V == 1) {
        out[0] = load_val(p, 0);
    } else {
        const typename Vec<T, V>::type v = *reinterpret_cast<const typename Vec<T, V>::type *>(p);
        out[0] = widen(v.x);
        out[1] = widen(v.y);
        out[2] = widen(v.z);
        out[3] = widen(v.w);
    }
}

template <typename T, int V>
__device__ __forceinline__ void vstore(T *p, const float (&in)[V])
{
    if constexpr (V == 1) {
        store_val(p, 0, in[0]);
    } else if constexpr (sizeof(T) == 2) {
        ushort4 v;
        v.x = __builtin_bit_cast(uint16_t, static_cast<__bf16>(in[0]));
        v.y = __builtin_bit_cast(uint16_t, static_cast<__bf16>(in[1]));
        v.z = __builtin_bit_cast(uint16_t, static_cast<__bf16>(in[2]));
        v.w = __builtin_bit_cast(uint16_t, static_cast<__bf16>(in[3]));
        *reinterpret_cast<ushort4 *>(p) = v;
    } else {
        *reinterpret_cast<float4 *>(p) = make_float4(in[0], in[1], in[2], in[3]);
    }
}

constexpr int kConvThreads = 256;
constexpr int kConvRows = 8; // steps requested together

// grid: (channel groups of kConvThreads * V, spans, batch)
template <typename T, int V, int K>
__global__ void __launch_bounds__(kConvThreads)
conv1d_silu_kernel(const T *__restrict__ x, const float *__restrict__ w,
                   const float *__restrict__ bias, const T *state_in, T *__restrict__ u,
                   T *state_out, int64_t L, int32_t Dn, int32_t span_len)
{
    constexpr int S = K - 1;
    const int b = blockIdx.z;
    const int span = blockIdx.y;
    const int d0 = (blockIdx.x * kConvThreads + threadIdx.x) * V;
    if (d0 >= Dn)
        return;
    const int64_t t_begin = (int64_t)span * span_len;
    const int64_t t_end = min(t_begin + (int64_t)span_len, L);
    const T *xb = x + (int64_t)b * L * Dn + d0;
    T *ub = u + (int64_t)b * L * Dn + d0;

    float wk[K][V], bs[V];
#pragma unroll
    for (int c = 0; c < V; ++c) {
        bs[c] = bias ? bias[d0 + c] : 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k)
            wk[k][c] = w[(int64_t)(d0 + c) * K + k];
    }

    // history: hist[j] = xe at t - S + j, j = 0..S-1 (oldest first)
    float hist[S > 0 ? S : 1][V];
    const int64_t st_base = ((int64_t)b * Dn + d0) * S;
#pragma unroll
    for (int j = 0; j < S; ++j) {
        const int64_t s = t_begin - S + j;
        if (s >= 0) {
            vload<T, V>(xb + s * Dn, hist[j]);
        } else {
#pragma unroll
            for (int c = 0; c < V; ++c)
                hist[j][c] = state_in ? load_val(state_in, st_base + (int64_t)c * S + (S + s))
                                      : 0.0f;
        }
    }

    // the outgoing state: the last S inputs of the sequence (read before anything is
    // written to state_out, by this thread only)
    if (state_out && span == 0) {
        float fin[S > 0 ? S : 1][V];
#pragma unroll
        for (int j = 0; j < S; ++j) {
            const int64_t s = L - S + j;
            if (s >= 0) {
                vload<T, V>(xb + s * Dn, fin[j]);
            } else {
#pragma unroll
                for (int c = 0; c < V; ++c)
                    fin[j][c] = state_in ? load_val(state_in, st_base + (int64_t)c * S + (S + s))
                                         : 0.0f;
            }
        }
#pragma unroll
        for (int j = 0; j < S; ++j)
#pragma unroll
            for (int c = 0; c < V; ++c)
                store_val(state_out, st_base + (int64_t)c * S + j, fin[j][c]);
    }

    for (int64_t t0 = t_begin; t0 < t_end; t0 += kConvRows) {
        const int nr = (int)min((int64_t)kConvRows, t_end - t0);
        float xr[kConvRows][V];
#pragma unroll
        for (int r = 0; r < kConvRows; ++r)
            if (r < nr)
                vload<T, V>(xb + (t0 + r) * Dn, xr[r]);
#pragma unroll
        for (int r = 0; r < kConvRows; ++r) {
            if (r < nr) {
                float out[V];
#pragma unroll
                for (int c = 0; c < V; ++c) {
                    float acc = bs[c];
#pragma unroll
                    for (int k = 0; k < S; ++k)
                        acc = __builtin_fmaf(wk[k][c], hist[k][c], acc);
                    acc = __builtin_fmaf(wk[S][c], xr[r][c], acc);
                    out[c] = silu_f(acc);
                }
                vstore<T, V>(ub + (t0 + r) * Dn, out);
#pragma unroll
                for (int j = 0; j + 1 < S; ++j)
#pragma unroll
                    for (int c = 0; c < V; ++c)
                        hist[j][c] = hist[j + 1][c];
                if constexpr (S > 0) {
#pragma unroll
                    for (int c = 0; c < V; ++c)
                        hist[S - 1][c] = xr[r][c];
                }
            }
        }
    }
}

// One decode token per (b, d): lane = channel.
template <typename T, int K>
__global__ void __launch_bounds__(kConvThreads)
conv1d_silu_update_kernel(T *state, const T *__restrict__ x, const float *__restrict__ w,
                          const float *__restrict__ bias, T *__restrict__ u, int64_t BD,
                          int32_t Dn)
{
    constexpr int S = K - 1;
    const int64_t i = (int64_t)blockIdx.x * kConvThreads + threadIdx.x; // b * Dn + d
    if (i >= BD)
        return;
    const int d = (int)(i % Dn);
    const float xn = load_val(x, i);
    float st[S];
#pragma unroll
    for (int k = 0; k < S; ++k)
        st[k] = load_val(state, i * S + k);
    float acc = bias ? bias[d] : 0.0f;
#pragma unroll
    for (int k = 0; k < S; ++k)
        acc = __builtin_fmaf(w[(int64_t)d * K + k], st[k], acc);
    acc = __builtin_fmaf(w[(int64_t)d * K + S], xn, acc);
    store_val(u, i, silu_f(acc));
#pragma unroll
    for (int k = 0; k + 1 < S; ++k)
        store_val(state, i * S + k, st[k + 1]);
    store_val(state, i * S + (S - 1), xn);
}

constexpr int kConvSpan = 128; // time steps per block

template <typename T, int V, int K>
hipError_t launch_conv_t(const ConvLaunch &p, hipStream_t stream)
{
    const int64_t groups = (p.d_inner + (int64_t)kConvThreads * V - 1) / ((int64_t)kConvThreads * V);
    // at least one span, so that an empty sequence still passes the state through
    const int64_t spans = p.L > 0 ? (p.L + kConvSpan - 1) / kConvSpan : 1;
    if (groups <= 0 || p.batch <= 0)
        return hipSuccess;
    hipLaunchKernelGGL((conv1d_silu_kernel<T, V, K>),
                       dim3((uint32_t)groups, (uint32_t)spans, (uint32_t)p.batch),
                       dim3(kConvThreads), 0, stream, (const T *)p.x, p.w, p.bias,
                       (const T *)p.state_in, (T *)p.u, (T *)p.state_out, p.L,
                       (int32_t)p.d_inner, kConvSpan);
    return hipGetLastError();
}

template <typename T, int K>
hipError_t launch_conv_update_t(const ConvLaunch &p, hipStream_t stream)
{
    const int64_t bd = p.batch * p.d_inner;
    const int64_t blocks = (bd + kConvThreads - 1) / kConvThreads;
    if (blocks <= 0)
        return hipSuccess;
    hipLaunchKernelGGL((conv1d_silu_update_kernel<T, K>), dim3((uint32_t)blocks),
                       dim3(kConvThreads), 0, stream, (T *)p.state_out, (const T *)p.x, p.w,
                       p.bias, (T *)p.u, bd, (int32_t)p.d_inner);
    return hipGetLastError();
}

template <typename T, int V>
hipError_t launch_conv_k(const ConvLaunch &p, hipStream_t stream)
{
    switch (p.d_conv) {
    case 2: return launch_conv_t<T, V, 2>(p, stream);
    case 3: return launch_conv_t<T, V, 3>(p, stream);
    case 4: return launch_conv_t<T, V, 4>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace

hipError_t launch_conv1d_silu(const ConvLaunch &p, hipStream_t stream)
{
    // 4 channels per lane where the channel count and alignment allow (8 bf16 channels
    // per lane with 16-byte accesses measured 37 % slower at 8 x 4096 x 5120)
    if (p.dtype == DType::BF16)
        return p.vec4 ? launch_conv_k<uint16_t, 4>(p, stream) : launch_conv_k<uint16_t, 1>(p, stream);
    return p.vec4 ? launch_conv_k<float, 4>(p, stream) : launch_conv_k<float, 1>(p, stream);
}

hipError_t launch_conv1d_silu_update(const ConvLaunch &p, hipStream_t stream)
{
    const bool bf = p.dtype == DType::BF16;
    switch (p.d_conv) {
    case 2: return bf ? launch_conv_update_t<uint16_t, 2>(p, stream) : launch_conv_update_t<float, 2>(p, stream);
    case 3: return bf ? launch_conv_update_t<uint16_t, 3>(p, stream) : launch_conv_update_t<float, 3>(p, stream);
    case 4: return bf ? launch_conv_update_t<uint16_t, 4>(p, stream) : launch_conv_update_t<float, 4>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace mambascan
