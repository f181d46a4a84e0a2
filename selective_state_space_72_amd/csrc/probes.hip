// Measurement probes: a device copy (achievable HBM bandwidth) and instruction-issue kernels
// (achievable rates of the VALU forms the selective scan's state update is made of).  They
// give the measured ceilings the scan kernels are compared with; they compute nothing of
// the scan.  Declared in include/mamba_probe.h.
#include "mamba_probe.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace {

// Keep the compiler from hoisting, folding or dropping a value without emitting any
// instruction.
#define PROBE_OPAQUE(x) asm volatile("" : "+v"(x))
#define PROBE_USE(x) asm volatile("" ::"v"(x))

constexpr int kChains = 8;     // independent dependency chains per lane
constexpr int kThreads = 256;  // one wave per SIMD per block
constexpr int kUpdSteps = 8;   // time steps per iteration of the update probe
constexpr int kUpdStates = 2;  // state indices per lane in the update probe

__global__ void __launch_bounds__(256) copy_kernel(const float4 *__restrict__ src,
                                                    float4 *__restrict__ dst, size_t n)
{
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride)
        dst[i] = src[i];
}

// Value of v in lane K of the caller's 16-lane row (DPP row_newbcast); as the first
// operand of a multiply or FMA the broadcast folds into the instruction.
template <int K>
__device__ __forceinline__ float row_bcast(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + K, 0xF, 0xF, true));
}

// acc += (v in lane K of the caller's 16-lane row) * w as one v_fmac_f32_dpp (the compiler
// does not fold a broadcast into v_fmac).  v must not have been written by a VALU
// instruction in the two instructions before (DPP read hazard): the callers' v comes from
// memory or is set up well before the loop.
template <int K>
__device__ __forceinline__ void fmac_bcast(float &acc, float v, float w)
{
    asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                 : "+v"(acc)
                 : "v"(v), "v"(w), "i"(K));
}

// One kernel per instruction form; `iters` iterations of kChains independent instructions.
template <int KIND>
__global__ void __launch_bounds__(kThreads) issue_kernel(float s, float s2, int iters,
                                                          float *__restrict__ sink)
{
    float acc[kChains];
    const float v1 = 0.9999f + threadIdx.x * 1e-9f, v2 = threadIdx.x * 1e-8f;
#pragma unroll
    for (int k = 0; k < kChains; ++k)
        acc[k] = threadIdx.x * 1e-4f + k * 0.01f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < kChains; ++k) {
            if constexpr (KIND == MAMBA_PROBE_FMA_VGPR) {
                acc[k] = __builtin_fmaf(v1, v2, acc[k]); // v_fmac_f32, VGPR operands
            } else if constexpr (KIND == MAMBA_PROBE_FMA_SGPR) {
                acc[k] = __builtin_fmaf(s, v1, acc[k]); // v_fmac_f32 with an SGPR operand
            } else if constexpr (KIND == MAMBA_PROBE_FMA_DPP) {
                // v_fmac_f32 with src0 = lane 5 of each 16-lane row (row_newbcast:5)
                fmac_bcast<5>(acc[k], v1, v2);
            } else if constexpr (KIND == MAMBA_PROBE_EXP) {
                PROBE_OPAQUE(acc[k]);
                const float r = __builtin_amdgcn_exp2f(acc[k]); // v_exp_f32
                PROBE_USE(r);
            }
        }
    }
    float r = 0.0f;
#pragma unroll
    for (int k = 0; k < kChains; ++k)
        r += acc[k];
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = r + s2;
}

// B and C of the update probe: kernel arguments, so scalar registers.
struct UpdBC {
    float b[kUpdSteps][kUpdStates], c[kUpdSteps][kUpdStates];
};

// The scan's state update as its kernels issue it: per element x = fma(Delta, A', c),
// a = exp2(x), h = fma(a, h, (Delta u) * B), y = fma(C, h, y), with B and C uniform scalar
// operands; kUpdStates states per lane, kUpdSteps steps per iteration, the exps of an
// iteration issued first.  Delta and Delta*u are opaque per step.
__global__ void __launch_bounds__(kThreads) update_kernel(UpdBC bc, int iters,
                                                           float *__restrict__ sink)
{
    float h[kUpdStates], a2[kUpdStates], y = 0.0f;
#pragma unroll
    for (int q = 0; q < kUpdStates; ++q) {
        h[q] = 0.0f;
        a2[q] = -(q + 1) * 1.4427f - threadIdx.x * 1e-6f;
    }
    float dt[kUpdSteps], du[kUpdSteps];
#pragma unroll
    for (int t = 0; t < kUpdSteps; ++t) {
        dt[t] = 1e-3f * (t + 1) + threadIdx.x * 1e-7f;
        du[t] = 0.3f * t;
    }
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int t = 0; t < kUpdSteps; ++t) {
            PROBE_OPAQUE(dt[t]);
            PROBE_OPAQUE(du[t]);
        }
        float a[kUpdSteps][kUpdStates];
#pragma unroll
        for (int t = 0; t < kUpdSteps; ++t)
#pragma unroll
            for (int q = 0; q < kUpdStates; ++q)
                a[t][q] = __builtin_amdgcn_exp2f(__builtin_fmaf(dt[t], a2[q], 8e-9f));
#pragma unroll
        for (int t = 0; t < kUpdSteps; ++t) {
#pragma unroll
            for (int q = 0; q < kUpdStates; ++q) {
                h[q] = __builtin_fmaf(a[t][q], h[q], du[t] * bc.b[t][q]);
                y = __builtin_fmaf(bc.c[t][q], h[q], y);
            }
        }
    }
    float r = y;
#pragma unroll
    for (int q = 0; q < kUpdStates; ++q)
        r += h[q];
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = r;
}

// The same update with B and C as vector registers holding one (step, state) value per lane
// of each 16-lane row (lane 2t + q), taken by row broadcasts folded into the multiply and the
// readout FMA: no scalar operands.
__global__ void __launch_bounds__(kThreads) update_dpp_kernel(UpdBC bc, int iters,
                                                               float *__restrict__ sink)
{
    float h[kUpdStates], a2[kUpdStates], y = 0.0f;
#pragma unroll
    for (int q = 0; q < kUpdStates; ++q) {
        h[q] = 0.0f;
        a2[q] = -(q + 1) * 1.4427f - threadIdx.x * 1e-6f;
    }
    const int j = threadIdx.x & 15;
    float vb = bc.b[0][0], vc = bc.c[0][0];
#pragma unroll
    for (int t = 0; t < kUpdSteps; ++t)
#pragma unroll
        for (int q = 0; q < kUpdStates; ++q) {
            vb = j == kUpdStates * t + q ? bc.b[t][q] : vb;
            vc = j == kUpdStates * t + q ? bc.c[t][q] : vc;
        }
    float dt[kUpdSteps], du[kUpdSteps];
#pragma unroll
    for (int t = 0; t < kUpdSteps; ++t) {
        dt[t] = 1e-3f * (t + 1) + threadIdx.x * 1e-7f;
        du[t] = 0.3f * t;
    }
    asm volatile("s_nop 4" ::: "memory"); // vb, vc written by VALU just above: DPP hazard
    auto bcast = [](float v, auto K) { return row_bcast<decltype(K)::value>(v); };
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int t = 0; t < kUpdSteps; ++t) {
            PROBE_OPAQUE(dt[t]);
            PROBE_OPAQUE(du[t]);
        }
        PROBE_OPAQUE(vb);
        PROBE_OPAQUE(vc);
        float a[kUpdSteps][kUpdStates];
#pragma unroll
        for (int t = 0; t < kUpdSteps; ++t)
#pragma unroll
            for (int q = 0; q < kUpdStates; ++q)
                a[t][q] = __builtin_amdgcn_exp2f(__builtin_fmaf(dt[t], a2[q], 8e-9f));
#define UPD_STEP(T, Q)                                                                       \
    h[Q] = __builtin_fmaf(a[T][Q], h[Q], bcast(vb, std::integral_constant<int, 2 * T + Q>{}) * du[T]); \
    fmac_bcast<2 * T + Q>(y, vc, h[Q]);
        UPD_STEP(0, 0) UPD_STEP(0, 1) UPD_STEP(1, 0) UPD_STEP(1, 1)
        UPD_STEP(2, 0) UPD_STEP(2, 1) UPD_STEP(3, 0) UPD_STEP(3, 1)
        UPD_STEP(4, 0) UPD_STEP(4, 1) UPD_STEP(5, 0) UPD_STEP(5, 1)
        UPD_STEP(6, 0) UPD_STEP(6, 1) UPD_STEP(7, 0) UPD_STEP(7, 1)
#undef UPD_STEP
    }
    float r = y;
#pragma unroll
    for (int q = 0; q < kUpdStates; ++q)
        r += h[q];
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = r;
}

} // namespace

extern "C" {

mamba_status_t mamba_probe_copy(const void *src, void *dst, size_t bytes, int32_t blocks,
                                void *stream)
{
    if (!src || !dst)
        return MAMBA_ERR_NULL_ARG;
    if (bytes % 16 != 0 || blocks <= 0)
        return MAMBA_ERR_BAD_SHAPE;
    if (reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16)
        return MAMBA_ERR_MISALIGNED;
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
    if (bytes > 0 && s0 < d0 + bytes && d0 < s0 + bytes)
        return MAMBA_ERR_ALIASING;
    if (bytes == 0)
        return MAMBA_OK;
    hipLaunchKernelGGL(copy_kernel, dim3((uint32_t)blocks), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream),
                       static_cast<const float4 *>(src), static_cast<float4 *>(dst), bytes / 16);
    return hipGetLastError() == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

mamba_status_t mamba_probe_issue(int32_t kind, int32_t waves_per_simd, int32_t iters,
                                 int32_t compute_units, float *sink, uint64_t *wave_instr,
                                 void *stream)
{
    if (!sink || !wave_instr)
        return MAMBA_ERR_NULL_ARG;
    if (waves_per_simd < 1 || waves_per_simd > 8 || iters < 1 || compute_units < 1)
        return MAMBA_ERR_BAD_SHAPE;
    const uint32_t blocks = (uint32_t)compute_units * (uint32_t)waves_per_simd;
    const uint64_t waves = (uint64_t)blocks * (kThreads / 64);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const float s = 1.0001f, s2 = 0.5f;
    switch (kind) {
    case MAMBA_PROBE_FMA_VGPR:
        hipLaunchKernelGGL(issue_kernel<MAMBA_PROBE_FMA_VGPR>, dim3(blocks), dim3(kThreads), 0, st,
                           s, s2, iters, sink);
        *wave_instr = waves * (uint64_t)iters * kChains;
        break;
    case MAMBA_PROBE_FMA_SGPR:
        hipLaunchKernelGGL(issue_kernel<MAMBA_PROBE_FMA_SGPR>, dim3(blocks), dim3(kThreads), 0, st,
                           s, s2, iters, sink);
        *wave_instr = waves * (uint64_t)iters * kChains;
        break;
    case MAMBA_PROBE_FMA_DPP:
        hipLaunchKernelGGL(issue_kernel<MAMBA_PROBE_FMA_DPP>, dim3(blocks), dim3(kThreads), 0, st,
                           s, s2, iters, sink);
        *wave_instr = waves * (uint64_t)iters * kChains;
        break;
    case MAMBA_PROBE_EXP:
        hipLaunchKernelGGL(issue_kernel<MAMBA_PROBE_EXP>, dim3(blocks), dim3(kThreads), 0, st, s,
                           s2, iters, sink);
        *wave_instr = waves * (uint64_t)iters * kChains;
        break;
    case MAMBA_PROBE_UPDATE:
    case MAMBA_PROBE_UPDATE_DPP: {
        UpdBC bc;
        for (int t = 0; t < kUpdSteps; ++t) {
            for (int q = 0; q < kUpdStates; ++q) {
                bc.b[t][q] = 0.1f * t + q;
                bc.c[t][q] = 0.05f * t - q;
            }
        }
        if (kind == MAMBA_PROBE_UPDATE)
            hipLaunchKernelGGL(update_kernel, dim3(blocks), dim3(kThreads), 0, st, bc, iters, sink);
        else
            hipLaunchKernelGGL(update_dpp_kernel, dim3(blocks), dim3(kThreads), 0, st, bc, iters,
                               sink);
        *wave_instr = waves * (uint64_t)iters * kUpdSteps * kUpdStates; // wave-element updates
        break;
    }
    default:
        return MAMBA_ERR_UNSUPPORTED;
    }
    return hipGetLastError() == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

} // extern "C"
