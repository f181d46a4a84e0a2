// Measurement probes: a device copy (achievable HBM bandwidth) and instruction-issue kernels
// (achievable rates of the VALU forms the selective scan's state update is made of).  They
// give the measured ceilings the scan kernels are compared with; they compute nothing of
// the scan.  Declared in include/mamba_probe.h.
#include "mamba_probe.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

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
    case MAMBA_PROBE_EXP:
        hipLaunchKernelGGL(issue_kernel<MAMBA_PROBE_EXP>, dim3(blocks), dim3(kThreads), 0, st, s,
                           s2, iters, sink);
        *wave_instr = waves * (uint64_t)iters * kChains;
        break;
    case MAMBA_PROBE_UPDATE: {
        UpdBC bc;
        for (int t = 0; t < kUpdSteps; ++t) {
            for (int q = 0; q < kUpdStates; ++q) {
                bc.b[t][q] = 0.1f * t + q;
                bc.c[t][q] = 0.05f * t - q;
            }
        }
        hipLaunchKernelGGL(update_kernel, dim3(blocks), dim3(kThreads), 0, st, bc, iters, sink);
        *wave_instr = waves * (uint64_t)iters * kUpdSteps * kUpdStates; // wave-element updates
        break;
    }
    default:
        return MAMBA_ERR_UNSUPPORTED;
    }
    return hipGetLastError() == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

} // extern "C"
