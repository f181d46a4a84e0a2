// Padding of the state index for d_state values the scan kernels are not compiled for.
//
// The kernels are built for d_state 4, 8, 16, 32 and 64.  Another d_state n in 1..64 runs
// at the next compiled size np: the arrays indexed by the state (A, B, C, h0 and the
// Mamba-3 theta and B_prev) are copied with rows of np entries, the extra entries of B, C,
// h0, theta and B_prev zero and those of A -1.  The extra states then start at zero and
// receive zero input, so they stay exactly zero and add exactly zero to every readout: the
// first n states follow the same recurrence as without them.  Results indexed by the state
// (h_last, and the gradients dB, dC, dA, dh0 of the backward pass) are copied back to rows
// of n entries.
#include "scan_common.h"

namespace mambascan {
namespace {

// dst[r * np + c] = src[r * ss + c] for c < n, else fill (per element of dst)
template <typename E>
__global__ void __launch_bounds__(256)
pad_rows_kernel(E *__restrict__ dst, const E *__restrict__ src, int64_t rows, int32_t n,
                int32_t np, int64_t ss, E fill)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= rows * np)
        return;
    const int64_t r = i / np;
    const int32_t c = (int32_t)(i - r * np);
    dst[i] = c < n ? src[r * ss + c] : fill;
}

// dst[r * n + c] = src[r * np + c] (per element of dst)
template <typename E>
__global__ void __launch_bounds__(256)
unpad_rows_kernel(E *__restrict__ dst, const E *__restrict__ src, int64_t rows, int32_t n,
                  int32_t np)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= rows * n)
        return;
    const int64_t r = i / n;
    const int32_t c = (int32_t)(i - r * n);
    dst[i] = src[r * np + c];
}

uint32_t grid_for(int64_t count) { return (uint32_t)((count + 255) / 256); }

} // namespace

hipError_t launch_pad_rows(void *dst, const void *src, int64_t rows, int32_t n, int32_t np,
                           int32_t elem_bytes, float fill, hipStream_t stream, int64_t src_stride)
{
    if (rows <= 0)
        return hipSuccess;
    const int64_t count = rows * np;
    const int64_t ss = src_stride > 0 ? src_stride : n;
    if (elem_bytes == 4)
        hipLaunchKernelGGL(pad_rows_kernel<float>, dim3(grid_for(count)), dim3(256), 0, stream,
                           static_cast<float *>(dst), static_cast<const float *>(src), rows, n,
                           np, ss, fill);
    else // 16-bit elements: the fill is zero
        hipLaunchKernelGGL(pad_rows_kernel<uint16_t>, dim3(grid_for(count)), dim3(256), 0,
                           stream, static_cast<uint16_t *>(dst),
                           static_cast<const uint16_t *>(src), rows, n, np, ss, (uint16_t)0);
    return hipGetLastError();
}

hipError_t launch_unpad_rows(void *dst, const void *src, int64_t rows, int32_t n, int32_t np,
                             int32_t elem_bytes, hipStream_t stream)
{
    if (rows <= 0)
        return hipSuccess;
    const int64_t count = rows * n;
    if (elem_bytes == 4)
        hipLaunchKernelGGL(unpad_rows_kernel<float>, dim3(grid_for(count)), dim3(256), 0,
                           stream, static_cast<float *>(dst), static_cast<const float *>(src),
                           rows, n, np);
    else
        hipLaunchKernelGGL(unpad_rows_kernel<uint16_t>, dim3(grid_for(count)), dim3(256), 0,
                           stream, static_cast<uint16_t *>(dst),
                           static_cast<const uint16_t *>(src), rows, n, np);
    return hipGetLastError();
}

} // namespace mambascan
