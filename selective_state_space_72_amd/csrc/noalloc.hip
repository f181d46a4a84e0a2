// mamba_scan_fwd without a caller workspace and without any allocation: the workspace the
// forward scan needs (staged B/C, relay flags and states, span summaries) lives in one
// file-scope device array, `scratch`, of kScratchBytes per device.  Its device address is
// looked up once per device (hipGetSymbolAddress, with that device current) and kept; host
// code never hands the array's own name to a kernel, only that address.  Every call on a
// device shares the array: calls that overlap on one device race (the caller serialises
// them, e.g. by using one stream).
#include "mamba_scan.h"

#include <hip/hip_runtime.h>

#include <mutex>
#include <stdint.h>

// Argument checks of mamba_scan_fwd short of the workspace (mamba_api.hip; not exported).
mamba_status_t mamba_scan_fwd_check(const void *u, const void *delta, const float *A,
                                    const void *B, const void *C, const float *D, const void *z,
                                    const float *delta_bias, const float *h0, void *y,
                                    float *h_last, int64_t batch, int64_t seqlen,
                                    int64_t d_inner, int64_t d_state, mamba_dtype_t dtype);

namespace {

constexpr size_t kScratchBytes = MAMBA_SCAN_NOALLOC_MAX_WORKSPACE; // per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on `dev` (looked up once, with dev current); NULL on failure.
void *scratch_on(int dev)
{
    if (dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev])
        return g_scratch_ptr[dev];
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess)
        return nullptr;
    if (prev != dev && hipSetDevice(dev) != hipSuccess)
        return nullptr;
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (prev != dev)
        (void)hipSetDevice(prev);
    if (e != hipSuccess || !ptr) {
        (void)hipGetLastError(); // leave no sticky error behind
        return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
    return ptr;
}

} // namespace

extern "C" {

mamba_status_t mamba_scan_fwd_noalloc(const void *u, const void *delta, const float *A,
                                      const void *B, const void *C, const float *D,
                                      const void *z, const float *delta_bias, const float *h0,
                                      void *y, float *h_last, int64_t batch, int64_t seqlen,
                                      int64_t d_inner, int64_t d_state, mamba_dtype_t dtype,
                                      void *stream)
{
    // every check first, before anything touches the device
    const mamba_status_t chk = mamba_scan_fwd_check(u, delta, A, B, C, D, z, delta_bias, h0, y,
                                                    h_last, batch, seqlen, d_inner, d_state,
                                                    dtype);
    if (chk != MAMBA_OK)
        return chk;
    const size_t need = mamba_scan_fwd_workspace_size(batch, seqlen, d_inner, d_state);
    if (need == (size_t)-1)
        return MAMBA_ERR_BAD_SHAPE;
    if (need > kScratchBytes)
        return MAMBA_ERR_WORKSPACE;
    void *ws = nullptr;
    if (need > 0) {
        int dev = -1;
        hipStream_t st = reinterpret_cast<hipStream_t>(stream);
        if (hipStreamGetDevice(st, &dev) != hipSuccess) {
            (void)hipGetLastError();
            return MAMBA_ERR_HIP;
        }
        ws = scratch_on(dev);
        if (!ws)
            return MAMBA_ERR_HIP;
    }
    return mamba_scan_fwd(u, delta, A, B, C, D, z, delta_bias, h0, y, h_last, batch, seqlen,
                          d_inner, d_state, dtype, ws, need > 0 ? kScratchBytes : 0, stream);
}

} // extern "C"
