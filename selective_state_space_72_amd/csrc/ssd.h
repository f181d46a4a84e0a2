// Internal declarations of the Mamba-2 SSD scan (ssd.hip), shared with the C ABI.
// Not part of the public ABI (see include/mamba_scan.h).
#pragma once

#include "scan_common.h"

namespace mambascan {

struct SsdLaunch {
    const void *x, *dt, *B, *C, *z; // activation dtype; z nullable
    const float *A, *D, *dt_bias;   // (n_heads); D, dt_bias nullable
    const float *h0;                // (batch, n_heads * head_dim, d_state), nullable
    void *y;
    float *h_last;                  // nullable
    int64_t batch, L, n_heads, head_dim, d_state;
    DType dtype;
};

// True if (head_dim, d_state) is compiled in.
bool ssd_supported(int64_t head_dim, int64_t d_state);
hipError_t launch_ssd(const SsdLaunch &p, hipStream_t stream);

} // namespace mambascan
