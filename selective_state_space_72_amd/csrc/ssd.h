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
    // Relay: the last relay_units (batch row, head) units run as two blocks each, the
    // second continuing from step relay_mid (a multiple of the chunk) with the first's
    // final state, handed over through relay_state (head_dim x d_state fp32 per unit) and
    // relay_sync (one flag per unit).  relay_units = 0: no relay.
    // relay_sync[relay_units] counts waits that gave up; relay_withhold (testing): the first
    // parts keep their states, so the waits give up.
    int64_t relay_units, relay_mid;
    uint32_t *relay_sync;
    float *relay_state;
    bool relay_withhold;
    // Sequence split (no relay then): n_spans spans of span_len steps (a multiple of the
    // chunk), the spans after the first starting from the state the carry gives them;
    // span_state (n_spans - 1) x units x head_dim x d_state fp32, span_decay (n_spans - 1) x
    // units fp32.  n_spans <= 1: no split.
    int64_t n_spans, span_len;
    float *span_state, *span_decay;
};

// One decode token of the SSD (ssd_step.hip).
struct SsdStepLaunch {
    float *h;                       // (batch, n_heads * head_dim, d_state) fp32, in place
    const void *x, *dt, *B, *C, *z; // (batch, H*P), (batch, H), (batch, N) x2, (batch, H*P)
    const float *A, *D, *dt_bias;   // (n_heads); D, dt_bias nullable
    void *y;                        // (batch, n_heads * head_dim)
    int64_t batch, n_heads, head_dim, d_state;
    DType dtype;
};

// True if (head_dim, d_state) is compiled in.
bool ssd_supported(int64_t head_dim, int64_t d_state);
hipError_t launch_ssd_step(const SsdStepLaunch &p, hipStream_t stream);
// Blocks of the SSD kernel for (d_state, dtype) that the current device runs at once
// (blocks per compute unit x compute units); 0 if unknown.
int64_t ssd_block_slots(int64_t d_state, DType dtype);
hipError_t launch_ssd(const SsdLaunch &p, hipStream_t stream);

} // namespace mambascan
