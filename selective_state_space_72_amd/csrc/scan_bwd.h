// Internal declarations of the backward pass (scan_bwd.hip), shared with the C ABI.
// Not part of the public ABI (see include/mamba_scan.h).
#pragma once

#include "scan_common.h"

namespace mambascan {

// Backward pass (Euler discretisation).  Optional outputs are NULL when not wanted.
struct BwdLaunch {
    const void *u, *delta, *z, *dy, *B, *C;
    const float *A, *D, *bias, *h0, *dh_last;
    void *du, *ddelta, *dz, *dB, *dC; // activation dtype
    float *dA, *dD, *dbias, *dh0;
    float *ckpt;        // [block][segment][n][lane]
    bool ck_ext;        // ckpt written by the forward pass: no forward pass here
    float *dbc_part;    // [block][t][2N]
    float *dA_part;     // [span][b][d][n]
    float *dDb_part;    // [span][b][d][2]
    // sequence split (n_spans > 1): spans of span_len steps (a multiple of the segment
    // length); h_in = state entering each span (the forward carry pass), mu_dec / mu_loc
    // the adjoint span summaries and mu_in the adjoint entering each span from its end,
    // all [span][b][d][n]
    int32_t n_spans;
    int64_t span_len;
    const float *h_in;
    float *mu_dec, *mu_loc, *mu_in;
    int64_t batch, L, d_inner, d_state;
    DType dtype;
    bool zoh; // zero-order-hold input term (else Euler); not with ck_ext
};

// (waves, segment length) of the compiled backward variant for d_state; false if none.
bool bwd_variant(int64_t d_state, int *waves, int *seg_len);
hipError_t launch_scan_bwd(const BwdLaunch &p, hipStream_t stream);

} // namespace mambascan
