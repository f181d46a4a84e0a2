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

// Backward of the scan with the Mamba-3 options (trapezoid lam/u_prev/B_prev, rotation
// theta; the zero-order hold with the rotation): scan_bwd_m3.hip.  Workspace regions from
// m3_bwd_workspace_bytes (offsets off[0..4], total off[5]): stored states, dB/dC/dtheta
// tile partials, dB_prev tile partials, dA and dD/dbias per batch row.
struct M3BwdLaunch {
    const void *u, *delta, *z, *dy, *B, *C, *lam, *u_prev, *B_prev, *theta;
    const float *A, *D, *bias, *h0, *dh_last;
    void *du, *ddelta, *dz, *dB, *dC, *dlam, *du_prev, *dB_prev, *dtheta; // activation dtype
    float *dA, *dD, *dbias, *dh0;
    float *ckpt, *part, *bprev_part, *dA_part, *dDb_part; // workspace
    int64_t batch, L, d_inner, d_state;
    DType dtype;
    bool zoh;
};
size_t m3_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state,
                              bool rot, size_t off[6]);
hipError_t launch_scan_bwd_m3(const M3BwdLaunch &p, hipStream_t stream);

// (waves, segment length) of the compiled backward variant for d_state; false if none.
bool bwd_variant(int64_t d_state, int *waves, int *seg_len);
hipError_t launch_scan_bwd(const BwdLaunch &p, hipStream_t stream);

} // namespace mambascan
