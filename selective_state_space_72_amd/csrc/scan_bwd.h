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
// theta; the zero-order hold with the rotation): scan_bwd_m3.hip.  With a sequence split
// (n_spans > 1) the forward span pass and carry (scan_scalar.hip, scan_kernels.hip) give the
// state entering each span and the span transitions; the adjoint span pass and carry here give
// the adjoint entering each span from its end.  Workspace regions from m3_bwd_workspace_bytes
// (offsets off[0..13], total off[14]; every region 256-byte aligned):
//   0 stored states [block][segment][n][64 lanes]       1 dB/dC/dtheta tile partials [unit][t][V]
//   2 look-back dB shares [span][unit][N]               3 dA [span][b][d][n]
//   4 dD, dbias [span][b][d][2]
//   with spans: 5 staged B/C (theta) of the forward span pass, 6 span decays [c][span],
//   7 span local end states [c][span], 8 state entering each span [span][c], 9 pair
//   transitions [pair][span][4] (rotation), 10 adjoint span local [span][c], 11 adjoint
//   entering each span [span][c], 12 du of a span's last step [span][b][d], 13 the next
//   span's look-back share of that du [span][b][d]   (c = (b, d, n))
struct M3Plan {
    int n_spans;
    int64_t span_len;         // a multiple of the 8-step segment (and of fwd_chunk)
    int fwd_waves, fwd_chunk; // the forward span pass (scalar family)
};
struct M3BwdLaunch {
    const void *u, *delta, *z, *dy, *B, *C, *lam, *u_prev, *B_prev, *theta;
    const float *A, *D, *bias, *h0, *dh_last;
    void *du, *ddelta, *dz, *dB, *dC, *dlam, *du_prev, *dB_prev, *dtheta; // activation dtype
    float *dA, *dD, *dbias, *dh0;
    float *ckpt, *part, *bprev_part, *dA_part, *dDb_part; // workspace
    // sequence split: regions 6 .. 13 above (NULL with one span)
    const float *ws_decay, *ws_rot, *h_in;
    float *mu_loc, *mu_in, *du_edge, *du_lb;
    int32_t n_spans;
    int64_t span_len;
    int64_t batch, L, d_inner, d_state;
    DType dtype;
    bool zoh;
};
size_t m3_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t d_inner, int64_t d_state,
                              bool rot, const M3Plan &plan, size_t off[15]);
hipError_t launch_scan_bwd_m3(const M3BwdLaunch &p, hipStream_t stream);

// (waves, segment length) of the compiled backward variant for d_state; false if none.
bool bwd_variant(int64_t d_state, int *waves, int *seg_len);
hipError_t launch_scan_bwd(const BwdLaunch &p, hipStream_t stream);

} // namespace mambascan
