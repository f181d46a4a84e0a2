// Internal declarations shared by the HIP translation units of libmambascan.
// Not part of the public ABI (see include/mamba_scan.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mambascan {

enum class DType : int { F32 = 0, BF16 = 1 };

// One launch of the chunked scan kernel.  h_init points at the initial state of
// span 0 (h0) or at the per-span carry-in states written by the carry pass.
struct ScanLaunch {
    const void *u, *delta, *z, *B, *C;
    const float *A, *D, *bias;
    const float *h_init;        // nullable: zero initial state
    int64_t h_init_span_stride; // floats between consecutive spans' states (0: span 0 only)
    void *y;                    // FULL mode output
    float *h_last;              // FULL mode final state (nullable)
    float *ws_decay, *ws_hloc;  // END mode outputs, layout [(b*D + d)*N + n][span]
    float *ws_rot;              // END mode with the rotation: each state pair's transition
                                // over the span, 2x2 [(pair)][span][m00, m10, m01, m11]
    int64_t batch, L, d_inner, d_state;
    int64_t span_len;
    int32_t n_spans;
    int32_t first_span;         // spans [first_span, first_span + launch_spans) are launched
    int32_t launch_spans;
    int32_t waves, chunk;
    DType dtype;
    float *bc_staged;           // scalar family: B/C repacked as fp32 [b][wave][row][2 NQ]
    int64_t staged_rows;        // rows per (b, wave) in bc_staged (L plus one chunk of padding)
    // Relay (scalar family, single span): the last `relay_tiles` (batch row, channel tile)
    // units are split in time into `relay_parts` parts of `relay_len` steps run by different
    // blocks, each part handing its final state to the next through relay_state.
    // relay_sync[slot] are the hand-off flags and relay_sync[slots] counts waits that gave
    // up; the staging pass of the same call zeroes them.  relay_withhold (testing): part 0
    // of every relayed unit keeps its state, so the waits give up after relay_max_polls.
    uint32_t *relay_sync;
    float *relay_state;         // [slot][n][lane], slot = tile * (parts - 1) + part
    int32_t relay_tiles, relay_parts;
    int64_t relay_len;
    uint32_t relay_max_polls;
    bool relay_withhold;
    bool zoh; // zero-order-hold Bbar (scalar family); Euler otherwise
    // Options of the Mamba-3 formulation (scalar family; NULL / false = off):
    // exponential-trapezoidal input term with mixing coefficients lam (B,L,D) and the input
    // before t = 0 in u_prev (B,D), B_prev (B,N); rotation of state pairs by Delta * theta,
    // theta (B,L,N/2) staged next to B and C.
    bool trap, rot;
    const void *lam, *u_prev, *B_prev, *theta;
    // Checkpoints for the backward pass (scalar family, Euler, full-output pass; NULL = off):
    // the state entering every 8-step segment s >= 1, at ckpt[((unit * n_seg + s) * N + n)
    // * 64 + lane], unit = channel tile * batch + b, n_seg = ceil(L / 8).
    float *ckpt;
    // Row strides in elements: (b, t) rows of u, delta, z start su, sd, sz elements apart,
    // those of B and C sB, sC apart (d_inner, d_state when contiguous; the scalar family
    // reads other strides, the other families need the contiguous ones).
    int64_t su, sd, sz, sB, sC;
};

// Relay arguments as the scan kernel receives them.
struct RelayArgs {
    uint32_t *sync;
    uint32_t *fault;             // count of waits that gave up (after the flags)
    float *state;
    int32_t tiles, parts, units; // units = batch * channel tiles
    int32_t len;
    uint32_t max_polls;
    int32_t withhold;            // testing: part 0 does not hand its state over
};

enum class Family : int { Auto = 0, Block = 1, Rows = 2, Scalar = 3 };

// The carry pass joining span end states: for every state column c = (b, d, n)
// h_in[s][c] = state entering span s (s = 0 .. n_spans-1).
struct CarryLaunch {
    const float *ws_decay, *ws_hloc; // [c][span], spans 0 .. n_spans-2 used
    const float *ws_rot;             // non-null: the spans' 2x2 pair transitions replace decay
    const float *h0;                 // nullable
    float *h_in;                     // [span][c]
    int64_t columns;
    int32_t n_spans;
};

// Causal depthwise conv1d + SiLU: prefill (x -> u, state_in -> state_out) or one
// decode token (state_out is the in/out state).
struct ConvLaunch {
    const void *x;
    const float *w, *bias;
    const void *state_in;
    void *u, *state_out;
    int64_t batch, L, d_inner, d_conv;
    DType dtype;
    bool vec4; // 4 channels per lane (d_inner % 4 == 0, x and u 4-element aligned)
};

struct StepLaunch {
    float *h;
    const void *u, *delta, *z, *B, *C;
    const float *A, *D, *bias;
    void *y;
    int64_t batch, d_inner, d_state;
    DType dtype;
    bool zoh;
    bool trap, rot;                          // as in ScanLaunch
    const void *lam, *u_prev, *B_prev;       // (B,D), (B,D), (B,N)
    const void *theta;                       // (B,N/2)
    int64_t su, sd, sz, sB, sC;              // batch-row strides (elements) of u, delta, z, B, C
};

// Returns true if the (d_state, waves, chunk) combination is compiled in.
bool scan_variant_supported(int64_t d_state, int waves, int chunk);
int default_waves(int64_t d_state);
int default_chunk(int64_t d_state, int waves);

// LDS-exchange kernel: 64 channels per block, state indices split across its waves.
hipError_t launch_scan_full(const ScanLaunch &p, hipStream_t stream);
hipError_t launch_scan_end(const ScanLaunch &p, hipStream_t stream);
// Barrier-free kernel: 16 channels per wave, state indices split across its DPP rows.
hipError_t launch_rows_full(const ScanLaunch &p, hipStream_t stream);
hipError_t launch_rows_end(const ScanLaunch &p, hipStream_t stream);
// Scalar kernel: as the LDS-exchange kernel, with B/C staged as fp32 and read into SGPRs.
bool scalar_variant_supported(int64_t d_state, int waves, int chunk);
hipError_t launch_stage_bc(const ScanLaunch &p, hipStream_t stream);
hipError_t launch_scalar_full(const ScanLaunch &p, hipStream_t stream);
hipError_t launch_scalar_end(const ScanLaunch &p, hipStream_t stream);
hipError_t launch_carry(const CarryLaunch &p, hipStream_t stream);
hipError_t launch_state_update(const StepLaunch &p, hipStream_t stream);
hipError_t launch_conv1d_silu(const ConvLaunch &p, hipStream_t stream);
hipError_t launch_conv1d_silu_update(const ConvLaunch &p, hipStream_t stream);
// h_last = h0 (or zeros when h0 is NULL), for empty sequences.
hipError_t launch_copy_state(float *dst, const float *src, int64_t count, hipStream_t stream);
// Rows of n elements (2 or 4 bytes) to rows of np >= n, the extra entries `fill` (zero for
// 2-byte elements), and back (pad.hip: d_state values run at the next compiled size).
hipError_t launch_pad_rows(void *dst, const void *src, int64_t rows, int32_t n, int32_t np,
                           int32_t elem_bytes, float fill, hipStream_t stream,
                           int64_t src_stride = 0 /* elements between source rows; 0 = n */);
hipError_t launch_unpad_rows(void *dst, const void *src, int64_t rows, int32_t n, int32_t np,
                             int32_t elem_bytes, hipStream_t stream);

} // namespace mambascan
