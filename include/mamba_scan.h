/*
 * mamba_scan.h -- C ABI of libmambascan.so, the Mamba selective scan on AMD
 * Instinct MI355X (gfx950).
 *
 * Operation (selective scan).  For every batch row b, channel d and state index
 * n, sequentially over t = 0..L-1:
 *
 *   Delta_t   = softplus(delta[b,t,d] + delta_bias[d])
 *   h_t[n]    = exp(Delta_t * A[d,n]) * h_{t-1}[n] + Delta_t * B[b,t,n] * u[b,t,d]
 *   y[b,t,d]  = (sum_n C[b,t,n] * h_t[n] + D[d] * u[b,t,d]) * silu(z[b,t,d])
 *
 * with h_{-1} = h0[b,d,:] and h_last[b,d,:] = h_{L-1}.  This is the selective
 * state-space recurrence with input-dependent B, C and step size of
 * "Understanding Mamba" (aiattnstudio.link, sections 2.3, 4.4 and 5.2: the
 * selective_scan / _selective_scan functions and MambaBlock.forward's
 * y * silu(z) gate), in the readout form of "State Space Models and Mamba"
 * (metaphor-xennon.pages.dev, selective_scan: einsum 'bdn,bn->bd') with the
 * skip term y = C x + D u of "Understanding Mamba" section 12 and the bias
 * inside the softplus (metaphor-xennon, MambaBlock.forward).  The input term
 * is the Euler form Delta*B that all of the pages' code uses.
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers (HIP device memory visible to the stream's
 *     device).  The caller owns every buffer; the library never allocates,
 *     frees or retains memory, and keeps no state between calls.
 *   - dtype applies to u, delta, z, B, C and y (F32: float; BF16: bfloat16
 *     stored as 16-bit words).  A, D, delta_bias and all states (h0, h_last,
 *     h) are always float32.  Internal arithmetic is float32; y is rounded to
 *     dtype with round-to-nearest-even.
 *   - Layouts are dense, row-major, last index fastest:
 *       u, delta, z, y : (batch, seqlen, d_inner)       [decode: (batch, d_inner)]
 *       B, C           : (batch, seqlen, d_state)       [decode: (batch, d_state)]
 *       A              : (d_inner, d_state)
 *       D, delta_bias  : (d_inner)
 *       h0, h_last, h  : (batch, d_inner, d_state)
 *   - Optional pointers (documented as nullable) mean: D NULL -> 0,
 *     delta_bias NULL -> 0, z NULL -> no gate, h0 NULL -> zero initial state,
 *     h_last NULL -> final state not returned.
 *   - Pointers must be aligned to their element size (4 bytes for float, 2 for
 *     bf16); otherwise MAMBA_ERR_MISALIGNED.
 *   - All argument checks happen on the host before anything is launched; a
 *     failing call has no effect.  A successful call only means the work was
 *     enqueued on `stream` (a hipStream_t; NULL selects the null stream).  The
 *     call is asynchronous: device faults surface at the caller's next
 *     synchronisation.  MAMBA_ERR_HIP reports a failed launch.
 *   - Entry points are reentrant and thread-safe.  Results are bitwise
 *     deterministic for given inputs and options (no atomics).
 *   - NaN and Inf inputs propagate as IEEE arithmetic does; they are not
 *     checked.  Denormal intermediates may be flushed to zero.
 */
#ifndef MAMBA_SCAN_H
#define MAMBA_SCAN_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define MAMBA_API __attribute__((visibility("default")))
#else
#define MAMBA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MAMBA_DTYPE_F32 = 0,
    MAMBA_DTYPE_BF16 = 1
} mamba_dtype_t;

typedef enum {
    MAMBA_OK = 0,
    MAMBA_ERR_NULL_ARG = 1,     /* a required pointer is NULL                       */
    MAMBA_ERR_BAD_SHAPE = 2,    /* negative size, or sizes whose products overflow  */
    MAMBA_ERR_BAD_DTYPE = 3,    /* dtype is not a mamba_dtype_t value               */
    MAMBA_ERR_UNSUPPORTED = 4,  /* d_state out of range, or an unsupported option    */
    MAMBA_ERR_MISALIGNED = 5,   /* a pointer is not aligned to its element size     */
    MAMBA_ERR_ALIASING = 6,     /* an output overlaps an input or another output    */
    MAMBA_ERR_WORKSPACE = 7,    /* workspace missing or smaller than required       */
    MAMBA_ERR_HIP = 8           /* a HIP runtime call or kernel launch failed       */
} mamba_status_t;

/* Largest d_state of the selective scan.  The kernels are compiled for d_state 4, 8, 16,
 * 32 and 64; any other d_state from 1 to 64 runs at the next of those sizes: the arrays
 * indexed by the state index (A, B, C, h0 and the Mamba-3 theta, B_prev) are copied into the
 * workspace as rows of the larger size, the extra entries of A -1 and all others 0, so the
 * extra states start at zero, receive zero input, stay exactly zero and add exactly zero
 * to every readout; results indexed by the state (h_last, dB, dC, dA, dh0) are copied back
 * to rows of the caller's size.  Those calls need the workspace the size queries report
 * (larger than at the compiled size) and cost what the compiled size costs, plus the
 * copies.  The decode step needs no workspace: it runs the state indices of such a size
 * in the lanes of the next compiled size. */
#define MAMBA_MAX_D_STATE 64

/* Kernel families (mamba_scan_opts_t.kernel). */
#define MAMBA_KERNEL_AUTO 0
#define MAMBA_KERNEL_BLOCK 1 /* 64 channels per block; state indices split across its
                                waves, which exchange through LDS with barriers      */
#define MAMBA_KERNEL_ROWS 2  /* 16 channels per wave; state indices split across the
                                wave's four 16-lane rows; no barriers                */
#define MAMBA_KERNEL_SCALAR 3 /* as BLOCK, with B/C repacked to fp32 by a staging pass
                                 and read by each wave through scalar registers      */

/* Tuning and testing options for mamba_scan_fwd_ex.  Zero fields mean "auto".
 *   chunk_len : BLOCK/SCALAR kernels: time steps per iteration (4 to 32).
 *   waves     : BLOCK/SCALAR kernels: wavefronts per block (4 or 8); each
 *               handles d_state/waves state indices of 64 channels.
 *   n_spans   : the sequence is split into n_spans spans scanned in parallel
 *               and joined by a carry pass (1..64; 1 = no split).
 *   kernel    : MAMBA_KERNEL_* family.  AUTO picks SCALAR when the grid fills the
 *               device and d_state <= 32, else ROWS; with chunk_len or waves set,
 *               AUTO picks SCALAR if it has that shape, else BLOCK.  SCALAR needs
 *               span length x d_inner x 4 < 2^31 (it raises an automatic span count
 *               to get there; a fixed n_spans that misses it is unsupported).
 *   relay     : SCALAR kernel, single span: the (batch row, 64-channel tile)
 *               units left over after filling every compute unit equally are
 *               split in time into parts run by different blocks, each part
 *               handing its final state to the next (no recomputation).
 *               0 = auto (two parts, when it evens out the load), 1 = off,
 *               2..8 = that many equal parts (when no units are left over, every
 *               unit is split; for testing), -8..-2 = the same, with the first part
 *               of every relayed unit withholding its hand-off (failure test: the
 *               next part's bounded wait gives up; see mamba_scan_fwd_relay_faults).
 *               A wait for a hand-off is bounded (about 2^20 polls of ~8k cycles,
 *               2^10 in the failure test); one that gives up is counted in the
 *               workspace and the part continues from a NaN state, so its outputs
 *               and the unit's final state are NaN, never silently wrong.
 *   discretization : MAMBA_DISC_EULER (0, default) or MAMBA_DISC_ZOH; the zero-
 *               order hold needs the SCALAR family (AUTO selects it).
 * Every supported setting of the other fields gives the same result up to
 * float32 rounding; an unsupported one makes the call return
 * MAMBA_ERR_UNSUPPORTED. */
typedef struct {
    int32_t chunk_len;
    int32_t waves;
    int32_t n_spans;
    int32_t kernel;
    int32_t relay;
    int32_t discretization;
} mamba_scan_opts_t;

/* Discretisation of the input matrix (mamba_scan_opts_t.discretization and
 * mamba_state_update_ex):
 *   EULER: Bbar = Delta * B, as all of the pages' selective_scan code does;
 *   ZOH:   Bbar = A^-1 (exp(Delta A) - I) B = (exp(Delta A[d,n]) - 1) / A[d,n] * B[n],
 *          the zero-order hold of "Understanding Mamba" section 12 and of "State
 *          Space Models and Mamba" (ZOH); Delta * B where A[d,n] = 0 (the limit).
 * Abar = exp(Delta A) in both. */
#define MAMBA_DISC_EULER 0
#define MAMBA_DISC_ZOH 1

/* Returns 1 if the selective scan and its decode step take this d_state (1..64), else 0.
 * (The backward pass takes 1..32; the SSD has its own sizes, mamba_ssd_supported.) */
MAMBA_API int32_t mamba_d_state_supported(int64_t d_state);

/*
 * Number of bytes of device workspace mamba_scan_fwd needs for these sizes
 * (auto options) -- 0 means no workspace is needed and NULL may be passed.
 * Depends on the current device's compute-unit count.  Returns (size_t)-1
 * for invalid sizes.
 */
MAMBA_API size_t mamba_scan_fwd_workspace_size(int64_t batch, int64_t seqlen, int64_t d_inner,
                                     int64_t d_state);

/* The same for explicit options (opts may be NULL for auto). */
MAMBA_API size_t mamba_scan_fwd_workspace_size_ex(int64_t batch, int64_t seqlen, int64_t d_inner,
                                        int64_t d_state, const mamba_scan_opts_t *opts);

/*
 * Selective scan forward (the operation above) over a whole sequence.
 *
 *   u, delta   (batch, seqlen, d_inner) dtype        required
 *   A          (d_inner, d_state) float32            required (normally A < 0)
 *   B, C       (batch, seqlen, d_state) dtype        required
 *   D          (d_inner) float32                     nullable
 *   z          (batch, seqlen, d_inner) dtype        nullable (gate)
 *   delta_bias (d_inner) float32                     nullable
 *   h0         (batch, d_inner, d_state) float32     nullable
 *   y          (batch, seqlen, d_inner) dtype        output, required if seqlen > 0
 *   h_last     (batch, d_inner, d_state) float32     output, nullable
 *   workspace  device memory of workspace_bytes      see mamba_scan_fwd_workspace_size
 *
 * Sizes: batch, seqlen, d_inner >= 0; d_state must be supported (see
 * mamba_d_state_supported).  With seqlen == 0 only h_last is written (h0, or
 * zeros); u, delta, B, C, z and y may then be NULL.  With batch == 0 or
 * d_inner == 0 nothing is done.
 * Aliasing: y must not overlap any other argument.  h_last may be exactly h0
 * (in-place continuation of a state) but must not otherwise overlap anything.
 * The workspace must not overlap any argument.
 */
MAMBA_API mamba_status_t mamba_scan_fwd(const void *u, const void *delta, const float *A, const void *B,
                              const void *C, const float *D, const void *z,
                              const float *delta_bias, const float *h0, void *y, float *h_last,
                              int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                              mamba_dtype_t dtype, void *workspace, size_t workspace_bytes,
                              void *stream);

/* mamba_scan_fwd with explicit tuning options (opts NULL = auto).  Used by the
 * tests to check that the result does not depend on the internal split. */
MAMBA_API mamba_status_t mamba_scan_fwd_ex(const void *u, const void *delta, const float *A,
                                 const void *B, const void *C, const float *D, const void *z,
                                 const float *delta_bias, const float *h0, void *y,
                                 float *h_last, int64_t batch, int64_t seqlen, int64_t d_inner,
                                 int64_t d_state, mamba_dtype_t dtype, void *workspace,
                                 size_t workspace_bytes, const mamba_scan_opts_t *opts,
                                 void *stream);

/*
 * One recurrent decode step (a single token) on a persistent state: the loop
 * body of the operation above with seqlen = 1 and h read and written in place,
 * as in the token-by-token decoder "output, h = ssm(token, h)" of "State Space
 * Models and Mamba" (metaphor-xennon.pages.dev, MambaDecoder), whose memory is
 * the constant-size state.
 *
 *   h          (batch, d_inner, d_state) float32     in/out, required
 *   u, delta   (batch, d_inner) dtype                required
 *   A          (d_inner, d_state) float32            required
 *   B, C       (batch, d_state) dtype                required
 *   D          (d_inner) float32                     nullable
 *   z          (batch, d_inner) dtype                nullable (gate)
 *   delta_bias (d_inner) float32                     nullable
 *   y          (batch, d_inner) dtype                output, required
 *
 * Alignment: for d_state 4, 8, 16, 32 and 64, h and A must be 16-byte aligned (each
 * lane moves 4 state values at once); for other sizes 4-byte aligned.  The other
 * pointers as for every entry point.
 * Aliasing: y and h must not overlap each other or any input.
 */
MAMBA_API mamba_status_t mamba_state_update(float *h, const void *u, const void *delta, const float *A,
                                  const void *B, const void *C, const float *D, const void *z,
                                  const float *delta_bias, void *y, int64_t batch,
                                  int64_t d_inner, int64_t d_state, mamba_dtype_t dtype,
                                  void *stream);

/* ------------------------------------------------------------------------
 * Causal depthwise convolution + SiLU: the Mamba block's conv1d, which produces
 * the scan's input u from the inner activations x.  "Understanding Mamba"
 * (aiattnstudio.link), sections 3.2 and 5.2: a depthwise nn.Conv1d (one filter
 * per channel) with kernel d_conv = K, padding K - 1 and a bias, of which the
 * first seqlen outputs are kept, followed by F.silu; the same block in "State
 * Space Models and Mamba" (metaphor-xennon.pages.dev), MambaBlock.forward.
 * (The scan's Delta, B and C are projections of this output, so it runs before
 * the scan as its own pass.)
 *
 *   u[b,t,d] = silu(conv_bias[d] + sum_{k<K} w[d,k] * xe[b, t-(K-1)+k, d])
 *
 * xe[b,s,d] = x[b,s,d] for s >= 0; for -(K-1) <= s < 0 it is the carried state
 * state_in[b,d,(K-1)+s] -- the previous segment's last K-1 inputs, oldest
 * first -- or 0 when state_in is NULL (the zero padding of nn.Conv1d).  On
 * return state_out[b,d,j] = xe[b, seqlen-(K-1)+j, d], j < K-1, the state a
 * following segment or decode step needs.
 *
 *   x, u                (batch, seqlen, d_inner) dtype   required (unless empty)
 *   w                   (d_inner, d_conv) float32        required
 *   conv_bias           (d_inner) float32                nullable (0)
 *   state_in, state_out (batch, d_inner, d_conv-1) dtype nullable
 *
 * d_conv must be 2, 3 or 4 (else MAMBA_ERR_UNSUPPORTED).  state_in == state_out
 * is allowed (in-place continuation); u must not overlap x, w or the states, and
 * state_out must not overlap x (MAMBA_ERR_ALIASING).  Pointers must be aligned to
 * their element size.  Other conventions as above.
 */
MAMBA_API mamba_status_t mamba_conv1d_silu_fwd(const void *x, const float *w,
                                               const float *conv_bias, const void *state_in,
                                               void *u, void *state_out, int64_t batch,
                                               int64_t seqlen, int64_t d_inner, int64_t d_conv,
                                               mamba_dtype_t dtype, void *stream);

/* One decode token of the convolution:
 *   u[b,d] = silu(conv_bias[d] + sum_{k<K-1} w[d,k] state[b,d,k] + w[d,K-1] x[b,d])
 *   state[b,d,:] <- (state[b,d,1:], x[b,d])
 *
 *   state      (batch, d_inner, d_conv-1) dtype     in/out, required
 *   x, u       (batch, d_inner) dtype               required
 *   w          (d_inner, d_conv) float32            required
 *   conv_bias  (d_inner) float32                    nullable
 *
 * d_conv 2..4.  u must not overlap state, x or w; state must not overlap x or w.
 */
MAMBA_API mamba_status_t mamba_conv1d_silu_update(void *state, const void *x, const float *w,
                                                  const float *conv_bias, void *u,
                                                  int64_t batch, int64_t d_inner, int64_t d_conv,
                                                  mamba_dtype_t dtype, void *stream);

/* mamba_state_update with a choice of discretisation (MAMBA_DISC_*); anything
 * else returns MAMBA_ERR_UNSUPPORTED. */
MAMBA_API mamba_status_t mamba_state_update_ex(float *h, const void *u, const void *delta,
                                               const float *A, const void *B, const void *C,
                                               const float *D, const void *z,
                                               const float *delta_bias, void *y, int64_t batch,
                                               int64_t d_inner, int64_t d_state,
                                               mamba_dtype_t dtype, int32_t discretization,
                                               void *stream);

/* ------------------------------------------------------------------------
 * Backward pass of the selective scan (Euler discretisation): the gradients of a
 * loss with respect to every input of mamba_scan_fwd, given its gradients dy with
 * respect to y and, optionally, dh_last with respect to h_last.  "Understanding
 * Mamba" (aiattnstudio.link) section 7.3 and the hnwysp.cn slides (section 4.4)
 * train the scan with a backward pass that recomputes the states instead of storing
 * them; the pages do not write the gradients out, so they are the chain rule
 * applied to the recurrence at the top of this file.  With mu_t = dLoss/dh_t,
 * s_t = sum_n C_t[n] h_t[n] + D u_t and ds_t = dy_t * silu(z_t) (ds_t = dy_t
 * without a gate):
 *
 *   mu_{L-1} = dh_last + ds_{L-1} C_{L-1},   mu_t = Abar_{t+1} mu_{t+1} + ds_t C_t
 *   du[b,t,d]     = ds_t D[d] + Delta_t sum_n mu_t[n] B_t[n]
 *   ddelta[b,t,d] = sigmoid(delta + delta_bias) * sum_n mu_t[n] (A[d,n] Abar_t[n]
 *                   h_{t-1}[n] + B_t[n] u_t)
 *   dz[b,t,d]     = dy_t s_t silu'(z_t)
 *   dB[b,t,n] = sum_d mu_t[n] Delta_t u_t          dC[b,t,n] = sum_d ds_t h_t[n]
 *   dA[d,n]   = sum_{b,t} mu_t[n] Delta_t Abar_t[n] h_{t-1}[n]
 *   dD[d]     = sum_{b,t} ds_t u_t                 d_delta_bias[d] = sum_{b,t} ddelta
 *   dh0[b,d,n] = Abar_0[n] mu_0[n]
 *
 *   inputs u, delta, A, B, C, D, z, delta_bias, h0: as for mamba_scan_fwd
 *   dy            (batch, seqlen, d_inner) dtype    required if seqlen > 0
 *   dh_last       (batch, d_inner, d_state) float32 nullable (0)
 *   du, ddelta    (batch, seqlen, d_inner) dtype    outputs, required if seqlen > 0
 *   dz            (batch, seqlen, d_inner) dtype    output, required when z is given
 *                                                   (ignored without z)
 *   dB, dC        (batch, seqlen, d_state) dtype    outputs, nullable (not computed)
 *   dA            (d_inner, d_state) float32        output, nullable
 *   dD, d_delta_bias (d_inner) float32              outputs, nullable (dD is returned
 *                                                   also when D is NULL)
 *   dh0           (batch, d_inner, d_state) float32 output, nullable
 *   workspace     see mamba_scan_bwd_workspace_size (required when seqlen > 0)
 *
 * Outputs are written, not accumulated.  Sums over channels, batch rows and time are
 * formed in float32 in a fixed order (results are bitwise reproducible); outputs in
 * dtype are rounded to nearest even.  d_state must be in 1..32 (4, 8, 16, 32 run as
 * compiled, the others padded as described at MAMBA_MAX_D_STATE; MAMBA_ERR_UNSUPPORTED
 * otherwise).  With seqlen == 0 only dh0 (= dh_last, or 0),
 * dA, dD and d_delta_bias (0) are written.  Aliasing: no output may overlap an input
 * or another output, and the workspace overlaps nothing (MAMBA_ERR_ALIASING).
 * Other conventions as for every entry point.
 */
MAMBA_API size_t mamba_scan_bwd_workspace_size(int64_t batch, int64_t seqlen, int64_t d_inner,
                                               int64_t d_state);

/* The same for explicit options (see mamba_scan_bwd_ex; opts may be NULL). */
MAMBA_API size_t mamba_scan_bwd_workspace_size_ex(int64_t batch, int64_t seqlen,
                                                  int64_t d_inner, int64_t d_state,
                                                  const mamba_scan_opts_t *opts);

MAMBA_API mamba_status_t mamba_scan_bwd(const void *u, const void *delta, const float *A,
                                        const void *B, const void *C, const float *D,
                                        const void *z, const float *delta_bias,
                                        const float *h0, const void *dy, const float *dh_last,
                                        void *du, void *ddelta, float *dA, void *dB, void *dC,
                                        float *dD, void *dz, float *d_delta_bias, float *dh0,
                                        int64_t batch, int64_t seqlen, int64_t d_inner,
                                        int64_t d_state, mamba_dtype_t dtype, void *workspace,
                                        size_t workspace_bytes, void *stream);

/* mamba_scan_bwd with explicit options (opts NULL = auto).  n_spans: the sequence is
 * split into that many spans (1..64) scanned in parallel and joined by carry passes for
 * the state (forward) and for its gradient (backward in time); the automatic choice splits
 * when the (batch row, 64-channel tile) units cannot fill the device, and depends on the
 * current device's compute-unit count.  discretization: MAMBA_DISC_ZOH gives the gradients
 * of the zero-order-hold scan (mamba_scan_fwd_ex with the same option): through Bbar =
 * (exp(Delta A) - 1) / A B, dBbar/dDelta = Abar B and dBbar/dA = (Delta Abar - Bbar / B) / A
 * B (Delta^2 / 2 B at A = 0); not with stored checkpoints (mamba_scan_bwd_ckpt,
 * MAMBA_ERR_UNSUPPORTED).  Any other nonzero field returns MAMBA_ERR_UNSUPPORTED.  Results
 * agree across span counts up to float32 rounding. */
MAMBA_API mamba_status_t mamba_scan_bwd_ex(const void *u, const void *delta, const float *A,
                                           const void *B, const void *C, const float *D,
                                           const void *z, const float *delta_bias,
                                           const float *h0, const void *dy,
                                           const float *dh_last, void *du, void *ddelta,
                                           float *dA, void *dB, void *dC, float *dD, void *dz,
                                           float *d_delta_bias, float *dh0, int64_t batch,
                                           int64_t seqlen, int64_t d_inner, int64_t d_state,
                                           mamba_dtype_t dtype, void *workspace,
                                           size_t workspace_bytes,
                                           const mamba_scan_opts_t *opts, void *stream);

/* Bytes of the checkpoint buffer that mamba_scan_fwd_ext writes (ext->ckpt) and
 * mamba_scan_bwd_ckpt reads: (batch * ceil(d_inner / 64)) * ceil(seqlen / 8) * n * 64 * 4,
 * n the compiled size d_state runs at (4, 8, 16 or 32: the next one up).  SIZE_MAX for
 * negative sizes, overflow or a d_state outside 1..32. */
MAMBA_API size_t mamba_scan_ckpt_size(int64_t batch, int64_t seqlen, int64_t d_inner,
                                      int64_t d_state);

/* Workspace size for mamba_scan_bwd_ckpt (opts may be NULL): mamba_scan_bwd_workspace_size
 * without the checkpoint region and, on a split sequence, without the forward span
 * summaries. */
MAMBA_API size_t mamba_scan_bwd_ckpt_workspace_size(int64_t batch, int64_t seqlen,
                                                    int64_t d_inner, int64_t d_state,
                                                    const mamba_scan_opts_t *opts);

/* mamba_scan_bwd_ex reading the states from ckpt, written by mamba_scan_fwd_ext (ext->ckpt)
 * on the same inputs, instead of running a forward pass of its own.  ckpt is required when
 * seqlen > 0 (MAMBA_ERR_NULL_ARG) and read only; it must not overlap an output or the
 * workspace.  Results equal mamba_scan_bwd_ex's up to float32 rounding (the states are the
 * forward scan's rather than the backward's own recomputation).  Other arguments and
 * conventions as for mamba_scan_bwd_ex. */
MAMBA_API mamba_status_t mamba_scan_bwd_ckpt(const void *u, const void *delta, const float *A,
                                             const void *B, const void *C, const float *D,
                                             const void *z, const float *delta_bias,
                                             const float *h0, const void *dy,
                                             const float *dh_last, const float *ckpt, void *du,
                                             void *ddelta, float *dA, void *dB, void *dC,
                                             float *dD, void *dz, float *d_delta_bias,
                                             float *dh0, int64_t batch, int64_t seqlen,
                                             int64_t d_inner, int64_t d_state,
                                             mamba_dtype_t dtype, void *workspace,
                                             size_t workspace_bytes,
                                             const mamba_scan_opts_t *opts, void *stream);

/* ------------------------------------------------------------------------
 * Options of the Mamba-3 formulation ("State space models and the Mamba series",
 * jsqmd.com, sections 2.1 and 2.2), taken as that page writes them.  A NULL pointer
 * switches an option off.
 *
 *   lambda  (batch, seqlen, d_inner) dtype [decode: (batch, d_inner)]
 *       exponential-trapezoidal rule: the input term of step t becomes
 *         (1 - lambda_t) Delta_t B_{t-1}[n] u_{t-1} + lambda_t Delta_t B_t[n] u_t
 *       (the page's look-back term carries no decay factor), with lambda_t the caller's
 *       data-dependent mixing coefficient (in [0, 1]; not checked).  lambda = 1 is the
 *       Euler rule.  Not combinable with the zero-order hold.
 *   u_prev  (batch, d_inner) dtype, B_prev (batch, d_state) dtype
 *       the input (u, B) of the step before t = 0, for continuing a sequence; NULL = 0.
 *       Used only with lambda.
 *   theta   (batch, seqlen, d_state/2) dtype [decode: (batch, d_state/2)]
 *       data-dependent rotation: h_t = exp(Delta_t A) R(Delta_t theta_t) h_{t-1} + (input
 *       term), where R turns each state pair (2k, 2k+1) by the angle
 *       Delta_t * theta[b,t,k]: (x, w) -> (cos x - sin w, sin x + cos w), before the decay.
 *       d_state must be even; in the scan it needs an even d_state from 10 to 32 (run at
 *       16 or 32, where a wave holds whole state pairs), else MAMBA_ERR_UNSUPPORTED.  A split sequence (n_spans > 1) carries
 *       each pair's 2x2 transition over a span (the turn and the pair's two decays do not
 *       commute): more workspace (mamba_scan_fwd_workspace_size_ext) and span passes.
 *
 * Both options run in the SCALAR family (AUTO selects it; ROWS or BLOCK return
 * MAMBA_ERR_UNSUPPORTED).  The extension inputs follow the alignment and aliasing rules
 * of the other inputs.
 *
 *   ckpt    float32 output of mamba_scan_ckpt_size bytes, nullable
 *       the states the backward pass needs ("Understanding Mamba" section 7.3: the
 *       backward recomputes states from stored checkpoints rather than storing every
 *       step): the state h entering every 8-step segment s >= 1 of each (batch row,
 *       64-channel tile), for mamba_scan_bwd_ckpt.  Its layout is internal to the
 *       library; it is written only, 4-byte aligned, and overlaps no other argument or
 *       the workspace (MAMBA_ERR_ALIASING).  Needs the Euler rule without lambda or
 *       theta and d_state 1..32, and runs in the SCALAR family (else
 *       MAMBA_ERR_UNSUPPORTED).  It does not change y or h_last.
 *
 * Row strides of the inputs (elements; 0 = contiguous).  In the Mamba block of
 * "Understanding Mamba" section 5.2 the scan's z (and x) are the two halves of one
 * projection, xz.chunk(2, -1), and B, C slices of another: views whose rows (b, t) are
 * further apart than d_inner (d_state) elements.  With these the scan reads such views in
 * place instead of the caller copying them:
 *   u_stride, delta_stride, z_stride : elements from row (b, t) to row (b, t + 1) of u,
 *       delta, z -- every row, so also from (b, seqlen - 1) to (b + 1, 0): element (b, t, d)
 *       at ptr[(b * seqlen + t) * stride + d]; >= d_inner.  Decode step: from batch row b to
 *       b + 1.
 *   B_stride, C_stride : the same for B and C; >= d_state.
 * A stride below the row length returns MAMBA_ERR_BAD_SHAPE.  Strides other than the row
 * length run in the SCALAR family (AUTO selects it; ROWS, BLOCK and d_state above 32 return
 * MAMBA_ERR_UNSUPPORTED).  The inputs may overlap each other (views of one buffer); y, h_last
 * and the workspace may not overlap the strided extent of any of them.  lambda, u_prev,
 * B_prev, theta and every output stay contiguous; the backward entry points take contiguous
 * inputs only. */
typedef struct {
    const void *lambda;
    const void *u_prev;
    const void *B_prev;
    const void *theta;
    float *ckpt;
    int64_t u_stride, delta_stride, z_stride, B_stride, C_stride;
} mamba_scan_ext_t;

/* ------------------------------------------------------------------------
 * Backward of the scan with the Mamba-3 options of mamba_scan_ext_t: the gradients of
 * mamba_scan_fwd_ext's outputs with lambda (with u_prev, B_prev) and/or theta given, with
 * the Euler rule or (with theta only) the zero-order hold of opts->discretization -- the
 * chain rule through the trapezoidal input term and the pair rotation.  Besides the
 * outputs of mamba_scan_bwd (same shapes, dtypes, rules):
 *   dlam     (batch, seqlen, d_inner) dtype   dLoss/dlambda        (lambda given; nullable)
 *   du_prev  (batch, d_inner) dtype           dLoss/du_prev        (lambda given; nullable)
 *   dB_prev  (batch, d_state) dtype           dLoss/dB_prev        (lambda given; nullable)
 *   dtheta   (batch, seqlen, d_state/2) dtype dLoss/dtheta         (theta given; nullable)
 * d_state 4, 8, 16 or 32 (even with theta); opts may set only discretization and n_spans;
 * ext->ckpt and the row strides must be 0 (else MAMBA_ERR_UNSUPPORTED).  B, C, B_prev and
 * theta must be 16-byte aligned (read as vectors of up to 16 bytes; MAMBA_ERR_MISALIGNED
 * otherwise).  With neither lambda nor theta the call is mamba_scan_bwd_ex.  This path runs
 * one block per (span, batch row, 64 channels), the states of a channel split over 4 lanes
 * (2 for a rotation at d_state 4).  Sequence split (opts->n_spans: 0 automatic, 1 none, up to
 * 64): when the (batch row, 64-channel) units leave compute units idle the sequence is cut
 * into spans of a multiple of 8 steps; the forward's span pass and carry give the state
 * entering each span, an adjoint span pass and a reverse carry the gradient entering it from
 * its end, and the trapezoid's look-back shares at span boundaries are added after the spans
 * (one rounding).  A split with theta needs d_state 16 or 32 (else: unsplit when automatic,
 * MAMBA_ERR_UNSUPPORTED when requested); its workspace grows by the span regions
 * (mamba_scan_bwd_ext_workspace_size with the same options). */
typedef struct {
    void *dlam;
    void *du_prev;
    void *dB_prev;
    void *dtheta;
} mamba_scan_ext_grads_t;

MAMBA_API size_t mamba_scan_bwd_ext_workspace_size(int64_t batch, int64_t seqlen,
                                                   int64_t d_inner, int64_t d_state,
                                                   const mamba_scan_ext_t *ext,
                                                   const mamba_scan_opts_t *opts);

MAMBA_API mamba_status_t mamba_scan_bwd_ext(const void *u, const void *delta, const float *A,
                                            const void *B, const void *C, const float *D,
                                            const void *z, const float *delta_bias,
                                            const float *h0, const void *dy,
                                            const float *dh_last, void *du, void *ddelta,
                                            float *dA, void *dB, void *dC, float *dD, void *dz,
                                            float *d_delta_bias, float *dh0,
                                            const mamba_scan_ext_t *ext,
                                            const mamba_scan_ext_grads_t *ext_grads,
                                            int64_t batch, int64_t seqlen, int64_t d_inner,
                                            int64_t d_state, mamba_dtype_t dtype,
                                            void *workspace, size_t workspace_bytes,
                                            const mamba_scan_opts_t *opts, void *stream);

/* Workspace size for mamba_scan_fwd_ext (ext and opts may be NULL). */
MAMBA_API size_t mamba_scan_fwd_workspace_size_ext(int64_t batch, int64_t seqlen,
                                                   int64_t d_inner, int64_t d_state,
                                                   const mamba_scan_ext_t *ext,
                                                   const mamba_scan_opts_t *opts);

/* mamba_scan_fwd_ex with the Mamba-3 options (ext NULL = none). */
MAMBA_API mamba_status_t mamba_scan_fwd_ext(const void *u, const void *delta, const float *A,
                                            const void *B, const void *C, const float *D,
                                            const void *z, const float *delta_bias,
                                            const float *h0, void *y, float *h_last,
                                            int64_t batch, int64_t seqlen, int64_t d_inner,
                                            int64_t d_state, mamba_dtype_t dtype,
                                            void *workspace, size_t workspace_bytes,
                                            const mamba_scan_opts_t *opts,
                                            const mamba_scan_ext_t *ext, void *stream);

/*
 * Relay hand-offs that timed out in the last mamba_scan_fwd_ex / _ext call that used
 * `workspace` with the same sizes, opts and ext (mamba_scan_opts_t.relay): *faults = the
 * number of relay parts whose wait for the previous part's state gave up (their outputs are
 * NaN).  0 whenever that call planned no relay.  Synchronises `stream` (the call must have
 * been enqueued on it) and copies one word to the host.  Errors: MAMBA_ERR_NULL_ARG (faults
 * NULL), the size and option errors of mamba_scan_fwd_ext, MAMBA_ERR_WORKSPACE (workspace
 * smaller than that call's), MAMBA_ERR_HIP (the copy or the synchronisation failed).
 */
MAMBA_API mamba_status_t mamba_scan_fwd_relay_faults(const void *workspace,
                                                     size_t workspace_bytes, int64_t batch,
                                                     int64_t seqlen, int64_t d_inner,
                                                     int64_t d_state,
                                                     const mamba_scan_opts_t *opts,
                                                     const mamba_scan_ext_t *ext,
                                                     uint32_t *faults, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): mamba_scan_fwd with the same arguments
 * minus the workspace.  The workspace mamba_scan_fwd_workspace_size reports for these sizes
 * is taken from a device array the library holds on every device it runs on (reserved when
 * the library's code is loaded, kept until the process ends); the call itself allocates and
 * frees nothing.  Limit: that size must be at most MAMBA_SCAN_NOALLOC_MAX_WORKSPACE (64 MiB:
 * the large prefill 8 x 4096 x 5120 needs 4.5 MiB, the long sequence 1 x 131072 x 2048
 * 40 MiB), else MAMBA_ERR_WORKSPACE and nothing is launched.  The array belongs to the
 * device of `stream` (the current device for NULL); all calls on one device share it, so
 * calls that overlap on one device race and must be serialised by the caller (for example
 * by issuing them on one stream).  Results are those of mamba_scan_fwd, bitwise.  Errors as
 * mamba_scan_fwd; MAMBA_ERR_HIP if the array's address cannot be looked up.
 */
#define MAMBA_SCAN_NOALLOC_MAX_WORKSPACE ((size_t)64 << 20)
MAMBA_API mamba_status_t mamba_scan_fwd_noalloc(const void *u, const void *delta,
                                                const float *A, const void *B, const void *C,
                                                const float *D, const void *z,
                                                const float *delta_bias, const float *h0,
                                                void *y, float *h_last, int64_t batch,
                                                int64_t seqlen, int64_t d_inner,
                                                int64_t d_state, mamba_dtype_t dtype,
                                                void *stream);

/* mamba_state_update_ex with the Mamba-3 options (shapes of the decode step; ext NULL =
 * none).  With lambda the caller passes the previous token's u and B as u_prev, B_prev.
 * ext->ckpt must be NULL (MAMBA_ERR_UNSUPPORTED otherwise). */
MAMBA_API mamba_status_t mamba_state_update_ext(float *h, const void *u, const void *delta,
                                                const float *A, const void *B, const void *C,
                                                const float *D, const void *z,
                                                const float *delta_bias, void *y,
                                                int64_t batch, int64_t d_inner,
                                                int64_t d_state, mamba_dtype_t dtype,
                                                int32_t discretization,
                                                const mamba_scan_ext_t *ext, void *stream);

/* ------------------------------------------------------------------------
 * Mamba-2 SSD scan: the state-space-duality form of "Understanding Mamba"
 * (aiattnstudio.link) section 6 -- y_t = sum_{s<=t} C_t . B_s (prod_{l=s+1..t} Abar_l)
 * Bbar_s x_s -- with the scalar state transition per head of Mamba-2 ("State space models
 * and the Mamba series", jsqmd.com, section 1.2: A = diag(a)), computed in chunks with
 * matrix products on the matrix cores.  d_inner = n_heads * head_dim channels; head h owns
 * channels [h * head_dim, (h+1) * head_dim).  For every b, h, channel p of the head and n:
 *
 *   Delta_t   = softplus(dt[b,t,h] + dt_bias[h])
 *   h_t[p,n]  = exp(Delta_t * A[h]) * h_{t-1}[p,n] + Delta_t * B[b,t,n] * x[b,t,h*P+p]
 *   y[b,t,h*P+p] = (sum_n C[b,t,n] * h_t[p,n] + D[h] * x[b,t,h*P+p]) * silu(z[b,t,h*P+p])
 *
 * i.e. the selective scan above with Delta and A shared by the channels of a head.
 *
 *   x, z, y   (batch, seqlen, n_heads * head_dim) dtype   z nullable (no gate)
 *   dt        (batch, seqlen, n_heads) dtype
 *   A         (n_heads) float32 (normally < 0)         D, dt_bias (n_heads) float32 nullable
 *   B, C      (batch, seqlen, d_state) dtype (shared by all heads)
 *   h0, h_last (batch, n_heads * head_dim, d_state) float32, nullable
 *
 * head_dim must be 64 and d_state 64 or 128 (mamba_ssd_supported), and 64 rows of x must
 * span fewer than 2^31 bytes (n_heads * head_dim * element size * 64), else
 * MAMBA_ERR_UNSUPPORTED.  Arithmetic: bf16 inputs use bf16 matrix-core products with fp32
 * accumulation; the operands computed in fp32 (the chunk's decay-weighted C.B^T, the
 * decay-weighted x and the state read by C h) enter as a bf16 pair hi + lo, about 16
 * significant bits; the carried state is fp32.  fp32 inputs use fp32 products.
 * mamba_ssd_fwd needs no workspace; mamba_ssd_fwd_ex may (below).  x, z, B and C must be
 * 16-byte aligned (they are read as 16-byte vectors; MAMBA_ERR_MISALIGNED otherwise).  y and
 * h_last must not overlap any input or each other (h_last may not be h0).  Other
 * conventions as for every entry point. */
MAMBA_API int32_t mamba_ssd_supported(int64_t head_dim, int64_t d_state);

MAMBA_API mamba_status_t mamba_ssd_fwd(const void *x, const void *dt, const float *A,
                                       const void *B, const void *C, const float *D,
                                       const void *z, const float *dt_bias, const float *h0,
                                       void *y, float *h_last, int64_t batch, int64_t seqlen,
                                       int64_t n_heads, int64_t head_dim, int64_t d_state,
                                       mamba_dtype_t dtype, void *stream);

/*
 * mamba_ssd_fwd with the device kept busy.  The (batch row, head) units run one block each,
 * a fixed number at a time (blocks per compute unit x compute units, the "slots"):
 *  - relay: when the units overflow the slots by a partial round, the units of that round
 *    would run on a mostly idle device; instead each runs in two parts -- the first half of
 *    the sequence (whole 64-step chunks) in the first round, the second, continuing from
 *    the first's final state, in the slots the last full round frees (the balance the
 *    scan's relay gives, mamba_scan_opts_t.relay).  Results equal mamba_ssd_fwd bitwise.
 *  - split: when the units fill at most half of the slots, the sequence is cut into spans
 *    (whole chunks) that run in parallel: a first pass gives each span's final state from
 *    zero and its total decay, a carry turns them into the state entering each span, and
 *    the output pass runs every span from its true state (the scan's span split).  Results
 *    equal mamba_ssd_fwd within the stated bounds (the carry rounds differently).
 * Options (NULL = automatic):
 *   relay:   0 automatic (the overflow is at most half of the slots and the sequence has at
 *            least 8 chunks); 1 off; 2 force two parts on the overflow units, or on every
 *            unit when they fit the slots (testing; sequences of at least 2 chunks); -2 as 2,
 *            with the first parts withholding their hand-off (failure test).  A second part's
 *            wait is bounded; one that gives up is counted in the workspace (read with
 *            mamba_ssd_relay_faults) and the part continues from a NaN state, so its outputs
 *            and the unit's final state are NaN, never silently wrong.
 *   n_spans: 0 automatic (as many spans as fill one round, each of at least 8 chunks); 1 no
 *            split; k in [2, 64] force k spans (fewer when the sequence has fewer chunks).
 *   A split takes precedence over the relay; forcing both is MAMBA_ERR_UNSUPPORTED, as are
 *   values out of range.
 * Workspace (caller-owned device memory, 4-byte aligned, not overlapping any argument),
 * size from mamba_ssd_workspace_size for the same arguments on the same device (0: none
 * needed, NULL allowed; (size_t)-1 for arguments mamba_ssd_fwd_ex would reject): relay, one
 * flag per relayed unit and a fault word (256-byte aligned block) and one head_dim x d_state
 * fp32 state per relayed unit; split, (n_spans - 1) states
 * and decays per unit.  MAMBA_ERR_WORKSPACE when missing or too small.  Its contents on
 * entry do not matter and are overwritten.  Concurrent calls must not share a workspace.
 */
typedef struct {
    int32_t relay;
    int32_t n_spans;
} mamba_ssd_opts_t;

MAMBA_API size_t mamba_ssd_workspace_size(int64_t batch, int64_t seqlen, int64_t n_heads,
                                          int64_t head_dim, int64_t d_state,
                                          mamba_dtype_t dtype, const mamba_ssd_opts_t *opts);

MAMBA_API mamba_status_t mamba_ssd_fwd_ex(const void *x, const void *dt, const float *A,
                                          const void *B, const void *C, const float *D,
                                          const void *z, const float *dt_bias, const float *h0,
                                          void *y, float *h_last, int64_t batch,
                                          int64_t seqlen, int64_t n_heads, int64_t head_dim,
                                          int64_t d_state, mamba_dtype_t dtype,
                                          void *workspace, size_t workspace_bytes,
                                          const mamba_ssd_opts_t *opts, void *stream);

/* Relay hand-offs that timed out in the last mamba_ssd_fwd_ex call that used `workspace`
 * with the same arguments and opts: *faults as for mamba_scan_fwd_relay_faults (0 when that
 * call planned no relay).  Synchronises `stream`.  Errors as mamba_ssd_fwd_ex's size and
 * option checks, MAMBA_ERR_NULL_ARG, MAMBA_ERR_WORKSPACE, MAMBA_ERR_HIP. */
MAMBA_API mamba_status_t mamba_ssd_relay_faults(const void *workspace, size_t workspace_bytes,
                                                int64_t batch, int64_t seqlen, int64_t n_heads,
                                                int64_t head_dim, int64_t d_state,
                                                mamba_dtype_t dtype,
                                                const mamba_ssd_opts_t *opts, uint32_t *faults,
                                                void *stream);

/*
 * One decode token of the Mamba-2 SSD on a persistent fp32 state: the recurrence of
 * mamba_ssd_fwd for a single step ("Understanding Mamba" section 6, "State space models and
 * the Mamba series" section 1.2, in their recurrent form), with Delta = softplus(dt[b,h] +
 * dt_bias[h]) and exp(Delta A[h]) shared by the head's channels and state indices:
 *   h[b,h*P+p,n] <- exp(Delta A[h]) h[b,h*P+p,n] + Delta B[b,n] x[b,h*P+p]
 *   y[b,h*P+p]    = (sum_n C[b,n] h[b,h*P+p,n] + D[h] x[b,h*P+p]) * silu(z[b,h*P+p])
 *   h          (batch, n_heads * head_dim, d_state) float32, updated in place, 16-byte
 *              aligned (moved as 16-byte vectors)
 *   x, z, y    (batch, n_heads * head_dim) dtype        z nullable (no gate)
 *   dt         (batch, n_heads) dtype
 *   B, C       (batch, d_state) dtype
 *   A          (n_heads) float32        D, dt_bias (n_heads) float32 nullable
 * Sizes, dtypes and supported (head_dim, d_state) as for mamba_ssd_fwd.  y must not overlap
 * h or any input, and h no input.  fp32 arithmetic throughout; chained steps follow the
 * scan's recurrence exactly, while mamba_ssd_fwd evaluates it in chunked matrix form (equal
 * within the stated bounds, not bitwise).  No workspace.
 */
MAMBA_API mamba_status_t mamba_ssd_state_update(float *h, const void *x, const void *dt,
                                                const float *A, const void *B, const void *C,
                                                const float *D, const void *z,
                                                const float *dt_bias, void *y, int64_t batch,
                                                int64_t n_heads, int64_t head_dim,
                                                int64_t d_state, mamba_dtype_t dtype,
                                                void *stream);

/* Static, human-readable name of a status code (never NULL). */
MAMBA_API const char *mamba_status_string(mamba_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_SCAN_H */
