// Mamba-2 SSD (state-space duality) scan for gfx950, chunked, with the dense parts on MFMA.
//
// Operation.  "Understanding Mamba" (aiattnstudio.link) section 6 and "State space models
// and the Mamba series" (jsqmd.com) section 1.2: Mamba-2 makes the state transition a
// scalar per head, A = a I, which turns the scan into the dual "attention" form
//   y_t = sum_{s<=t} C_t . B_s (prod_{l=s+1..t} Abar_l) Bbar_s x_s
// evaluated with matrix products.  Per batch row b and head h (d_inner = H heads of P
// channels), with Delta_t = softplus(dt[b,t,h] + dt_bias[h]), Abar_t = exp(Delta_t A[h]),
// Bbar_t = Delta_t B_t (Euler, as Mamba-1/2 use), state H_t (N x P):
//   H_t = Abar_t H_{t-1} + Delta_t B_t x_t^T,   y_t = C_t^T H_t + D[h] x_t   (* silu(z_t))
// -- the selective scan with A[d,n] = A[h] and Delta shared by the head's channels.
//
// Chunked evaluation (chunks of Q = 64 steps; cs = inclusive cumulative sum of Delta A
// within the chunk, in log2 units): per chunk,
//   S      = C B^T                                   (Q x Q, contraction over N)
//   M[t,s] = S[t,s] exp(cs_t - cs_s) Delta_s  (s <= t, else 0),  plus D on the diagonal
//   Y      = M X + diag(exp(cs)) C H_in               (Q x P)
//   H_out  = exp(cs_{Q-1}) H_in + B^T Xtil,   Xtil[s,p] = exp(cs_{Q-1} - cs_s) Delta_s X[s,p]
// One block per (batch row, head) walks the chunks in order; nothing of the chunk states
// goes to HBM.  When the units overflow the device's block slots by a partial round, the
// units of that round are relayed: each runs as two blocks, the second continuing from
// the first's final state (relay.h), so the last round is not left mostly idle.  When the
// units are too few for the device, the sequence is split into spans instead: a span pass
// (END) gives each span's final state from zero and its total decay, a carry kernel folds
// them into the state entering each span, and the output pass runs the spans in parallel.
//
// Work split.  Wave w of the block's four owns the columns p in [16w, 16w + 16) of Y and of
// H, and keeps its N x 16 slab of H in MFMA accumulators (16 x 16 tiles) from chunk to
// chunk.  That slab is also the right operand of C H_in: the contraction index of an MFMA
// may be permuted freely as long as both operands agree, and the accumulator rows a lane
// holds (4 consecutive n in each of two tiles) are exactly as many as an operand lane
// takes, so C is read from LDS in the same permuted order and H never passes through LDS.
// The causal tiles of S (10 of the 16 tiles of 16 x 16) are shared out among the waves
// and M goes through LDS; the Xtil operand is formed in registers from columns of X.
//
// Precision.  The products use v_mfma_f32_16x16x32_bf16 for bf16 inputs and
// v_mfma_f32_16x16x4f32 for fp32 inputs.  With bf16 inputs, X, B and C are exact bf16
// values, but M, Xtil and H are computed in fp32: each is split as hi + lo (hi = its bf16
// rounding, lo = the bf16 rounding of the remainder) and enters as two products, which
// keeps about 16 significant bits (rounding any one of them to a single bf16 measured
// 2.2e-2 to 4.4e-2 relative error in y on a CPU emulation of this arithmetic).
//
// Memory.  Inputs are read with 16-byte buffer loads through descriptors that end at the
// chunk's last row, so rows past the end of the sequence read as zero and stores to them
// are dropped.  The loads of the next chunk are issued before the current chunk's products
// and land in registers; the block barriers wait only for LDS traffic, so those loads stay
// in flight across them.  Every matrix is staged in LDS as rows only: the products that
// contract over the steps (B^T Xtil, M X) take their X and B operands down the columns
// with gfx950's transposing LDS reads, so no transposed copy is written.  C and M, read
// only along rows, are unpadded with the 16-byte granules of each row permuted by an XOR
// key of the row; X and B rows are padded by 32 bytes, which keeps their addresses affine
// (unrolled column blocks are immediate offsets) and spreads the rows a transposing read
// covers over distinct banks.
// Blocks are numbered so that each XCD takes a contiguous range of (batch row, head) pairs:
// the heads of one batch row share B and C in that XCD's L2.
#include <atomic>

#include "device_math.h"
#include "relay.h"
#include "scan_common.h"
#include "ssd.h"

namespace mambascan {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kQ = 64;        // chunk length
constexpr int kP = 64;        // head dimension
constexpr int kThreads = 256; // 4 waves
constexpr int kRsrcWord3 = 0x00020000; // gfx9 raw-buffer descriptor word 3

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kRsrcWord3);
}

// Block barrier that waits for this wave's LDS accesses only (a __syncthreads also waits
// for every outstanding global load, which would drain the prefetch).
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0); vmcnt and expcnt not waited for
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// The MFMA used for an element type: k per instruction (KI) and per lane (KL).
template <typename T> struct Mma;
template <> struct Mma<uint16_t> {
    static constexpr int KI = 32, KL = 8;
    static constexpr bool SPLIT = true; // computed operands as hi + lo
    typedef __bf16 E;
    typedef bf16x8 Frag;
    static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ E from_float(float v) { return static_cast<__bf16>(v); }
    static __device__ __forceinline__ float to_float(E v) { return static_cast<float>(v); }
};
template <> struct Mma<float> {
    static constexpr int KI = 4, KL = 1;
    static constexpr bool SPLIT = false;
    typedef float E;
    typedef float Frag;
    static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ E from_float(float v) { return v; }
    static __device__ __forceinline__ float to_float(E v) { return v; }
};

// Layouts of the LDS matrices (RL elements of ES bytes per row; 64 banks of 4 bytes).
// LayX: rows unpadded, the 16-byte granules of row r permuted by an XOR key of r, for the
// matrices read along their rows (operand loads of 16 lanes on 16 consecutive rows at one
// granule, which the key puts in distinct banks).
template <int RL, int ES> struct LayX {
    static constexpr int size(int rows) { return rows * RL; }
    static __device__ __forceinline__ int idx(int r, int c)
    {
        constexpr int G = 16 / ES, RB = RL * ES;
        static_assert(RB % 128 == 0, "row bytes");
        const int key = RB == 128 ? (r >> 1) & 7 : r & 15;
        return r * RL + (((c / G) ^ key) * G) + (c % G);
    }
};
// LayT: rows padded by 32 bytes, so consecutive rows start 8 banks apart, for the matrices
// also read down their columns (col_frag: 32 lanes on 8 consecutive rows, 32 bytes of
// each).  Addresses stay affine in the column, so the column blocks of an unrolled loop are
// immediate offsets of one address.
template <int RL, int ES> struct LayT {
    static constexpr int kPitch = RL + 32 / ES;
    static constexpr int size(int rows) { return rows * kPitch; }
    static __device__ __forceinline__ int idx(int r, int c) { return r * kPitch + c; }
};

// Staging map of a chunk's 64-row matrix of RB-byte rows: a thread's unit j is the 16-byte
// granule gran(lane) of row row(j, w, lane), and each wave instruction covers whole rows, so
// a quarter-wave's 16-byte writes cover 256 contiguous bytes of one row (RB >= 256) or two
// 128-byte rows, D apart: rows that start 32 banks apart (D = 4 for the 32-byte-padded
// LayT, whose rows start 40 banks apart) or rows of different parity (D = 1 for LayX).
template <int RB, int D> struct StageMap {
    static constexpr int LPR = RB / 16;           // lanes per row
    static constexpr int U = 64 * LPR / kThreads; // units per thread
    static_assert(LPR == 8 || LPR == 16 || LPR == 32, "row bytes");
    static __device__ __forceinline__ int row(int j, int w, int lane)
    {
        if constexpr (LPR >= 16) {
            return j * (kThreads / LPR) + w * (64 / LPR) + lane / LPR;
        } else {
            const int q = lane >> 4, h = (lane >> 3) & 1;
            return 32 * j + 8 * w + (D == 4 ? q + 4 * h : 2 * q + h);
        }
    }
    static __device__ __forceinline__ int gran(int lane) { return lane % LPR; }
};

// MFMA operand of KL contiguous elements at index i of an LDS matrix.
template <typename T>
__device__ __forceinline__ typename Mma<T>::Frag frag(const typename Mma<T>::E *m, int i)
{
    if constexpr (Mma<T>::KL == 8)
        return *reinterpret_cast<const bf16x8 *>(m + i);
    else
        return m[i];
}

// MFMA operand running down a column of a row-major LDS matrix, the operand of a
// contraction over the matrix's rows.  fp32: row r0 of column c0 + r16 (r16 = lane % 16).
// bf16: operand slots 0..3 from rows r0 .. r0 + 3 and slots 4..7 from rows r1 .. r1 + 3 of
// column c0 + r16 (r0, r1 may differ between the 16-lane groups), by two transposing reads
// (ds_read_b64_tr_b16): within each 16-lane group, the lane with index l in the group
// addresses the 4 elements at row r0 + l / 4, columns c0 + 4 (l % 4) .. + 3, and lane
// 4a + b of the group receives element b of the lanes a, a + 4, a + 8, a + 12, in that
// order (measured on gfx950), i.e. rows r0 .. r0 + 3 of column c0 + 4a + b.
template <typename T, typename LAY>
__device__ __forceinline__ typename Mma<T>::Frag col_frag(const typename Mma<T>::E *m, int r0,
                                                          int r1, int c0, int r16)
{
    if constexpr (Mma<T>::KL == 8) {
        typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
        typedef __attribute__((address_space(3))) __bf16 lds_bf16;
        lds_bf16 *base = (lds_bf16 *)(const_cast<__bf16 *>(m));
        const int dr = r16 >> 2, c = c0 + 4 * (r16 & 3);
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4 *)(base + LAY::idx(r0 + dr, c)));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4 *)(base + LAY::idx(r1 + dr, c)));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
        return m[LAY::idx(r0, c0 + r16)];
    }
}

// Split v into hi (its bf16 rounding) and lo (the bf16 rounding of v - hi).
__device__ __forceinline__ void split_bf16(float v, __bf16 &hi, __bf16 &lo)
{
    hi = static_cast<__bf16>(v);
    lo = static_cast<__bf16>(v - static_cast<float>(hi));
}

// a + b = s + e exactly (Knuth's TwoSum; no reassociation, no FMA is involved).
__device__ __forceinline__ void two_sum(float a, float b, float &s, float &e)
{
    s = a + b;
    const float bb = s - a;
    e = (a - (s - bb)) + (b - bb);
}

// v from the lane that DPP control CTRL names, in the rows of ROWS; 0 where there is none.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp0(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xf, false));
}

__device__ __forceinline__ float lane_63(float v)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

struct SsdArgs {
    const void *x, *dt, *B, *C, *z;
    const float *A, *D, *dt_bias, *h0;
    void *y;
    float *h_last;
    int64_t L;
    int32_t H; // heads
    // relay: units = batch * heads; the last r_units of them run in two parts, the second
    // from step r_mid; 0 = none
    int32_t units, r_units;
    int64_t r_mid;
    uint32_t *r_sync;  // hand-off flags, then the count of waits that gave up
    float *r_state;
    uint32_t r_polls;  // poll limit of a wait
    int32_t r_withhold; // testing: part 0 does not hand its state over
    // sequence split into n_spans spans of span_len steps (a multiple of the chunk); sp holds
    // per span s < n_spans - 1 and unit its final state (END pass, from h0 for span 0 and
    // from zero otherwise), turned by the carry into the state entering span s + 1; sp_dec
    // the span's total decay
    int32_t n_spans;
    int64_t span_len;
    float *sp, *sp_dec;
};

// bf16: two blocks per CU (75 KB of LDS each at N = 128), so registers are held to 256.
// END: the span pass of a split sequence, which only carries the state (no outputs).
template <typename T, int N, bool GATED, bool END = false>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 2 : 1)))
ssd_chunk_kernel(SsdArgs p)
{
    typedef Mma<T> M;
    typedef typename M::E E;
    typedef typename M::Frag F;
    constexpr int Q = kQ, P = kP, ES = (int)sizeof(T);
    constexpr int G = 16 / ES;           // elements per 16-byte vector
    constexpr int KI = M::KI, KL = M::KL;
    constexpr int NT = N / 16;           // 16-row tiles of this wave's H slab
    constexpr int NS = M::SPLIT ? 2 : 1;
    static_assert(N % 32 == 0 && Q == 64 && P == 64, "shape");

    // X [t][p], B [s][n], C [t][n], M [t][s] (hi, then lo when split), all row-major; X and
    // B are also read down their columns (col_frag) as operands of B^T Xtil and M X
    typedef LayT<P, ES> LX;
    typedef LayT<N, ES> LB;
    typedef LayX<N, ES> LC;
    typedef LayX<Q, ES> LM;
    __shared__ __attribute__((aligned(16))) E s_x[LX::size(Q)];
    __shared__ __attribute__((aligned(16))) E s_b[LB::size(Q)];
    __shared__ __attribute__((aligned(16))) E s_c[LC::size(Q)];
    __shared__ __attribute__((aligned(16))) E s_m[NS * LM::size(Q)];
    // per step: cumulative decay cs = cs_hi + cs_lo (a compensated sum: M uses differences
    // cs_t - cs_s, which a plain fp32 sum would lose when |cs| is large), Delta, the weight
    // of Xtil, exp(cs); and the chunk's total decay
    __shared__ __attribute__((aligned(16))) float s_cs[Q], s_csl[Q], s_dl[Q], s_w[Q], s_e[Q];
    __shared__ float s_dec;

    const int tid = threadIdx.x;
    const int lane = tid & 63, g = lane >> 4, r16 = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

    // Work unit (batch row, head) and steps [t_begin, L) of this block.  Blocks go
    // round-robin over the 8 XCDs; the whole units are renumbered so each XCD takes a
    // contiguous range (the heads of a batch row share B and C in one L2).  With relay the
    // grid is [part 0 of each relayed unit][whole units][part 1 of each relayed unit]:
    // workgroups are dispatched in index order, so the part-0 blocks start in the first
    // round, the part-1 blocks take the slots the whole units' last round frees, and a
    // part 1 waits only for a block of smaller index.
    const int idx = (int)blockIdx.x;
    const int whole = p.units - p.r_units;
    int bh = idx - p.r_units, part = -1, span = 0, slot = 0;
    const int64_t L = p.L;
    int64_t t_begin = 0, t_end = L;
    if (p.n_spans > 1) { // split sequence: block = (span, unit), no relay
        span = idx / p.units;
        bh = idx % p.units;
        if (p.units % 8 == 0)
            bh = (bh % 8) * (p.units / 8) + bh / 8;
        t_begin = (int64_t)span * p.span_len;
        t_end = min(t_begin + p.span_len, L);
    } else {
        // j: index within the block's group (part 0, whole, part 1); a relayed unit's slot
        int j = idx - p.r_units;
        if (idx < p.r_units) {
            j = idx;
            part = 0;
            t_end = p.r_mid;
        } else if (idx >= p.units) {
            j = idx - p.units;
            part = 1;
            t_begin = p.r_mid;
        }
        const bool relayed = part >= 0;
        if (p.units % 8 == 0 && p.r_units % 8 == 0) {
            // every group starts on XCD 0: XCD x takes units [x, x + 1) * units / 8, its
            // whole units first, then its relayed ones
            bh = (j % 8) * (p.units / 8) + (relayed ? whole / 8 : 0) + j / 8;
        } else {
            bh = relayed ? whole + j : j;
        }
        slot = j;
    }
    const int b = bh / p.H, h = bh % p.H;
    const int64_t Dn = (int64_t)p.H * P;
    const int pc = 16 * w + r16; // this lane's column of Y and of H

    const char *xb = (const char *)p.x + ((int64_t)b * L * Dn + (int64_t)h * P) * ES;
    const char *zb = GATED ? (const char *)p.z + ((int64_t)b * L * Dn + (int64_t)h * P) * ES
                           : nullptr;
    char *yb = (char *)p.y + ((int64_t)b * L * Dn + (int64_t)h * P) * ES;
    const char *bb = (const char *)p.B + (int64_t)b * L * N * ES;
    const char *cb = (const char *)p.C + (int64_t)b * L * N * ES;
    const char *db = (const char *)p.dt + ((int64_t)b * L * p.H + h) * ES;
    const float a2 = p.A[h] * kLog2e;
    const float dtb = p.dt_bias ? p.dt_bias[h] : 0.0f;
    const float Dh = p.D ? p.D[h] : 0.0f;
    const uint32_t row_x = (uint32_t)(Dn * ES), row_b = (uint32_t)(N * ES);

    // ---- state slab: tile m holds rows n = 16m + 4g + v, column pc ----
    f32x4 hacc[NT];
    // row pc of this unit's P x N state block: a uniform base plus a 32-bit lane offset
    // (one register to keep across the chunk loop for the final stores, not a 64-bit index)
    const int64_t hbase = ((int64_t)b * Dn + (int64_t)h * P) * N;
    const int hcol = pc * N;
    // (the span arrays share this layout: unit bh = b * H + h holds P rows of N at hbase)
    const int64_t sp_stride = (int64_t)p.units * P * N;
    if (p.h0 && part != 1 && span == 0) {
#pragma unroll
        for (int m = 0; m < NT; ++m)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                hacc[m][v] = p.h0[hbase + hcol + 16 * m + 4 * g + v];
    } else if (!END && span > 0) { // the state entering this span, from the carry
        const float *src = p.sp + (int64_t)(span - 1) * sp_stride + hbase + hcol;
#pragma unroll
        for (int m = 0; m < NT; ++m)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                hacc[m][v] = src[16 * m + 4 * g + v];
    } else {
#pragma unroll
        for (int m = 0; m < NT; ++m)
            hacc[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // M's tiles above the diagonal stay zero; the causal tiles are rewritten every chunk
    for (int e = tid; e < NS * LM::size(Q); e += kThreads)
        s_m[e] = M::from_float(0.0f);

    // ---- loads of one chunk into registers, then into LDS as rows (StageMap: each
    // 16-byte unit of a thread is one granule of one row) ----
    typedef StageMap<P * ES, 4> MX; // X, B: padded rows (LayT)
    typedef StageMap<N * ES, 4> MB;
    typedef StageMap<N * ES, 1> MC; // C: XOR-permuted rows (LayX)
    u32x4 fx[MX::U], fb[MB::U], fc[MC::U];
    uint32_t fdt = 0;
    auto fetch = [&](int64_t c0) {
        const int nok = (int)min((int64_t)Q, t_end - c0);
        const rsrc_t rx = make_rsrc(xb + c0 * row_x, (uint32_t)(nok - 1) * row_x + P * ES);
        const rsrc_t rb = make_rsrc(bb + c0 * row_b, (uint32_t)nok * row_b);
        const rsrc_t rc = make_rsrc(cb + c0 * row_b, (uint32_t)nok * row_b);
#pragma unroll
        for (int j = 0; j < MX::U; ++j)
            fx[j] = __builtin_amdgcn_raw_buffer_load_b128(
                rx, (int)(MX::row(j, w, lane) * row_x + MX::gran(lane) * 16), 0, 0);
#pragma unroll
        for (int j = 0; j < MB::U; ++j) {
            fb[j] = __builtin_amdgcn_raw_buffer_load_b128(
                rb, (int)(MB::row(j, w, lane) * row_b + MB::gran(lane) * 16), 0, 0);
            if constexpr (!END) // (the span pass reads no C)
                fc[j] = __builtin_amdgcn_raw_buffer_load_b128(
                    rc, (int)(MC::row(j, w, lane) * row_b + MC::gran(lane) * 16), 0, 0);
        }
        if (w == 3) {
            const rsrc_t rd = make_rsrc(db + c0 * p.H * ES, (uint32_t)((nok - 1) * p.H + 1) * ES);
            if constexpr (ES == 2)
                fdt = __builtin_amdgcn_raw_buffer_load_b16(rd, lane * p.H * ES, 0, 0);
            else
                fdt = __builtin_amdgcn_raw_buffer_load_b32(rd, lane * p.H * ES, 0, 0);
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int j = 0; j < MX::U; ++j)
            *reinterpret_cast<u32x4 *>(s_x + LX::idx(MX::row(j, w, lane), MX::gran(lane) * G)) =
                fx[j];
#pragma unroll
        for (int j = 0; j < MB::U; ++j) {
            *reinterpret_cast<u32x4 *>(s_b + LB::idx(MB::row(j, w, lane), MB::gran(lane) * G)) =
                fb[j];
            if constexpr (!END)
                *reinterpret_cast<u32x4 *>(s_c + LC::idx(MC::row(j, w, lane),
                                                         MC::gran(lane) * G)) = fc[j];
        }
    };

    // Delta and the decays of the chunk at c0 (wave 3, which has one causal tile of S fewer
    // than waves 0 and 1): an inclusive, compensated prefix sum
    // over the 64 steps by DPP row shifts, then row broadcasts across the 16-lane rows
    auto decays = [&](int64_t c0) {
        const int nn = (int)min((int64_t)Q, t_end - c0);
        const float dv = ES == 2 ? __uint_as_float(fdt << 16) : __uint_as_float(fdt);
        const float dl = lane < nn ? softplus_act<T>(dv + dtb) : 0.0f;
        float cs = dl * a2, csl = 0.0f;
        auto add = [&](float vh, float vl) {
            float sh, e;
            two_sum(cs, vh, sh, e);
            const float l = csl + vl + e;
            cs = sh + l; // renormalise (|sh| >= |l|)
            csl = l - (cs - sh);
        };
        add(dpp0<0x111, 0xf>(cs), dpp0<0x111, 0xf>(csl)); // row_shr:1
        add(dpp0<0x112, 0xf>(cs), dpp0<0x112, 0xf>(csl)); // row_shr:2
        add(dpp0<0x114, 0xf>(cs), dpp0<0x114, 0xf>(csl)); // row_shr:4
        add(dpp0<0x118, 0xf>(cs), dpp0<0x118, 0xf>(csl)); // row_shr:8
        add(dpp0<0x142, 0xa>(cs), dpp0<0x142, 0xa>(csl)); // row_bcast:15 into rows 1 and 3
        add(dpp0<0x143, 0xc>(cs), dpp0<0x143, 0xc>(csl)); // row_bcast:31 into rows 2 and 3
        const float ce = lane_63(cs), cel = lane_63(csl);
        s_cs[lane] = cs;
        s_csl[lane] = csl;
        s_dl[lane] = dl;
        s_w[lane] = hw_exp2((ce - cs) + (cel - csl)) * dl;
        s_e[lane] = hw_exp2(cs + csl);
        if (lane == 0)
            s_dec = hw_exp2(ce + cel);
    };

    // Pipeline: chunk c is staged into LDS while chunk c - 1 finishes (M X and the stores),
    // and its global loads were issued while chunk c - 2 did.
    if (t_begin < t_end) {
        fetch(t_begin);
        stage();
        if (w == 3)
            decays(t_begin);
        if (t_begin + Q < t_end)
            fetch(t_begin + Q);
    }
    if (part == 1) {
        // part 0's final state, once its first chunk is on the way
        // (a wait that gives up is counted and leaves a NaN state: the outputs of this part
        // and the final state become NaN instead of wrong)
        const bool got = relay_receive(p.r_sync + slot, p.r_sync + p.r_units, p.r_polls);
#pragma unroll
        for (int m = 0; m < NT; ++m)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                hacc[m][v] = got ? (p.r_state + (int64_t)slot * P * N)[hcol + 16 * m + 4 * g + v]
                                 : __builtin_nanf("");
    }
    float decp = 1.0f; // END: the span's total decay, the product of its chunks'
    for (int64_t t0 = t_begin; t0 < t_end; t0 += Q) {
        const int nt = (int)min((int64_t)Q, t_end - t0);
        const uint32_t ybytes = (uint32_t)(nt - 1) * row_x + P * ES;
        // gate of this lane's outputs (rows 16 rt + 4g + v), wanted at the end of the chunk
        uint32_t fz[16];
        if constexpr (GATED) {
            const rsrc_t rz = make_rsrc(zb + t0 * row_x, ybytes);
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int off = (int)((16 * (q >> 2) + 4 * g + (q & 3)) * row_x + pc * ES);
                if constexpr (ES == 2)
                    fz[q] = __builtin_amdgcn_raw_buffer_load_b16(rz, off, 0, 0);
                else
                    fz[q] = __builtin_amdgcn_raw_buffer_load_b32(rz, off, 0, 0);
            }
        }
        lds_barrier(); // this chunk is in LDS; the previous chunk's M is no longer read

        // ---- the causal tiles of S = C B^T given to this wave, weighted into M ----
        // (computed transposed, B C^T, so that a lane holds 4 consecutive s of one row t of
        // M and writes them with one store per array)
        if constexpr (!END) {
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                const int k = w + 4 * q; // tiles in row order: (0,0) (1,0) (1,1) (2,0) ...
                if (k < 10) {
                    const int r = k < 1 ? 0 : k < 3 ? 1 : k < 6 ? 2 : 3, c = k - r * (r + 1) / 2;
                    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int ks = 0; ks < N / KI; ++ks)
                        acc = M::mma(frag<T>(s_b, LB::idx(16 * c + r16, KI * ks + KL * g)),
                                     frag<T>(s_c, LC::idx(16 * r + r16, KI * ks + KL * g)), acc);
                    const int t = 16 * r + r16, s0 = 16 * c + 4 * g;
                    const float cst = s_cs[t], cstl = s_csl[t];
                    const f32x4 css = *reinterpret_cast<const f32x4 *>(s_cs + s0);
                    const f32x4 csls = *reinterpret_cast<const f32x4 *>(s_csl + s0);
                    const f32x4 dls = *reinterpret_cast<const f32x4 *>(s_dl + s0);
                    float mv[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int s = s0 + v;
                        float m = s <= t ? acc[v] * hw_exp2((cst - css[v]) + (cstl - csls[v])) *
                                               dls[v]
                                         : 0.0f;
                        if (s == t)
                            m += Dh;
                        mv[v] = m;
                    }
                    const int i = LM::idx(t, s0);
                    if constexpr (M::SPLIT) {
                        bf16x4 hi, lo;
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            __bf16 a, b2;
                            split_bf16(mv[v], a, b2);
                            hi[v] = a;
                            lo[v] = b2;
                        }
                        *reinterpret_cast<bf16x4 *>(s_m + i) = hi;
                        *reinterpret_cast<bf16x4 *>(s_m + LM::size(Q) + i) = lo;
                    } else {
                        *reinterpret_cast<f32x4 *>(s_m + i) = f32x4{mv[0], mv[1], mv[2], mv[3]};
                    }
                }
            }
        }

        // ---- Y = diag(exp(cs)) C H_in on this wave's columns ----
        f32x4 yacc[4];
        if constexpr (!END) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
                yacc[rt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < N / KI; ++ks) {
                if constexpr (KL == 8) {
                    // operand slot (g, e) <-> n = 32 ks + 16 (e / 4) + 4 g + e % 4
                    bf16x8 hh, hl;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        __bf16 a, c;
                        split_bf16(hacc[2 * ks + e / 4][e % 4], a, c);
                        hh[e] = a;
                        hl[e] = c;
                    }
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt) {
                        const int t = 16 * rt + r16;
                        const bf16x4 c0 =
                            *reinterpret_cast<const bf16x4 *>(s_c + LC::idx(t, 32 * ks + 4 * g));
                        const bf16x4 c1 =
                            *reinterpret_cast<const bf16x4 *>(s_c + LC::idx(t, 32 * ks + 16 + 4 * g));
                        const bf16x8 cf = __builtin_shufflevector(c0, c1, 0, 1, 2, 3, 4, 5, 6, 7);
                        yacc[rt] = M::mma(cf, hh, yacc[rt]);
                        yacc[rt] = M::mma(cf, hl, yacc[rt]);
                    }
                } else {
                    // operand slot g <-> n = 16 (ks / 4) + 4 g + ks % 4
                    const float hv = hacc[ks / 4][ks % 4];
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt)
                        yacc[rt] = M::mma(s_c[LC::idx(16 * rt + r16, 16 * (ks / 4) + 4 * g + ks % 4)],
                                          hv, yacc[rt]);
                }
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
                yacc[rt] *= *reinterpret_cast<const f32x4 *>(s_e + 16 * rt + 4 * g);
        }

        // ---- H_out = exp(cs_end) H_in + B^T Xtil on this wave's columns ----
        F xf[Q / KI]; // X operands down this lane's column, also used by M X below
        {
            const float dec = s_dec;
            if constexpr (END)
                decp *= dec;
#pragma unroll
            for (int m = 0; m < NT; ++m)
                hacc[m] *= dec;
#pragma unroll
            for (int js = 0; js < Q / KI; ++js) {
                // the steps of this lane's operand slots: bf16, slots 0..3 at t0 .. t0 + 3
                // and 4..7 at t0 + 16 .. t0 + 19 (an order of the contraction index that
                // M X follows too); fp32, t0
                const int k0 = KL == 8 ? KI * js + 4 * g : KI * js + g, k1 = k0 + 16;
                xf[js] = col_frag<T, LX>(s_x, k0, k1, 16 * w, r16);
                F xh, xl;
                if constexpr (KL == 8) {
                    const f32x4 w0 = *reinterpret_cast<const f32x4 *>(s_w + k0);
                    const f32x4 w1 = *reinterpret_cast<const f32x4 *>(s_w + k1);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        __bf16 a, c;
                        split_bf16(M::to_float(xf[js][e]) * (e < 4 ? w0[e] : w1[e - 4]), a, c);
                        xh[e] = a;
                        xl[e] = c;
                    }
                } else {
                    xh = xf[js] * s_w[k0];
                    xl = 0.0f;
                }
#pragma unroll
                for (int m = 0; m < NT; ++m) {
                    const F a = col_frag<T, LB>(s_b, k0, k1, 16 * m, r16);
                    hacc[m] = M::mma(a, xh, hacc[m]);
                    if constexpr (M::SPLIT)
                        hacc[m] = M::mma(a, xl, hacc[m]);
                }
            }
        }
        lds_barrier(); // M complete; X, B, C and the decays of this chunk no longer read

        // ---- the next chunk into LDS and its decays; the loads of the one after ----
        if (t0 + Q < t_end) {
            stage();
            if (w == 3)
                decays(t0 + Q);
            if (t0 + 2 * Q < t_end)
                fetch(t0 + 2 * Q);
        }

        // ---- Y += M X (D included), gate, store ----
        if constexpr (!END) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
                for (int js = 0; js <= (16 * rt + 15) / KI; ++js) {
                    // M's columns in the order of xf's slots (s = 32 js + 4 g + 0..3, then
                    // 32 js + 16 + 4 g + 0..3 for bf16)
                    const int t = 16 * rt + r16;
                    F mh, ml;
                    if constexpr (KL == 8) {
                        auto m8 = [&](const E *mm) {
                            const bf16x4 a = *reinterpret_cast<const bf16x4 *>(
                                mm + LM::idx(t, KI * js + 4 * g));
                            const bf16x4 c = *reinterpret_cast<const bf16x4 *>(
                                mm + LM::idx(t, KI * js + 16 + 4 * g));
                            return __builtin_shufflevector(a, c, 0, 1, 2, 3, 4, 5, 6, 7);
                        };
                        mh = m8(s_m);
                        if constexpr (M::SPLIT)
                            ml = m8(s_m + LM::size(Q));
                    } else {
                        mh = s_m[LM::idx(t, KI * js + g)];
                    }
                    yacc[rt] = M::mma(mh, xf[js], yacc[rt]);
                    if constexpr (M::SPLIT)
                        yacc[rt] = M::mma(ml, xf[js], yacc[rt]);
                }
            }
            const rsrc_t ry = make_rsrc(yb + t0 * row_x, ybytes);
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                float yv = yacc[q >> 2][q & 3];
                if constexpr (GATED)
                    yv *= silu_f(ES == 2 ? __uint_as_float(fz[q] << 16) : __uint_as_float(fz[q]));
                const int off = (int)((16 * (q >> 2) + 4 * g + (q & 3)) * row_x + pc * ES);
                if constexpr (ES == 2)
                    __builtin_amdgcn_raw_buffer_store_b16(
                        __builtin_bit_cast(uint16_t, static_cast<__bf16>(yv)), ry, off, 0, 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yv), ry, off, 0, 0);
            }
        }
    }

    if constexpr (END) {
        // the span's final state and total decay, for the carry
        float *dst = p.sp + (int64_t)span * sp_stride + hbase + hcol;
#pragma unroll
        for (int m = 0; m < NT; ++m)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                dst[16 * m + 4 * g + v] = hacc[m][v];
        if (tid == 0)
            p.sp_dec[(int64_t)span * p.units + bh] = decp;
        return;
    }
    if (part == 0) {
        if (p.r_withhold)
            return; // failure test: part 1's wait gives up
        // hand the final state to part 1 (the part covers whole chunks: no tail rows)
#pragma unroll
        for (int m = 0; m < NT; ++m)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                (p.r_state + (int64_t)slot * P * N)[hcol + 16 * m + 4 * g + v] = hacc[m][v];
        relay_signal(p.r_sync + slot);
        return;
    }
    if (p.h_last && span == p.n_spans - 1) {
#pragma unroll
        for (int m = 0; m < NT; ++m)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                (p.h_last + hbase)[hcol + 16 * m + 4 * g + v] = hacc[m][v];
    }
}

// Carry over the spans of a split sequence, per unit and state element (in place): the END
// pass left span s's final state from zero (span 0: from h0) and total decay; the state
// entering span s + 1 is decay(s) * (state entering s) + (final state of s from zero).
__global__ void ssd_span_carry_kernel(float *sp, const float *sp_dec, int64_t units,
                                      int32_t n_spans, int32_t pn)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; // unit * pn + element
    if (i >= units * pn)
        return;
    const int64_t u = i / pn, stride = units * pn;
    float run = sp[i];
    for (int s = 1; s < n_spans - 1; ++s) {
        run = __builtin_fmaf(sp_dec[(int64_t)s * units + u], run, sp[s * stride + i]);
        sp[s * stride + i] = run;
    }
}

// Zeroes the relay flags and the fault word before a relayed launch (a kernel, not a
// memset: the launch sequence stays capturable in a graph).
__global__ void ssd_relay_clear_kernel(uint32_t *sync, int32_t n)
{
    const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i < n)
        sync[i] = 0u;
}

template <typename T, int N>
hipError_t launch_ssd_t(const SsdLaunch &q, hipStream_t stream)
{
    SsdArgs a{};
    a.x = q.x;
    a.dt = q.dt;
    a.B = q.B;
    a.C = q.C;
    a.z = q.z;
    a.A = q.A;
    a.D = q.D;
    a.dt_bias = q.dt_bias;
    a.h0 = q.h0;
    a.y = q.y;
    a.h_last = q.h_last;
    a.L = q.L;
    a.H = (int32_t)q.n_heads;
    const int64_t units = q.batch * q.n_heads;
    if (units <= 0)
        return hipSuccess;
    a.units = (int32_t)units;
    a.r_units = (int32_t)q.relay_units;
    a.r_mid = q.relay_mid;
    a.r_sync = q.relay_sync;
    a.r_state = q.relay_state;
    a.r_polls = q.relay_withhold ? kRelayTestPolls : kRelayPolls;
    a.r_withhold = q.relay_withhold ? 1 : 0;
    a.n_spans = q.n_spans > 1 ? (int32_t)q.n_spans : 1;
    a.span_len = q.span_len;
    a.sp = q.span_state;
    a.sp_dec = q.span_decay;
    if (a.n_spans > 1) {
        // the spans' final states from zero, the carry, then the outputs from the true states
        hipLaunchKernelGGL((ssd_chunk_kernel<T, N, false, true>),
                           dim3((uint32_t)(units * (a.n_spans - 1))), dim3(kThreads), 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        const int64_t n = units * kP * N;
        if ((n + 255) / 256 > (int64_t)UINT32_MAX)
            return hipErrorInvalidValue;
        hipLaunchKernelGGL(ssd_span_carry_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0,
                           stream, a.sp, a.sp_dec, units, a.n_spans, (int32_t)(kP * N));
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    const int64_t blocks = units * a.n_spans + q.relay_units;
    if (q.relay_units > 0) {
        const int32_t n = (int32_t)q.relay_units + 1; // flags and the fault word
        hipLaunchKernelGGL(ssd_relay_clear_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256),
                           0, stream, q.relay_sync, n);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    if (q.z)
        hipLaunchKernelGGL((ssd_chunk_kernel<T, N, true>), dim3((uint32_t)blocks), dim3(kThreads),
                           0, stream, a);
    else
        hipLaunchKernelGGL((ssd_chunk_kernel<T, N, false>), dim3((uint32_t)blocks),
                           dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

} // namespace

bool ssd_supported(int64_t head_dim, int64_t d_state)
{
    return head_dim == kP && (d_state == 64 || d_state == 128);
}

namespace {
template <typename T, int N>
int64_t block_slots_t(int dev)
{
    int cu = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void *>(ssd_chunk_kernel<T, N, true>), kThreads,
            0) != hipSuccess ||
        cu <= 0 || per_cu <= 0) {
        (void)hipGetLastError(); // do not leave a sticky error behind
        return 0;
    }
    return (int64_t)cu * per_cu;
}

// Per device and kernel variant, queried once (the planner asks on every call).
constexpr int kSlotDevices = 64;
std::atomic<int64_t> g_slots[kSlotDevices][4];
} // namespace

int64_t ssd_block_slots(int64_t d_state, DType dtype)
{
    const bool bf = dtype == DType::BF16;
    if (d_state != 64 && d_state != 128)
        return 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    const int v = (d_state == 128 ? 2 : 0) + (bf ? 1 : 0);
    if (dev >= 0 && dev < kSlotDevices) {
        const int64_t c = g_slots[dev][v].load(std::memory_order_relaxed);
        if (c > 0)
            return c;
    }
    int64_t n = 0;
    switch (v) {
    case 0: n = block_slots_t<float, 64>(dev); break;
    case 1: n = block_slots_t<uint16_t, 64>(dev); break;
    case 2: n = block_slots_t<float, 128>(dev); break;
    default: n = block_slots_t<uint16_t, 128>(dev); break;
    }
    if (n > 0 && dev >= 0 && dev < kSlotDevices)
        g_slots[dev][v].store(n, std::memory_order_relaxed);
    return n;
}

hipError_t launch_ssd(const SsdLaunch &q, hipStream_t stream)
{
    if (q.head_dim != kP)
        return hipErrorInvalidValue;
    const bool bf = q.dtype == DType::BF16;
    switch (q.d_state) {
    case 64: return bf ? launch_ssd_t<uint16_t, 64>(q, stream) : launch_ssd_t<float, 64>(q, stream);
    case 128: return bf ? launch_ssd_t<uint16_t, 128>(q, stream) : launch_ssd_t<float, 128>(q, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace mambascan
