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
//   M[t,s] = S[t,s] exp(cs_t - cs_s) Delta_s  (s <= t, else 0)
//   Y      = M X + diag(exp(cs)) C H_in + D X        (Q x P)
//   H_out  = exp(cs_{Q-1}) H_in + Btil^T X,   Btil[s,n] = B[s,n] exp(cs_{Q-1} - cs_s) Delta_s
// One block per (batch row, head) walks the chunks in order and keeps H in the MFMA
// accumulators (fp32) from chunk to chunk, so nothing of the chunk states goes to HBM.
// The four products use v_mfma_f32_32x32x16_bf16 for bf16 inputs and v_mfma_f32_32x32x2f32
// for fp32 inputs.  With bf16 inputs, X, B and C are exact bf16 values, but M, Btil and
// the copy of H read by C H are computed in fp32: each is split as hi + lo (hi = its bf16
// rounding, lo = the bf16 rounding of the remainder) and enters as two products, which
// keeps about 16 significant bits (a single bf16 operand measured 1.4e-2 relative error in
// y and in the state on a CPU emulation of this arithmetic).  Each wave of the block owns
// one 32 x 32 tile of S and of Y and N/64 tiles of H.  Every operand is read from an LDS matrix stored with
// its contraction index contiguous (rows padded by 16 bytes against bank conflicts).
#include <type_traits>

#include "device_math.h"
#include "scan_common.h"
#include "ssd.h"

namespace mambascan {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kQ = 64;       // chunk length
constexpr int kP = 64;       // head dimension
constexpr int kThreads = 256; // 4 waves

// The MFMA used for an element type, its K, and the LDS element type.
template <typename T> struct Mma;
template <> struct Mma<uint16_t> {
    static constexpr int K = 16;   // contraction per instruction
    static constexpr int KL = 8;   // contiguous k values per lane
    static constexpr int PAD = 8;  // row padding (elements)
    typedef __bf16 E;
    typedef bf16x8 Frag;
    static __device__ __forceinline__ Frag load(const E *p) { return *reinterpret_cast<const Frag *>(p); }
    static __device__ __forceinline__ f32x16 mma(Frag a, Frag b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ E from_float(float v) { return static_cast<__bf16>(v); }
    static __device__ __forceinline__ E from_raw(uint16_t v) { return __builtin_bit_cast(__bf16, v); }
    static __device__ __forceinline__ float to_float(E v) { return static_cast<float>(v); }
    static constexpr bool SPLIT = true; // computed operands as hi + lo
};
template <> struct Mma<float> {
    static constexpr int K = 2;
    static constexpr int KL = 1;
    static constexpr int PAD = 1;
    typedef float E;
    typedef float Frag;
    static __device__ __forceinline__ Frag load(const E *p) { return *p; }
    static __device__ __forceinline__ f32x16 mma(Frag a, Frag b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ E from_float(float v) { return v; }
    static __device__ __forceinline__ E from_raw(float v) { return v; }
    static __device__ __forceinline__ float to_float(E v) { return v; }
    static constexpr bool SPLIT = false;
};

// Store v at hi[i] (and its rounding remainder at lo[i] when operands are split).
template <typename T>
__device__ __forceinline__ void put_split(typename Mma<T>::E *hi, typename Mma<T>::E *lo, int i,
                                          float v)
{
    typedef Mma<T> M;
    const typename M::E h = M::from_float(v);
    hi[i] = h;
    if constexpr (M::SPLIT)
        lo[i] = M::from_float(v - M::to_float(h));
}

// a + b = s + e exactly (Knuth's TwoSum; no reassociation, no FMA is involved).
__device__ __forceinline__ void two_sum(float a, float b, float &s, float &e)
{
    s = a + b;
    const float bb = s - a;
    e = (a - (s - bb)) + (b - bb);
}

// Row and column of accumulator element v of this lane in a 32 x 32 tile.
__device__ __forceinline__ int acc_row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }
__device__ __forceinline__ int acc_col(int lane) { return lane & 31; }

// acc += A B over k in [0, KTOT): A rows [i0, i0+32) of a [.][k] matrix with row stride ra,
// B columns [j0, j0+32) of a [j][k] matrix (stored transposed) with row stride rb.
template <typename T, int KTOT>
__device__ __forceinline__ void tile_mma(f32x16 &acc, const typename Mma<T>::E *a, int ra, int i0,
                                         const typename Mma<T>::E *b, int rb, int j0, int lane)
{
    typedef Mma<T> M;
    const int r = lane & 31, kh = (lane >> 5) * M::KL;
    const typename M::E *pa = a + (i0 + r) * ra + kh;
    const typename M::E *pb = b + (j0 + r) * rb + kh;
#pragma unroll
    for (int k = 0; k < KTOT; k += M::K)
        acc = M::mma(M::load(pa + k), M::load(pb + k), acc);
}

// acc += (A_hi + A_lo) B, or acc += A (B_hi + B_lo): the split side given twice (lo
// ignored when operands are not split).
template <typename T, int KTOT>
__device__ __forceinline__ void tile_mma_split_a(f32x16 &acc, const typename Mma<T>::E *ahi,
                                                 const typename Mma<T>::E *alo, int ra, int i0,
                                                 const typename Mma<T>::E *b, int rb, int j0,
                                                 int lane)
{
    tile_mma<T, KTOT>(acc, ahi, ra, i0, b, rb, j0, lane);
    if constexpr (Mma<T>::SPLIT)
        tile_mma<T, KTOT>(acc, alo, ra, i0, b, rb, j0, lane);
}

template <typename T, int KTOT>
__device__ __forceinline__ void tile_mma_split_b(f32x16 &acc, const typename Mma<T>::E *a,
                                                 int ra, int i0, const typename Mma<T>::E *bhi,
                                                 const typename Mma<T>::E *blo, int rb, int j0,
                                                 int lane)
{
    tile_mma<T, KTOT>(acc, a, ra, i0, bhi, rb, j0, lane);
    if constexpr (Mma<T>::SPLIT)
        tile_mma<T, KTOT>(acc, a, ra, i0, blo, rb, j0, lane);
}

struct SsdArgs {
    const void *x, *dt, *B, *C, *z;
    const float *A, *D, *dt_bias, *h0;
    void *y;
    float *h_last;
    int64_t L;
    int32_t H; // heads
};

template <typename T, int N, bool GATED>
__global__ void __launch_bounds__(kThreads)
ssd_chunk_kernel(SsdArgs p)
{
    typedef Mma<T> M;
    typedef typename M::E E;
    constexpr int Q = kQ, P = kP;
    constexpr int RQ = Q + M::PAD, RN = N + M::PAD; // row strides
    constexpr int HT = N / 64;                       // H tiles per wave (N/32 x 2 tiles / 4 waves)
    static_assert(N % 64 == 0 && Q == 64 && P == 64, "shape");

    // LDS: X^T [P][RQ]; B [Q][RN], then M [Q][RQ] (hi, lo) in the same place; C [Q][RN];
    // Btil^T [N][RQ] (hi, lo); H^T [P][RN] (hi, lo); cumulative decay and Delta per step.
    constexpr int NS = M::SPLIT ? 2 : 1;
    constexpr int BM = Q * RN > NS * Q * RQ ? Q * RN : NS * Q * RQ;
    __shared__ __attribute__((aligned(16))) E s_xt[P * RQ];
    __shared__ __attribute__((aligned(16))) E s_bm[BM];
    __shared__ __attribute__((aligned(16))) E s_c[Q * RN];
    __shared__ __attribute__((aligned(16))) E s_bt[NS * N * RQ];
    __shared__ __attribute__((aligned(16))) E s_ht[NS * P * RN];
    // cumulative decay cs = cs_hi + cs_lo (a compensated sum: the weights use differences
    // cs_t - cs_s, which a plain fp32 sum would lose when |cs| is large), Delta per step
    __shared__ float s_cs[Q], s_csl[Q], s_dl[Q];
    E *const s_ml = s_bm + (NS - 1) * Q * RQ;     // lo parts (alias the hi arrays when unsplit)
    E *const s_btl = s_bt + (NS - 1) * N * RQ;
    E *const s_htl = s_ht + (NS - 1) * P * RN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bh = blockIdx.x;
    const int b = bh / p.H, h = bh % p.H;
    const int64_t L = p.L;
    const int64_t Dn = (int64_t)p.H * P;

    const T *xg = (const T *)p.x + (int64_t)b * L * Dn + (int64_t)h * P;
    const T *zg = GATED ? (const T *)p.z + (int64_t)b * L * Dn + (int64_t)h * P : nullptr;
    T *yg = (T *)p.y + (int64_t)b * L * Dn + (int64_t)h * P;
    const T *bg = (const T *)p.B + (int64_t)b * L * N;
    const T *cg = (const T *)p.C + (int64_t)b * L * N;
    const T *dtg = (const T *)p.dt + (int64_t)b * L * p.H + h;
    const float a2 = p.A[h] * kLog2e;
    const float dtb = p.dt_bias ? p.dt_bias[h] : 0.0f;
    const float Dh = p.D ? p.D[h] : 0.0f;

    // state tiles of this wave: tile tau = w * HT + m -> rows 32 (tau / 2) (n), cols 32 (tau % 2) (p)
    f32x16 hacc[HT];
    const float *h0 = p.h0 ? p.h0 + ((int64_t)b * Dn + (int64_t)h * P) * N : nullptr;
#pragma unroll
    for (int m = 0; m < HT; ++m) {
        const int tau = w * HT + m, n0 = 32 * (tau >> 1), p0 = 32 * (tau & 1);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int n = n0 + acc_row(v, lane), pc = p0 + acc_col(lane);
            const float hv = h0 ? h0[(int64_t)pc * N + n] : 0.0f;
            hacc[m][v] = hv;
            put_split<T>(s_ht, s_htl, pc * RN + n, hv);
        }
    }

    const int ti0 = 32 * (w >> 1), tj0 = 32 * (w & 1); // this wave's tile of S and Y
    for (int64_t t0 = 0; t0 < L; t0 += Q) {
        const int nt = (int)min((int64_t)Q, L - t0);
        // ---- load the chunk: X^T, B, C; Delta and the cumulative decay ----
        for (int e = tid; e < Q * P; e += kThreads) {
            const int t = e / P, pc = e % P;
            s_xt[pc * RQ + t] = t < nt ? M::from_raw(xg[(t0 + t) * Dn + pc]) : M::from_float(0.0f);
        }
        for (int e = tid; e < Q * N; e += kThreads) {
            const int t = e / N, n = e % N;
            const bool ok = t < nt;
            s_bm[t * RN + n] = ok ? M::from_raw(bg[(t0 + t) * N + n]) : M::from_float(0.0f);
            s_c[t * RN + n] = ok ? M::from_raw(cg[(t0 + t) * N + n]) : M::from_float(0.0f);
        }
        if (w == 0) {
            const int t = lane;
            const float dl = t < nt ? softplus_f(load_val(dtg, (t0 + t) * p.H) + dtb) : 0.0f;
            float cs = dl * a2, csl = 0.0f;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) { // inclusive prefix sum over the 64 steps
                const float vh = __shfl_up(cs, o, 64), vl = __shfl_up(csl, o, 64);
                if (lane >= o) {
                    float sh, e;
                    two_sum(cs, vh, sh, e);
                    const float l = csl + vl + e;
                    cs = sh + l;               // renormalise (|sh| >= |l|)
                    csl = l - (cs - sh);
                }
            }
            s_cs[t] = cs;
            s_csl[t] = csl;
            s_dl[t] = dl;
        }
        __syncthreads();

        // ---- S = C B^T (this wave's tile), the weights of M; Btil^T ----
        f32x16 sacc = {};
        tile_mma<T, N>(sacc, s_c, RN, ti0, s_bm, RN, tj0, lane);
        float mv[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int i = ti0 + acc_row(v, lane), j = tj0 + acc_col(lane);
            mv[v] = j <= i ? sacc[v] * hw_exp2((s_cs[i] - s_cs[j]) + (s_csl[i] - s_csl[j])) * s_dl[j]
                           : 0.0f;
        }
        const float cs_end = s_cs[Q - 1], cs_endl = s_csl[Q - 1];
        for (int e = tid; e < Q * N; e += kThreads) {
            const int t = e % Q, n = e / Q;
            const float wgt = hw_exp2((cs_end - s_cs[t]) + (cs_endl - s_csl[t])) * s_dl[t];
            put_split<T>(s_bt, s_btl, n * RQ + t, M::to_float(s_bm[t * RN + n]) * wgt);
        }
        __syncthreads(); // B is no longer read: M takes its place
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int i = ti0 + acc_row(v, lane), j = tj0 + acc_col(lane);
            put_split<T>(s_bm, s_ml, i * RQ + j, mv[v]);
        }
        __syncthreads();

        // ---- Y = M X + diag(exp(cs)) C H_in + D X, gate, store ----
        f32x16 yacc = {}, oacc = {};
        tile_mma_split_a<T, Q>(yacc, s_bm, s_ml, RQ, ti0, s_xt, RQ, tj0, lane);
        tile_mma_split_b<T, N>(oacc, s_c, RN, ti0, s_ht, s_htl, RN, tj0, lane);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int i = ti0 + acc_row(v, lane), pc = tj0 + acc_col(lane);
            if (i < nt) {
                const float xv = M::to_float(s_xt[pc * RQ + i]);
                float yv = yacc[v] + hw_exp2(s_cs[i] + s_csl[i]) * oacc[v] + Dh * xv;
                if (GATED)
                    yv *= silu_f(load_val(zg, (t0 + i) * Dn + pc));
                store_val(yg, (t0 + i) * Dn + pc, yv);
            }
        }

        // ---- H_out = exp(cs_end) H_in + Btil^T X ----
        const float dec = hw_exp2(cs_end + cs_endl);
#pragma unroll
        for (int m = 0; m < HT; ++m) {
            const int tau = w * HT + m;
#pragma unroll
            for (int v = 0; v < 16; ++v)
                hacc[m][v] *= dec;
            tile_mma_split_a<T, Q>(hacc[m], s_bt, s_btl, RQ, 32 * (tau >> 1), s_xt, RQ,
                                   32 * (tau & 1), lane);
        }
        __syncthreads(); // every wave has read H_in (and X, C, M, Btil)
#pragma unroll
        for (int m = 0; m < HT; ++m) {
            const int tau = w * HT + m, n0 = 32 * (tau >> 1), p0 = 32 * (tau & 1);
#pragma unroll
            for (int v = 0; v < 16; ++v)
                put_split<T>(s_ht, s_htl, (p0 + acc_col(lane)) * RN + n0 + acc_row(v, lane),
                             hacc[m][v]);
        }
    }

    if (p.h_last) {
        float *hl = p.h_last + ((int64_t)b * Dn + (int64_t)h * P) * N;
#pragma unroll
        for (int m = 0; m < HT; ++m) {
            const int tau = w * HT + m, n0 = 32 * (tau >> 1), p0 = 32 * (tau & 1);
#pragma unroll
            for (int v = 0; v < 16; ++v)
                hl[(int64_t)(p0 + acc_col(lane)) * N + n0 + acc_row(v, lane)] = hacc[m][v];
        }
    }
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
    const int64_t blocks = q.batch * q.n_heads;
    if (blocks <= 0)
        return hipSuccess;
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
