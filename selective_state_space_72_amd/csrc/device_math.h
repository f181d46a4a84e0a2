// Device-side scalar helpers for the scan kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mambascan {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// --- storage formats --------------------------------------------------------

__device__ __forceinline__ float load_val(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_val(const uint16_t *p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16); // bf16 -> f32 is exact
}
__device__ __forceinline__ float widen(float x) { return x; }
__device__ __forceinline__ float widen(uint16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

__device__ __forceinline__ void store_val(float *p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_val(uint16_t *p, int64_t i, float v) {
    // round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
    p[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

// --- transcendental pieces ----------------------------------------------------
// v_exp_f32 / v_log_f32 compute 2^x and log2(x) directly.

__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(v) = log(1 + e^v) = max(v, 0) + log1p(e^-|v|).
// log1p(e) for e in (0, 1] is evaluated as log(s) - ((s - 1) - e) with
// s = fl(1 + e): (s - 1) - e is exactly the rounding error of 1 + e, and the
// first-order correction log(1 + e) = log(s) - ((s - 1) - e) / s + O(err^2)
// keeps the relative error near one ulp even when 1 + e rounds to 1 (where the
// plain log(1 + e) would return 0 instead of about e).
__device__ __forceinline__ float softplus_f(float v) {
    const float e = hw_exp2(-__builtin_fabsf(v) * kLog2e);
    const float s = 1.0f + e;
    const float err = (s - 1.0f) - e;
    const float l = __builtin_fmaf(hw_log2(s), kLn2, -err);
    return __builtin_fmaxf(v, 0.0f) + l;
}

// softplus for activations of element type T.  bf16 (uint16_t): the same formula without
// the compensation term, max(v, 0) + log2(fl(1 + e)) ln 2 as one FMA: the rounding of 1 + e
// and v_log_f32 leave an absolute error near 1e-7 in Delta (relative 1e-4 at Delta = 1e-3),
// more than ten times below what the bf16 rounding of delta itself moves Delta by
// (sigmoid(v) |delta| 2^-9); it saves three VALU operations per channel-step.  fp32
// activations keep softplus_f (1.9e-6 relative).
template <typename T>
__device__ __forceinline__ float softplus_act(float v) {
    if constexpr (sizeof(T) == 2) {
        const float e = hw_exp2(-__builtin_fabsf(v) * kLog2e);
        return __builtin_fmaf(hw_log2(1.0f + e), kLn2, __builtin_fmaxf(v, 0.0f));
    } else {
        return softplus_f(v);
    }
}

// v + v of lane ^ 16, then + the same of lane ^ 32: the sum over the four lanes l % 16
// (every lane gets it, in the same order).  v_permlane16_swap / v_permlane32_swap given
// two copies of v exchange rows 0 <-> 1 and 2 <-> 3, resp. the wave's halves, between
// them, so the two results hold v of the lane and of its partner.
__device__ __forceinline__ float lane_pair_sum(float v)
{
    const uint32_t x = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    const float a = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    const uint32_t y = __float_as_uint(a);
    const auto r2 = __builtin_amdgcn_permlane32_swap(y, y, false, false);
    return __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
}

// Decay factor of one recurrence step, exp(Delta * A) = 2^(Delta * A'), A' = A log2(e).
// v_exp_f32 rounds results just below 1 downward more often than to nearest: against a
// correctly rounded exp2 its mean relative error is about -7e-9 for arguments in
// (-1e-3, 0) and -4.5e-9 in (-1e-2, 0) (measured on gfx950 over 4M arguments per range).
// A state with a long memory multiplies about 1/|x| such factors, so the bias adds up to
// ~1e-5 relative after 1000 steps.  Shifting the argument by 8e-9 (a relative change of
// 5.5e-9 in the result) cancels most of it where it matters; for larger |x| the shift is
// below the argument's rounding unit or acts on short memories only.  It costs nothing:
// the multiply becomes an FMA.
constexpr float kExp2Shift = 8.0e-9f;
__device__ __forceinline__ float decay_exp2(float dt, float a2) {
    return hw_exp2(__builtin_fmaf(dt, a2, kExp2Shift));
}

// Zero-order-hold input term of one step, Bbar u / B = (exp(Delta A) - 1) / A * u
// = Delta u * phi(x) with x = Delta A and phi(x) = expm1(x) / x (phi(0) = 1, so A = 0
// gives Euler's Delta u).  For |x| < 1/16, phi comes from its series through x^3
// (truncation below 1.3e-7 relative); otherwise from the decay factor already at hand,
// abar * (u / A) - u / A in one FMA, where the cancellation in abar - 1 costs at most ~1e-6
// relative.  du = Delta u, u_over_a = u / A.  Both branches are evaluated (lanes mix them):
// 4 + 1 operations and a select.
__device__ __forceinline__ float zoh_input(float x, float abar, float du, float u_over_a) {
    const float p =
        __builtin_fmaf(x, __builtin_fmaf(x, __builtin_fmaf(x, 1.0f / 24.0f, 1.0f / 6.0f), 0.5f),
                       1.0f);
    const float small = du * p;
    const float large = __builtin_fmaf(abar, u_over_a, -u_over_a);
    return __builtin_fabsf(x) < 0.0625f ? small : large;
}

// zoh_input with the argument in base 2, xb = Delta A log2(e) (the decay factor's exp2
// argument, shift included): x = xb ln 2, so the series' coefficients carry the powers of
// ln 2 and the switch is at |xb| = 1 / (16 ln 2).  Saves the multiply that forms x; the
// shift moves x by 5.5e-9, and phi(x) by less than 3e-9.
__device__ __forceinline__ float zoh_input_b2(float xb, float abar, float du, float u_over_a) {
    constexpr float c1 = 0.34657359027997264f;  // ln 2 / 2
    constexpr float c2 = 0.08007550231970024f;  // (ln 2)^2 / 6
    constexpr float c3 = 0.013876027166205393f; // (ln 2)^3 / 24
    const float p = __builtin_fmaf(xb, __builtin_fmaf(xb, __builtin_fmaf(xb, c3, c2), c1), 1.0f);
    const float small = du * p;
    const float large = __builtin_fmaf(abar, u_over_a, -u_over_a);
    return __builtin_fabsf(xb) < 0.09016844005556021f ? small : large;
}

// sin and cos of x: reduction x = j pi/2 + r with the three-part constant of Cody and
// Waite (pi/2 = C1 + C2 + C3, C1 with 8 significant bits; each part removed with one FMA),
// then the single-precision minimax polynomials of S. Moshier's Cephes library for sin and
// cos on |r| <= pi/4, and the quadrant j mod 4.  Absolute error below 1.6 * 2^-24 for
// |x| <= 3e4 (checked in float32 emulation against float64 on 2e6 angles per range); NaN for
// infinite or NaN x.  About 21 operations, against some 40 and a branch for sincosf.
__device__ __forceinline__ void sincos_fast(float x, float &sn, float &cs) {
    const float j = __builtin_rintf(x * 0.636619772367581343f);
    float r = __builtin_fmaf(-j, 1.5703125f, x);
    r = __builtin_fmaf(-j, 4.837512969970703125e-4f, r);
    r = __builtin_fmaf(-j, 7.54978995489188216e-8f, r);
    const float z = r * r;
    float ps = __builtin_fmaf(z, -1.9515295891e-4f, 8.3321608736e-3f);
    ps = __builtin_fmaf(z, ps, -1.6666654611e-1f) * z;
    const float s = __builtin_fmaf(r, ps, r);
    float pc = __builtin_fmaf(z, 2.443315711809948e-5f, -1.388731625493765e-3f);
    pc = __builtin_fmaf(z, pc, 4.166664568298827e-2f) * z;
    const float c = __builtin_fmaf(z, pc, __builtin_fmaf(-0.5f, z, 1.0f));
    const int q = (int)j;
    const float s1 = (q & 1) ? c : s, c1 = (q & 1) ? s : c;
    sn = __int_as_float(__float_as_int(s1) ^ ((q & 2) << 30));
    cs = __int_as_float(__float_as_int(c1) ^ (((q + 1) & 2) << 30));
}

// Rotation of a state pair: (x, w) <- (cos phi x - sin phi w, sin phi x + cos phi w), given
// (sin phi, cos phi) (turn_pair) or the angle phi (rotate_pair, with sincos_fast: accurate to
// about 1.5 * 2^-24, not the hardware v_sin/v_cos approximation).
__device__ __forceinline__ void turn_pair(float sn, float cs, float &x, float &w) {
    const float nx = __builtin_fmaf(cs, x, -sn * w);
    const float nw = __builtin_fmaf(sn, x, cs * w);
    x = nx;
    w = nw;
}
__device__ __forceinline__ void rotate_pair(float phi, float &x, float &w) {
    float sn, cs;
    sincos_fast(phi, sn, cs);
    turn_pair(sn, cs, x, w);
}

// sin and cos of x by the hardware's v_sin_f32 / v_cos_f32 (argument in revolutions, so x is
// first divided by 2 pi): two transcendental instructions and a multiply instead of the ~21
// operations of sincos_fast.  Absolute error measured on gfx950 against double over 4M
// angles per range: 1.4e-7 for |x| <= 1, 3.9e-7 for |x| <= 4, 1.5e-6 for |x| <= 20 (the
// rounding of x / 2 pi; it grows with |x|).  Used for bf16 activations, whose outputs carry
// 4e-3 relative rounding; fp32 activations keep sincos_fast.
__device__ __forceinline__ void sincos_hw(float x, float &sn, float &cs) {
    const float r = x * 0.159154943091895336f;
    sn = __builtin_amdgcn_sinf(r);
    cs = __builtin_amdgcn_cosf(r);
}
// The sine and cosine for activations of element type T (uint16_t: bf16).
template <typename T>
__device__ __forceinline__ void sincos_act(float x, float &sn, float &cs) {
    if constexpr (sizeof(T) == 2)
        sincos_hw(x, sn, cs);
    else
        sincos_fast(x, sn, cs);
}
// The same from an angle staged for element type T: bf16 activations stage the rotation
// rate already divided by 2 pi, so phi_st is in revolutions and goes to v_sin_f32 /
// v_cos_f32 without the multiply; fp32 activations stage the rate as given.
constexpr float kInv2Pi = 0.159154943091895336f;
template <typename T>
__device__ __forceinline__ void sincos_staged(float phi_st, float &sn, float &cs) {
    if constexpr (sizeof(T) == 2) {
        sn = __builtin_amdgcn_sinf(phi_st);
        cs = __builtin_amdgcn_cosf(phi_st);
    } else {
        sincos_fast(phi_st, sn, cs);
    }
}

template <typename T>
__device__ __forceinline__ void rotate_pair_act(float phi, float &x, float &w) {
    float sn, cs;
    sincos_act<T>(phi, sn, cs);
    turn_pair(sn, cs, x, w);
}

// silu(z) = z * sigmoid(z) = z / (1 + e^-z); e^-z = +inf gives -0 as the limit.
__device__ __forceinline__ float silu_f(float z) {
    return z * hw_rcp(1.0f + hw_exp2(-z * kLog2e));
}

} // namespace mambascan
