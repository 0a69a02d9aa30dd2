// Exact fp32 building blocks for gfx950, used by the codec and step kernels.
//
// Every function here returns the same bits as the correctly rounded IEEE
// operation it replaces, over the stated domain.  The domains were checked
// exhaustively on gfx950 against the compiler's correctly rounded division
// and sqrt (tests/hip/fastmath_check.hip, run by the GPU test suite):
//   recip_cr       every fp32 significand, every positive finite fp16 value;
//   div_by_recip   every fp16 divisor significand x every fp32 dividend
//                  significand (2^33 pairs);
//   softsign       every y in [-1.5, 1.5];
//   sqrt_cr        every x in [0, 2^64) (and sqrt_x2p32_zero_tiny against it);
//   sqrt_quot_x2p32  every v with fl(v / b) in [2^-126, 2^63), for the bias
//                  correction divisors b of eight betas, and v = 0;
//   byte_u8        every fp32 pattern (v_cvt_pk_u8_f32 == clamp(rint(x), 0, 255),
//                  NaN -> 0);
//   div_markstein  2^32 random pairs of its stated domain plus every divisor
//                  significand at the domain's edges;
//   div_markstein with a bias correction as divisor  every dividend
//                  significand (both signs, hashed exponents over the step's
//                  range) x a set of bias-correction and random divisors;
//   code_s8_magic  every fp32 p (low byte == clamp(rint(p), -127, 127) as a
//                  two's-complement byte, for non-NaN p);
//   softsign_code_bytes  (not exact itself: two-sided) 4095 fp16 divisors x
//                  4096 dividends around each of the 127 code boundaries, and
//                  2^18 random dividends each: wherever its two bytes agree,
//                  the byte is the correctly rounded chain's code (and the
//                  sweep reaches inputs where the bytes disagree).
// Only fma, mul, add, v_rcp_f32 / v_rsq_f32, fp32 <-> fp64 conversions, an
// fp64 fma and integer ops are used, so the results do not depend on the
// FP mode beyond round-to-nearest-even with fp32 and fp64 denormals kept.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flashopt {
namespace math {

// Correctly rounded 1/d for d and 1/d normal: hardware reciprocal (1 ulp)
// refined by one Newton step on the residual.
__device__ __forceinline__ float recip_cr(float d)
{
    const float r0 = __builtin_amdgcn_rcpf(d);
    const float e = __builtin_fmaf(-d, r0, 1.0f);
    return __builtin_fmaf(e, r0, r0);
}

// Correctly rounded a/d given r = recip_cr(d) (Markstein's correction:
// q0 = a r, then one FMA residual step).  Exact whenever a/d is normal and
// the residual a - q0 d does not underflow, i.e. for |a/d| >= 2^-100 with
// d an fp16 scale; smaller quotients may be off by one unit, which cannot
// change an 8-bit code (they round to code 0 either way).
__device__ __forceinline__ float div_by_recip(float a, float d, float r)
{
    const float q0 = a * r;
    const float rem = __builtin_fmaf(-q0, d, a);
    return __builtin_fmaf(rem, r, q0);
}

// Softsign companding (2y) / (1 + |y|), correctly rounded for |y| <= 1.5
// (group quotients never exceed 1.5: the fp16 scale is at least 2/3 of the
// group max).  It runs the unrefined-reciprocal Markstein step on the
// halved operands y / ((1 + |y|) / 2): halving is exact, the hardware
// reciprocal of the halved denominator is exactly twice the reciprocal of the
// full one, so every product and residual is the full-size one scaled by an
// exact power of two and the result is bit-identical, one multiply cheaper.
// A zero input returns +0 (the code is 0 either way).
__device__ __forceinline__ float softsign(float y)
{
    const float hden = __builtin_fmaf(fabsf(y), 0.5f, 0.5f);   // (1 + |y|) / 2, exact
    const float r2 = __builtin_amdgcn_rcpf(hden);               // 2 / (1 + |y|), approx.
    const float q0 = y * r2;
    const float rem = __builtin_fmaf(-q0, hden, y);
    return __builtin_fmaf(rem, r2, q0);
}

// Correctly rounded num / den given r = recip_cr(den) (one Markstein residual
// step, with the residual taken as q0 den - num so that a zero numerator keeps
// its sign), for den in [2^-100, 2^100] and num either zero or with
// max(2^-102, 2^-126 den) <= |num| <= 2^100 den: then the residual is exact
// (|num| >= 2^-102) and the quotient is a normal number, which is what
// Markstein's theorem needs.  Callers route other numerators to the generic
// division.
__device__ __forceinline__ float div_markstein(float num, float den, float r)
{
    const float q0 = num * r;
    const float e = __builtin_fmaf(q0, den, -num);
    return __builtin_fmaf(-e, r, q0);
}

// Signed 8-bit code of p = y * 127 in the low byte of the result: clamp to
// [-127, 127] (v_med3_f32), then adding 1.5 * 2^23 rounds to an integer with
// ties to even (the sum lies in [2^23, 2^24), where the fp32 spacing is 1).
// The pattern of 1.5 * 2^23 has a zero low byte, so the sum's low byte is
// rint(p) modulo 256: the code's two's-complement byte.  NaN inputs are the
// caller's to route elsewhere.
__device__ __forceinline__ uint32_t code_s8_magic(float p)
{
    const float c = __builtin_amdgcn_fmed3f(p, -127.0f, 127.0f);
    return __float_as_uint(c + 12582912.0f);
}

// 1/254 rounded to fp32 (relative error 2^-28).
constexpr float kInv254 = 0x1.020408p-8f;

// v_cvt_pk_u8_f32 into byte I of acc: clamp(rint(x), 0, 255) with ties to
// even, NaN -> 0.
template <int I>
__device__ __forceinline__ uint32_t cvt_u8(float x, uint32_t acc)
{
    return __builtin_amdgcn_cvt_pk_u8_f32(x, I, acc);
}

// Half-width, in code units, of the band around the fast momentum code's p
// that softsign_code_bytes evaluates.
constexpr float kMomentumBand = 1e-4f;

// The companded int8 momentum codes of four finite values m of one group with
// divisor d, without the correctly rounded chain y = m / d, y'' = 2y /
// (1 + |y|), p = 127 y''.  In exact arithmetic p = 254 m / (d + |m|); here
// p = m rcp(t) with t = fma(|m|, 1/254, c0) and c0 = d kInv254 (formed once
// per group), whose relative error is at most 4.1 units of 2^-24 (kInv254, c0,
// the fma, v_rcp_f32's one ulp), against at most 4 for the chain (four
// roundings, none amplified: d y''/dy y / y'' <= 1): the two differ by less
// than 8.1 2^-24 127.5 < 6.2e-5 wherever a code can depend on it.  Each code
// is converted twice, from fma(m, rcp(t), 128 + kMomentumBand) into `hi` and
// from fma(m, rcp(t), 128 - kMomentumBand) into `lo` (byte i, round half to
// even, clamped to [0, 255]); each fma adds at most half an ulp below 256
// (2^-17).  Where the two bytes agree, no rounding boundary lies within
// 1e-4 - 2^-17 > 6.2e-5 of p, so the byte is the chain's code plus 128.  The
// caller needs |m / d| <= 1 + 2^-11 (true for a normal fp16 scale of the
// group's maximum), so that |p| < 127.5 and no clamp is needed.
__device__ __forceinline__ void softsign_code_bytes(float m0, float m1, float m2, float m3, float c0,
                                                    uint32_t &hi, uint32_t &lo)
{
    const float r0 = __builtin_amdgcn_rcpf(__builtin_fmaf(fabsf(m0), kInv254, c0));
    const float r1 = __builtin_amdgcn_rcpf(__builtin_fmaf(fabsf(m1), kInv254, c0));
    const float r2 = __builtin_amdgcn_rcpf(__builtin_fmaf(fabsf(m2), kInv254, c0));
    const float r3 = __builtin_amdgcn_rcpf(__builtin_fmaf(fabsf(m3), kInv254, c0));
    constexpr float up = 128.0f + kMomentumBand, dn = 128.0f - kMomentumBand;
    hi = cvt_u8<0>(__builtin_fmaf(m0, r0, up), 0u);
    lo = cvt_u8<0>(__builtin_fmaf(m0, r0, dn), 0u);
    hi = cvt_u8<1>(__builtin_fmaf(m1, r1, up), hi);
    lo = cvt_u8<1>(__builtin_fmaf(m1, r1, dn), lo);
    hi = cvt_u8<2>(__builtin_fmaf(m2, r2, up), hi);
    lo = cvt_u8<2>(__builtin_fmaf(m2, r2, dn), lo);
    hi = cvt_u8<3>(__builtin_fmaf(m3, r3, up), hi);
    lo = cvt_u8<3>(__builtin_fmaf(m3, r3, dn), lo);
}

// Half-width, in code units, of the band around the variance code's p that
// the step evaluates when it forms the codes from sqrt(vhat) (see
// flashopt_kernels.hip, variance_codes).
constexpr float kVarianceBand = 1.5e-4f;

// 2^32 times the correctly rounded sqrt(x), for 0 <= x < 2^64: the input is
// scaled by 2^64 (exact), which puts every denormal into the range where one
// residual correction of x * rsq(x) is exact, and sqrt(x 2^64) = sqrt(x) 2^32
// exactly.  rsq(0) = inf is clamped so that the result for 0 is 0.  Callers
// that can fold the factor 2^32 into later exact power-of-two scalings use
// this form; sqrt_cr applies it.
__device__ __forceinline__ float sqrt_cr_x2p32(float x)
{
    const float xs = x * 0x1p64f;
    const float y = fminf(__builtin_amdgcn_rsqf(xs), 0x1.fffffep127f);
    const float s = xs * y;
    const float h = 0.5f * y;
    const float r = __builtin_fmaf(-s, s, xs);
    return __builtin_fmaf(r, h, s);
}

// sqrt_cr_x2p32 without the clamp, for the step: the input is scaled as
// fma(x, 2^64, 2^-126).  For every x > 0 the added 2^-126 vanishes (x 2^64 >=
// 2^-85, whose half ulp is 2^-109), so the result is sqrt_cr_x2p32(x); at
// x = 0 it keeps rsq finite and the result is 2^-63 instead of 0.  A caller
// has to absorb that value: the step adds it to eps 2^32 >= 2^-6 (the short
// route needs eps >= 2^-38), whose half ulp is at least 2^-30, so the sum is
// eps 2^32 itself; its variance code and group scale round to 0 as for 0.
__device__ __forceinline__ float sqrt_x2p32_zero_tiny(float x)
{
    const float xs = __builtin_fmaf(x, 0x1p64f, 0x1p-126f);
    const float y = __builtin_amdgcn_rsqf(xs);
    const float s = xs * y;
    const float h = 0.5f * y;
    const float r = __builtin_fmaf(-s, s, xs);
    return __builtin_fmaf(r, h, s);
}

// 2^32 sqrt(q) for q = fl(v / b), the correctly rounded fp32 quotient of
// v >= 0 by an fp32 b > 0, given inv_s = 2^64 / b rounded to double.  The
// quotient and the 2^64 input scaling of sqrt_cr_x2p32 come out of one fp64
// fma: xs = fl(v inv_s + 2^-126).  Where q is normal, v inv_s >= 2^-62, so
// the added 2^-126 moves it by at most 2^-64 relative and the double result
// lies within 2^-51.9 + 2^-64 relative of the scaled quotient.  No quotient
// of two fp32 numbers lies that close to an fp32 rounding boundary without
// being on it (for a midpoint M of the result's binade, v - b M is a nonzero
// multiple of ulp(b) ulp(M) / 2, so |v / b - M| > 2^-25 ulp(M) >= 2^-49
// |v / b|), and none lies on one (b M would need 25 significant bits), so
// rounding to fp32 gives xs = q 2^64 exactly.  Where
// q is subnormal or zero, xs <= 2^-62 (2^-126 for v = 0, a normal number,
// which keeps v_rsq_f32 finite: it flushes subnormal inputs) and the result
// is below 2^-31 rather than q's exact root.  Domain: q < 2^63.
// OPAQUE: the (exact) conversion of v to fp64 is written as inline
// assembly, which the compiler neither merges with nor moves across other
// code; the arithmetic is the same.
template <bool OPAQUE = false>
__device__ __forceinline__ float sqrt_quot_x2p32(float v, double inv_s)
{
    double vd;
    if (OPAQUE) asm("v_cvt_f64_f32 %0, %1" : "=v"(vd) : "v"(v));
    else vd = static_cast<double>(v);
    const float xs = static_cast<float>(__builtin_fma(vd, inv_s, 0x1p-126));
    const float y = __builtin_amdgcn_rsqf(xs);
    const float s = xs * y;
    const float h = 0.5f * y;
    const float r = __builtin_fmaf(-s, s, xs);
    return __builtin_fmaf(r, h, s);
}

// Correctly rounded sqrt(x) for 0 <= x < 2^64 (the scaling back by 2^-32 is
// exact: the results are normal).
__device__ __forceinline__ float sqrt_cr(float x)
{
    return sqrt_cr_x2p32(x) * 0x1p-32f;
}

// v_cvt_i32_f32: truncation toward zero, saturating, NaN -> 0.
__device__ __forceinline__ int32_t cvt_i32(float x)
{
    int32_t r;
    asm("v_cvt_i32_f32 %0, %1" : "=v"(r) : "v"(x));
    return r;
}

// Clamp to [lo, hi] (v_med3_i32 after instruction selection).
__device__ __forceinline__ int32_t clamp_i32(int32_t x, int32_t lo, int32_t hi)
{
    return x < lo ? lo : (x > hi ? hi : x);
}

}  // namespace math
}  // namespace flashopt
