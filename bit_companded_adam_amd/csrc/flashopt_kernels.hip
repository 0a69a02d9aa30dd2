// HIP kernels of libflashopt.so for gfx950 (MI355X): the group-32 state codec,
// the bf16 + rho weight split, and the fused FlashAdamW and FlashSGD steps.
//
// Method pages: "code/flashsim/quantization.py" (Alg. 2/3: quantize(),
// dequantize()), "code/flashsim/flash_adamw_sim.py" (Alg. 4:
// FlashAdamWSim.step(), bytes_per_param), "code/gpu/equivalence.py" (bf16
// parameter and correction bits, eq_ecc()).
//
// Layout of the work: tensors are cut into 1024-element chunks, each lane
// taking 16 elements of a chunk as units of N consecutive elements placed so
// that every memory instruction of a wavefront covers one contiguous block
// of each stream (unit u of lane l starts at element 64 N u + N l).  The
// codec kernels give a wavefront a whole chunk; the split and step kernels
// give it one unit of one chunk (the multi-tensor steps renumber their
// workgroups so that each XCD streams one contiguous region).  The
// quantized steps use N = 8 (a lane quad owns a 32-element group; its
// maximum takes two DPP exchanges); fp32 states and the codec and split
// kernels use N = 4 (quantize's group maximum spans 8 lanes).  The path is
// elementwise, so there is no MFMA; LDS holds only the two 256-entry
// dequantization tables (built per workgroup), and the list steps' scalar
// block and per-tensor chunk table are read with scalar loads.  A tensor's
// quantized state is five streams (rho, m codes, v codes, m scales, v
// scales) or, in the blocked layout, one buffer of per-chunk blocks that
// holds the same five parts; chunk_ptrs resolves either, with scalar
// arithmetic, so the per-element code is the same.
//
// Arithmetic: fp32, one IEEE rounding per operation in the written order
// (built with -ffp-contract=off, fp32 and fp16 denormals preserved), so the
// results match a plain CPU evaluation bit for bit.  The update follows the
// operation order FlashAdamWSim.step prints: the bias-correction quotients
// use host-computed reciprocals (a Markstein step for m / bc1, one fp64 fma
// for v / bc2, both exact), and division by a group scale, the softsign
// division, the update division, the sqrt and the byte conversions use the
// exact short sequences of flashopt_math.h instead of the generic correctly
// rounded expansions.
// The momentum and variance codes use two-sided short forms; a word whose two
// evaluations disagree falls back to the correctly rounded chain.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <mutex>

#include "flashopt.h"
#include "flashopt_internal.h"
#include "flashopt_math.h"

namespace flashopt {
namespace {

// ----------------------------------------------------------------- helpers

// math::sqrt_cr is exact for the bit patterns [0, 0x5F800000): +0 up to
// below 2^64.  Negative values (sign bit), infinities and NaNs all compare
// at or above this bound as unsigned patterns.
constexpr uint32_t kSqrtFastEnd = 0x5F800000u;

// bf16 halves of a 32-bit word holding two consecutive elements
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> binary16 bits: v_cvt_f16_f32, round to nearest even, subnormals
// kept, overflow to infinity.
__device__ __forceinline__ uint32_t f16_bits(float x)
{
    const _Float16 h = static_cast<_Float16>(x);
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_value(uint32_t bits)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

// The divisor of a group: 1 when the stored scale is zero (either sign),
// else the scale itself, as quantize() divides by 1 for a zero scale.
__device__ __forceinline__ float group_divisor(uint32_t s)
{
    return (s & 0x7FFFu) ? f16_value(s) : 1.0f;
}

// Maximum over aligned groups of G lanes (G = 2, 4 or 8): v_max_f32 with a
// DPP source, quad_perm [1, 0, 3, 2] (lane ^ 1), quad_perm [2, 3, 0, 1]
// (lane ^ 2), row_half_mirror (the other quad of each 8 lanes).  The s_nop
// gives the two wait states a DPP read needs after a VALU write of its
// source.  v_max_f32 returns the number when one operand is a quiet NaN
// (IEEE maxNum).  Every lane of the wavefront must be active.
__device__ __forceinline__ float max_dpp_x1(float x)
{
    float r;
    asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
        : "=v"(r) : "v"(x));
    return r;
}
__device__ __forceinline__ float max_dpp_x2(float x)
{
    float r;
    asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
        : "=v"(r) : "v"(x));
    return r;
}
__device__ __forceinline__ float max_dpp_mirror8(float x)
{
    float r;
    asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 row_half_mirror row_mask:0xf bank_mask:0xf"
        : "=v"(r) : "v"(x));
    return r;
}

template <int G>
__device__ __forceinline__ float group_max(float x)
{
    x = max_dpp_x1(x);
    if (G >= 4) x = max_dpp_x2(x);
    if (G >= 8) x = max_dpp_mirror8(x);
    return x;
}

// Byte j of a register block, zero- or sign-extended; 16-bit half j,
// sign-extended.
template <int W>
__device__ __forceinline__ uint32_t ubyte(const uint32_t (&w)[W], int j)
{
    return (w[j >> 2] >> (8 * (j & 3))) & 0xFFu;
}
template <int W>
__device__ __forceinline__ int32_t sbyte(const uint32_t (&w)[W], int j)
{
    return static_cast<int32_t>(w[j >> 2] << (24 - 8 * (j & 3))) >> 24;
}
template <int W>
__device__ __forceinline__ int32_t shalf(const uint32_t (&w)[W], int j)
{
    return static_cast<int32_t>(w[j >> 1] << (16 - 16 * (j & 1))) >> 16;
}

// Dequantization before the scale: y = q/127 or q/255, then the softsign
// inverse y / (2 - |y|) (dequantize()), each operation correctly rounded.
// The dequantize kernel evaluates the 256 entries of its spec into LDS, one
// entry per thread, before its barrier, so the evaluation must be short: it
// uses multiplies and FMAs only, no division sequence and no load (2.8%
// faster than loading the entries there).
//  * q / D: y0 = q R with R = RN(1/D), then one Markstein correction,
//    y = y0 + (q - D y0) R.
//  * y / den with den = 2 - |y|: a reciprocal x of den from the linear
//    estimate 48/17 - 32/17 (den/2) of 1/(den/2) and three Newton steps,
//    then the same correction, z = z0 + (y - den z0) x with z0 = y x.
// Both give the correctly rounded quotient for every code of every spec,
// as an exact (rational) evaluation of each rounding shows; the tests
// repeat that check.
constexpr float kRecipLin0 = 0x1.69696ap+1f;   // 48/17 in fp32
constexpr float kRecipLin1 = 0x1.e1e1e2p+0f;   // 32/17 in fp32
constexpr int kRecipSteps = 3;

template <unsigned SPEC>
__device__ __forceinline__ float dequant_unit(int c)
{
    constexpr bool kSigned = (SPEC & FLASHOPT_Q_SIGNED) != 0;
    constexpr float kD = kSigned ? 127.0f : 255.0f;
    constexpr float kR = 1.0f / kD;
    const float q = kSigned ? static_cast<float>(static_cast<int8_t>(c)) : static_cast<float>(c);
    const float y0 = q * kR;
    float y = __builtin_fmaf(__builtin_fmaf(-kD, y0, q), kR, y0);
    if constexpr ((SPEC & FLASHOPT_Q_SOFTSIGN) != 0) {
        const float den = 2.0f - fabsf(y);
        const float h = den * 0.5f;
        float x = __builtin_fmaf(-kRecipLin1, h, kRecipLin0);
#pragma unroll
        for (int k = 0; k < kRecipSteps; ++k) x = __builtin_fmaf(x, __builtin_fmaf(-h, x, 1.0f), x);
        x = x * 0.5f;
        const float z0 = y * x;
        y = __builtin_fmaf(__builtin_fmaf(-den, z0, y), x, z0);
    }
    return y;
}

// The same entries as compile-time constants in device memory (constant
// evaluation rounds each operation to nearest even, as the device does), for
// the step kernels: each thread loads its entries before its unit's stream
// loads and writes them to LDS once those have arrived, so an entry costs a
// load and no arithmetic.  Computing them there instead added about 2.4 VALU
// instructions per element and cost the 8.0B list step 0.4-1.4%.
template <unsigned SPEC>
struct alignas(16) DequantTable {
    float v[256];
};

template <unsigned SPEC>
constexpr DequantTable<SPEC> make_dequant_table()
{
    constexpr bool kSigned = (SPEC & FLASHOPT_Q_SIGNED) != 0;
    DequantTable<SPEC> t{};
    for (int c = 0; c < 256; ++c) {
        const float q = kSigned ? static_cast<float>(static_cast<int8_t>(c)) : static_cast<float>(c);
        float y = q / (kSigned ? 127.0f : 255.0f);
        if (SPEC & FLASHOPT_Q_SOFTSIGN) {
            const float den = 2.0f - (y < 0.0f ? -y : y);
            y = y / den;
        }
        t.v[c] = y;
    }
    return t;
}

template <unsigned SPEC>
__device__ const DequantTable<SPEC> kDequantTable = make_dequant_table<SPEC>();

// A group's divisor d (1 for a zero scale, else the scale) with its
// correctly rounded reciprocal r.  An infinite scale yields d = r = 0, for
// which div_by_recip returns a/inf = 0 exactly like the plain division.
struct GroupDiv {
    float d, r;
};

__device__ __forceinline__ GroupDiv group_div(uint32_t s)
{
    const uint32_t mag = s & 0x7FFFu;
    const float d = group_divisor(s);
    GroupDiv g{d, math::recip_cr(d)};
    if (mag == 0x7C00u) { g.d = 0.0f; g.r = 0.0f; }
    return g;
}

// Signed code (quantize(), SIGNED): round half to even of y*127 after
// optional softsign companding, clamped to [-127, 127]; NaN -> 0.  Returns
// the int8 value in an int32.
template <bool SOFTSIGN>
__device__ __forceinline__ int32_t code_s8(float y)
{
    if (SOFTSIGN) y = math::softsign(y);
    return math::clamp_i32(math::cvt_i32(rintf(y * 127.0f)), -127, 127);
}

// Unsigned code (quantize(), not SIGNED): round half to even of y*255
// clamped to [0, 255], NaN -> 0, written into byte BYTE of acc
// (v_cvt_pk_u8_f32 does the rounding, clamping and packing in one step).
template <int BYTE>
__device__ __forceinline__ uint32_t code_u8(float y, uint32_t acc)
{
    return __builtin_amdgcn_cvt_pk_u8_f32(y * 255.0f, BYTE, acc);
}

// Low bytes of four int32 values packed into one word.
__device__ __forceinline__ uint32_t pack_bytes(int32_t b0, int32_t b1, int32_t b2, int32_t b3)
{
    const uint32_t lo = __builtin_amdgcn_perm(static_cast<uint32_t>(b1), static_cast<uint32_t>(b0), 0x0C0C0400u);
    const uint32_t hi = __builtin_amdgcn_perm(static_cast<uint32_t>(b3), static_cast<uint32_t>(b2), 0x0C0C0400u);
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// Upper halves of two words packed into one (two bf16 from two fp32 patterns).
__device__ __forceinline__ uint32_t pack_hi16(uint32_t w0, uint32_t w1)
{
    return __builtin_amdgcn_perm(w1, w0, 0x07060302u);
}

// Low halves of two words packed into one.
__device__ __forceinline__ uint32_t pack_lo16(uint32_t w0, uint32_t w1)
{
    return __builtin_amdgcn_perm(w1, w0, 0x05040100u);
}

// Weight split of one fp32 value: theta' = nearest bf16 with ties away from
// zero, D = pattern(x) - (pattern(theta') << 16) in [-32768, 32767], which is
// the low half of the pattern read as a signed 16-bit integer; rho = D
// (32-bit master) or round-half-even(D / 256) clamped to 127 (24-bit).
// Returns pattern(theta') << 16 in `top`.  NaN keeps its upper half, quieted,
// with rho = 0.
template <int MB>
__device__ __forceinline__ void split_elem(float x, uint32_t &top, int32_t &rho)
{
    const uint32_t u = __float_as_uint(x);
    const int32_t D = static_cast<int32_t>(u << 16) >> 16;
    top = u - static_cast<uint32_t>(D);
    if (MB == 32) {
        rho = D;
    } else {
        // floor((D + 127 + parity(floor(D / 256))) / 256): ties go to even
        const int32_t q = (D + 127 + ((D >> 8) & 1)) >> 8;
        rho = q < 127 ? q : 127;
    }
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) {
        top = (u & 0xFFFF0000u) | 0x00400000u;
        rho = 0;
    }
}

// Inverse split: pattern = (theta' << 16) + rho * 2^(16 - w), wrapping.
template <int MB>
__device__ __forceinline__ float reconstruct_elem(uint32_t hi_shifted, int32_t rho)
{
    const uint32_t add = (MB == 24) ? (static_cast<uint32_t>(rho) << 8) : static_cast<uint32_t>(rho);
    return __uint_as_float(hi_shifted + add);
}

// p + e elements with the byte offset formed in 32 bits, so that the access
// takes the scalar base plus a 32-bit lane offset (e sizeof(T) < 2^32).
template <typename T>
__device__ __forceinline__ T *at(T *p, uint32_t e)
{
    return reinterpret_cast<T *>(reinterpret_cast<uintptr_t>(p) + static_cast<uint32_t>(e * sizeof(T)));
}

// Global-address-space views: loads and stores become global_* with an
// SGPR base and a 32-bit lane offset instead of flat accesses.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 g_cu4;
typedef __attribute__((address_space(1))) u32x4 g_u4;
typedef __attribute__((address_space(1))) const uint16_t g_cu16;
typedef __attribute__((address_space(1))) uint16_t g_u16;
typedef __attribute__((address_space(1))) const uint8_t g_cu8;
typedef __attribute__((address_space(1))) uint8_t g_u8;
typedef __attribute__((address_space(1))) const float g_cf32;
typedef __attribute__((address_space(1))) float g_f32;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const u32x2 g_cu2;
typedef __attribute__((address_space(1))) u32x2 g_u2;
typedef __attribute__((address_space(1))) const uint32_t g_cu32;
typedef __attribute__((address_space(1))) uint32_t g_u32;

// Streaming (nontemporal) 16-byte accesses: the step touches every byte once.
__device__ __forceinline__ uint4 ld16s(const void *p, int k = 0)
{
    const u32x4 v = __builtin_nontemporal_load((g_cu4 *)p + k);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st16s(void *p, uint4 v, int k = 0)
{
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, (g_u4 *)p + k);
}
// Streaming 8- and 4-byte accesses.
__device__ __forceinline__ u32x2 ld8s(const void *p) { return __builtin_nontemporal_load((g_cu2 *)p); }
__device__ __forceinline__ void st8s(void *p, u32x2 v) { __builtin_nontemporal_store(v, (g_u2 *)p); }
__device__ __forceinline__ uint32_t ld4s(const void *p) { return __builtin_nontemporal_load((g_cu32 *)p); }
__device__ __forceinline__ void st4s(void *p, uint32_t v) { __builtin_nontemporal_store(v, (g_u32 *)p); }
__device__ __forceinline__ uint16_t ld_u16(const uint16_t *p) { return *(g_cu16 *)p; }
__device__ __forceinline__ void st_u16(uint16_t *p, uint16_t v) { *(g_u16 *)p = v; }

// Codes of N values y_j = a_j / d of one group under SPEC, packed four to a
// word.
template <unsigned SPEC, int N>
__device__ __forceinline__ void encode(const float (&a)[N], const GroupDiv &gd,
                                       uint32_t (&out)[N / 4])
{
    if (SPEC & FLASHOPT_Q_SIGNED) {
#pragma unroll
        for (int k = 0; k < N / 4; ++k) {
            int32_t c[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                c[i] = code_s8<(SPEC & FLASHOPT_Q_SOFTSIGN) != 0>(math::div_by_recip(a[4 * k + i], gd.d, gd.r));
            out[k] = pack_bytes(c[0], c[1], c[2], c[3]);
        }
    } else {
#pragma unroll
        for (int k = 0; k < N / 4; ++k) {
            float y[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                y[i] = math::div_by_recip(a[4 * k + i], gd.d, gd.r);
                if (SPEC & FLASHOPT_Q_SOFTSIGN) y[i] = math::softsign(y[i]);
            }
            uint32_t w = 0u;
            w = code_u8<0>(y[0], w);
            w = code_u8<1>(y[1], w);
            w = code_u8<2>(y[2], w);
            w = code_u8<3>(y[3], w);
            out[k] = w;
        }
    }
}

// rho words of N elements: int16 for the 32-bit master, else int8.
constexpr int rho_words(int mb, int n) { return mb == 32 ? n / 2 : n / 4; }

// parameter (and gradient) words of N elements: fp32, or two bf16 per word.
constexpr int param_words(int mb, int n) { return mb == kParamF32 ? n : n / 2; }

// Re-split of N fp32 values into packed bf16 words and packed rho words.
// theta' (ties away from zero) is the upper half of pattern + 0x8000; D is
// the lower half of the pattern read as a signed 16-bit integer.  For the
// 24-bit master, rho = clamp(round-half-even(D / 256), -128, 127) is formed
// as v_cvt_pk_u8_f32(D / 256 + 128) - 128: D / 256 + 128 is exact, the
// conversion rounds half to even, clamps to [0, 255] (so D >= 32640 gives
// 127) and packs the byte in place; the -128 is a per-word XOR.  NaN inputs
// are not handled here (split_pack_exact covers them).
template <int MB, int N>
__device__ __forceinline__ void split_pack(const float (&x)[N], uint32_t (&po)[N / 2],
                                           uint32_t (&ro)[rho_words(MB, N)])
{
#pragma unroll
    for (int i = 0; i < N / 2; ++i)
        po[i] = pack_hi16(__float_as_uint(x[2 * i]) + 0x8000u, __float_as_uint(x[2 * i + 1]) + 0x8000u);
    if constexpr (MB == 32) {
#pragma unroll
        for (int i = 0; i < N / 2; ++i)
            ro[i] = pack_lo16(__float_as_uint(x[2 * i]), __float_as_uint(x[2 * i + 1]));
    } else {
#pragma unroll
        for (int k = 0; k < N / 4; ++k) {
            uint32_t w = 0u;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int32_t D = static_cast<int32_t>(__float_as_uint(x[4 * k + b]) << 16) >> 16;
                const float f = __builtin_fmaf(static_cast<float>(D), 0x1p-8f, 128.0f);
                w = (b == 0) ? __builtin_amdgcn_cvt_pk_u8_f32(f, 0, w)
                  : (b == 1) ? __builtin_amdgcn_cvt_pk_u8_f32(f, 1, w)
                  : (b == 2) ? __builtin_amdgcn_cvt_pk_u8_f32(f, 2, w)
                             : __builtin_amdgcn_cvt_pk_u8_f32(f, 3, w);
            }
            ro[k] = w ^ 0x80808080u;
        }
    }
}

// The same re-split element by element, NaN included (NaN keeps its upper
// half, quieted, with rho = 0).
template <int MB, int N>
__device__ __forceinline__ void split_pack_exact(const float (&x)[N], uint32_t (&po)[N / 2],
                                                 uint32_t (&ro)[rho_words(MB, N)])
{
    uint32_t top[N];
    int32_t rr[N];
#pragma unroll
    for (int j = 0; j < N; ++j) split_elem<MB>(x[j], top[j], rr[j]);
#pragma unroll
    for (int i = 0; i < N / 2; ++i) po[i] = pack_hi16(top[2 * i], top[2 * i + 1]);
    if constexpr (MB == 32) {
#pragma unroll
        for (int i = 0; i < N / 2; ++i)
            ro[i] = pack_lo16(static_cast<uint32_t>(rr[2 * i]), static_cast<uint32_t>(rr[2 * i + 1]));
    } else {
#pragma unroll
        for (int i = 0; i < N / 4; ++i) ro[i] = pack_bytes(rr[4 * i], rr[4 * i + 1], rr[4 * i + 2], rr[4 * i + 3]);
    }
}

// The exact signed code word (four int8 codes) of four values of one group:
// y = a / d, softsign y if SOFTSIGN, round half to even of y * 127 clamped to
// [-127, 127] (magic-number rounding, flashopt_math.h).  Finite values only.
template <bool SOFTSIGN>
__device__ __forceinline__ uint32_t s8_word_exact(float a0, float a1, float a2, float a3,
                                                  const GroupDiv &gd)
{
    float y[4] = {a0, a1, a2, a3};
    uint32_t b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float q = math::div_by_recip(y[i], gd.d, gd.r);
        if (SOFTSIGN) q = math::softsign(q);
        b[i] = math::code_s8_magic(q * 127.0f);
    }
    return pack_bytes(static_cast<int32_t>(b[0]), static_cast<int32_t>(b[1]),
                      static_cast<int32_t>(b[2]), static_cast<int32_t>(b[3]));
}

// Signed codes of N group quotients with the magic-number rounding of
// flashopt_math.h (finite inputs only; callers send lanes holding NaN or
// infinite values to encode).
template <bool SOFTSIGN, int N>
__device__ __forceinline__ void encode_s8_finite(const float (&a)[N], const GroupDiv &gd,
                                                 uint32_t (&out)[N / 4])
{
#pragma unroll
    for (int k = 0; k < N / 4; ++k)
        out[k] = s8_word_exact<SOFTSIGN>(a[4 * k], a[4 * k + 1], a[4 * k + 2], a[4 * k + 3], gd);
}

// Companded momentum codes of N finite values of one group with fp16 scale
// bits s, through the two-sided short form (math::softsign_code_bytes): a
// word (four codes) whose two evaluations disagree, i.e. with a value within
// 1e-4 of a code's rounding boundary, is recomputed with the correctly
// rounded chain, whose reciprocal of the divisor only that path needs.  An
// fp16-subnormal scale (its rounding may leave |m / d| up to 1.5, beyond the
// short form's unclamped range) or an infinite one takes the chain for the
// whole unit.  Both routes give the same bits.
template <int N>
__device__ __forceinline__ void encode_s8_softsign_fast(const float (&a)[N], uint32_t s,
                                                        uint32_t (&out)[N / 4])
{
    const uint32_t mag = s & 0x7FFFu;
    if ((mag != 0u && mag < 0x0400u) || mag == 0x7C00u) {
        encode_s8_finite<true, N>(a, group_div(s), out);
        return;
    }
    const float c0 = group_divisor(s) * math::kInv254;
    bool amb[N / 4], any = false;
#pragma unroll
    for (int k = 0; k < N / 4; ++k) {
        uint32_t hi, lo;
        math::softsign_code_bytes(a[4 * k], a[4 * k + 1], a[4 * k + 2], a[4 * k + 3], c0, hi, lo);
        out[k] = hi ^ 0x80808080u;            // byte = code + 128 -> the code's two's-complement byte
        amb[k] = hi != lo;
        any |= amb[k];
    }
    if (any) {                                 // rare: a code within 1e-4 of a rounding boundary
        const GroupDiv gd = group_div(s);
#pragma unroll
        for (int k = 0; k < N / 4; ++k)
            if (amb[k]) out[k] = s8_word_exact<true>(a[4 * k], a[4 * k + 1], a[4 * k + 2], a[4 * k + 3], gd);
    }
}

// ------------------------------------------------------- standalone codec

// Element offset of unit u (0..3) of the calling lane in its wavefront's
// 1024-element chunk: 4 consecutive elements, the 64 lanes of a unit covering
// 256 consecutive elements, so that every access instruction of the
// wavefront touches one contiguous block of each stream.  The quantize and
// dequantize kernels use it (16 bytes of fp32 per lane and unit).
__device__ __forceinline__ int64_t quad_first(int u)
{
    const int64_t chunk =
        (static_cast<int64_t>(blockIdx.x) * (kBlockThreads / kWaveLanes) + (threadIdx.x >> 6)) *
        kChunkElems;
    return chunk + 256 * u + 4 * static_cast<int>(threadIdx.x & 63u);
}

__device__ __forceinline__ int quad_count(int64_t n, int64_t e)
{
    const int64_t r = n - e;
    return r >= 4 ? 4 : (r > 0 ? static_cast<int>(r) : 0);
}

template <unsigned SPEC>
__global__ void __launch_bounds__(kBlockThreads)
quantize_kernel(const float *__restrict__ x, int64_t n, void *__restrict__ codes,
                uint16_t *__restrict__ scales)
{
    constexpr bool kSigned = (SPEC & FLASHOPT_Q_SIGNED) != 0;
    uint8_t *cb = static_cast<uint8_t *>(codes);
    // every lane runs every unit (the group maximum exchanges values between
    // lanes); elements past n are the zero pad
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t e = quad_first(u);
        const int cnt = quad_count(n, e);
        float a[4];
        if (cnt == 4) {
            const uint4 v = ld16s(x + e);
            a[0] = __uint_as_float(v.x); a[1] = __uint_as_float(v.y);
            a[2] = __uint_as_float(v.z); a[3] = __uint_as_float(v.w);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) a[j] = j < cnt ? ((g_cf32 *)(x + e))[j] : 0.0f;
        }
        if (SPEC & FLASHOPT_Q_SQRT) {
            uint32_t ubits = 0u;
#pragma unroll
            for (int j = 0; j < 4; ++j) ubits = max(ubits, __float_as_uint(a[j]));
            if (ubits < kSqrtFastEnd) {
#pragma unroll
                for (int j = 0; j < 4; ++j) a[j] = math::sqrt_cr(a[j]);
            } else {                         // rare: inputs outside the fast sqrt's range
#pragma unroll
                for (int j = 0; j < 4; ++j) a[j] = sqrtf(a[j]);
            }
        }
        // maxNum over the group's elements: NaNs are ignored unless all are NaN
        float amax = kSigned ? fabsf(a[0]) : a[0];
#pragma unroll
        for (int j = 1; j < 4; ++j) amax = fmaxf(amax, kSigned ? fabsf(a[j]) : a[j]);
        amax = group_max<8>(amax);
        const uint32_t s = f16_bits(amax);
        uint32_t w[1];
        if constexpr (SPEC == FLASHOPT_SPEC_MOMENTUM) {
            // finite values take the guarded short code sequence
            bool finite = true;
#pragma unroll
            for (int j = 0; j < 4; ++j) finite &= fabsf(a[j]) <= 0x1.fffffep127f;
            if (finite) encode_s8_softsign_fast<4>(a, s, w);
            else encode<SPEC, 4>(a, group_div(s), w);
        } else {
            encode<SPEC, 4>(a, group_div(s), w);
        }
        if (cnt == 4) st4s(cb + e, w[0]);
        else
            for (int j = 0; j < cnt; ++j) ((g_u8 *)(cb + e))[j] = static_cast<uint8_t>(w[0] >> (8 * j));
        if ((threadIdx.x & 7u) == 0 && cnt > 0) st_u16(scales + e / kGroup, static_cast<uint16_t>(s));
    }
}

template <unsigned SPEC>
__global__ void __launch_bounds__(kBlockThreads)
dequantize_kernel(const void *__restrict__ codes, const uint16_t *__restrict__ scales, int64_t n,
                  float *__restrict__ out)
{
    __shared__ float unit[256];
    unit[threadIdx.x] = dequant_unit<SPEC>(static_cast<int>(threadIdx.x));
    __syncthreads();

    const uint8_t *cb = static_cast<const uint8_t *>(codes);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t e = quad_first(u);
        const int cnt = quad_count(n, e);
        if (cnt == 0) continue;
        uint32_t w[1] = {0u};
        if (cnt == 4) w[0] = ld4s(cb + e);
        else
            for (int j = 0; j < cnt; ++j) w[0] |= static_cast<uint32_t>(((g_cu8 *)(cb + e))[j]) << (8 * j);
        const float s = f16_value(ld_u16(scales + e / kGroup));
        float o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float v = unit[ubyte(w, j)] * s;
            if (SPEC & FLASHOPT_Q_SQRT) v = v * v;
            o[j] = v;
        }
        if (cnt == 4) st16s(out + e, make_uint4(__float_as_uint(o[0]), __float_as_uint(o[1]),
                                                __float_as_uint(o[2]), __float_as_uint(o[3])));
        else
            for (int j = 0; j < cnt; ++j) ((g_f32 *)(out + e))[j] = o[j];
    }
}

// ------------------------------------------------------- standalone split

// Element offset of unit u of the calling lane in the split and reconstruct
// kernels: a wavefront takes U consecutive 256-element units, 4 consecutive
// elements per lane and unit (16 bytes of fp32), so that every access
// instruction of the wavefront covers one contiguous block of each stream; a
// workgroup takes 1024 U elements (a "block" of launch_flat), a launch the
// blocks from `base` on.  One unit per wavefront streams faster for the
// split and the 24-bit reconstruct (one load and one store instruction per
// stream and wavefront; 6-8% over four units), four units for the 32-bit
// reconstruct (3%).
template <int U>
__device__ __forceinline__ int64_t split_lane_first(int64_t base, int u)
{
    const int64_t wave = (base + blockIdx.x) * (kBlockThreads / kWaveLanes) + (threadIdx.x >> 6);
    return wave * (256 * U) + 256 * u + 4 * static_cast<int64_t>(threadIdx.x & 63u);
}

// Units per wavefront of the split and reconstruct kernels, by master
// width (measured, see split_lane_first).
constexpr int split_units(int mb, bool reconstruct) { return reconstruct && mb == 32 ? 4 : 1; }

template <int MB>
__global__ void __launch_bounds__(kBlockThreads)
split_kernel(const float *__restrict__ master, int64_t n, uint16_t *__restrict__ param,
             void *__restrict__ rho, int64_t base)
{
    constexpr int U = split_units(MB, false);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t e = split_lane_first<U>(base, u);
        const int cnt = quad_count(n, e);
        if (cnt == 0) continue;
        float x[4];
        if (cnt == 4) {
            const uint4 v = ld16s(master + e);
            x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
            x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = j < cnt ? ((g_cf32 *)(master + e))[j] : 0.0f;
        }
        uint32_t pw[2], rw[rho_words(MB, 4)];
        bool any_nan = false;
#pragma unroll
        for (int j = 0; j < 4; ++j) any_nan |= x[j] != x[j];
        if (any_nan) split_pack_exact<MB, 4>(x, pw, rw);
        else split_pack<MB, 4>(x, pw, rw);
        if (cnt == 4) {
            st8s(param + e, u32x2{pw[0], pw[1]});
            if constexpr (MB == 32) st8s(static_cast<uint16_t *>(rho) + e, u32x2{rw[0], rw[1]});
            else st4s(static_cast<uint8_t *>(rho) + e, rw[0]);
        } else {
            for (int j = 0; j < cnt; ++j) {
                ((g_u16 *)(param + e))[j] = static_cast<uint16_t>(pw[j >> 1] >> (16 * (j & 1)));
                if constexpr (MB == 32)
                    ((g_u16 *)(static_cast<uint16_t *>(rho) + e))[j] =
                        static_cast<uint16_t>(rw[j >> 1] >> (16 * (j & 1)));
                else
                    ((g_u8 *)(static_cast<uint8_t *>(rho) + e))[j] = static_cast<uint8_t>(rw[0] >> (8 * j));
            }
        }
    }
}

template <int MB>
__global__ void __launch_bounds__(kBlockThreads)
reconstruct_kernel(const uint16_t *__restrict__ param, const void *__restrict__ rho, int64_t n,
                   float *__restrict__ master, int64_t base)
{
    constexpr int U = split_units(MB, true);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t e = split_lane_first<U>(base, u);
        const int cnt = quad_count(n, e);
        if (cnt == 0) continue;
        uint32_t pw[2] = {0u, 0u}, rw[MB == 32 ? 2 : 1] = {};
        if (cnt == 4) {
            const u32x2 p2 = ld8s(param + e);
            pw[0] = p2.x; pw[1] = p2.y;
            if constexpr (MB == 32) {
                const u32x2 r2 = ld8s(static_cast<const uint16_t *>(rho) + e);
                rw[0] = r2.x; rw[1] = r2.y;
            } else {
                rw[0] = ld4s(static_cast<const uint8_t *>(rho) + e);
            }
        } else {
            for (int j = 0; j < cnt; ++j) {
                pw[j >> 1] |= static_cast<uint32_t>(((g_cu16 *)(param + e))[j]) << (16 * (j & 1));
                if constexpr (MB == 32)
                    rw[j >> 1] |= static_cast<uint32_t>(((g_cu16 *)(static_cast<const uint16_t *>(rho) + e))[j])
                                  << (16 * (j & 1));
                else
                    rw[0] |= static_cast<uint32_t>(((g_cu8 *)(static_cast<const uint8_t *>(rho) + e))[j])
                             << (8 * j);
            }
        }
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t hs = (j & 1) ? (pw[j >> 1] & 0xFFFF0000u) : (pw[j >> 1] << 16);
            int32_t r;
            if constexpr (MB == 32) r = shalf(rw, j);
            else r = sbyte(rw, j);
            x[j] = reconstruct_elem<MB>(hs, r);
        }
        if (cnt == 4) st16s(master + e, make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]),
                                                   __float_as_uint(x[2]), __float_as_uint(x[3])));
        else
            for (int j = 0; j < cnt; ++j) ((g_f32 *)(master + e))[j] = x[j];
    }
}

// ---------------------------------------------------- fused FlashAdamW step

// bf16 of an fp32 pattern rounded to nearest, ties to even (torch's cast, the
// parameter update without a master split), in the upper half of the result.
// Finite and infinite values only; NaN is handled by plain_elem.
__device__ __forceinline__ uint32_t bf16_rne_top(uint32_t u)
{
    return u + 0x7FFFu + ((u >> 16) & 1u);
}

// The same with NaN kept (upper half, quieted).
__device__ __forceinline__ uint32_t plain_elem(float x)
{
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u & 0xFFFF0000u) | 0x00400000u;
    return bf16_rne_top(u);
}

// The new parameter words (and rho words with a master split) of N updated
// values: the split, the bf16 cast, or the fp32 value itself.  EXACT selects
// the element-wise NaN-safe routines.
template <int MB, bool EXACT, int N>
__device__ __forceinline__ void pack_theta(const float (&x)[N], uint32_t (&po)[param_words(MB, N)],
                                           uint32_t (&ro)[rho_words(MB, N)])
{
    if constexpr (MB == kParamF32) {          // an fp32 parameter keeps the update as is
#pragma unroll
        for (int i = 0; i < N; ++i) po[i] = __float_as_uint(x[i]);
    } else if constexpr (MB == 0) {
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            if (EXACT) po[i] = pack_hi16(plain_elem(x[2 * i]), plain_elem(x[2 * i + 1]));
            else po[i] = pack_hi16(bf16_rne_top(__float_as_uint(x[2 * i])),
                                   bf16_rne_top(__float_as_uint(x[2 * i + 1])));
        }
    } else if constexpr (EXACT) {
        split_pack_exact<MB, N>(x, po, ro);
    } else {
        split_pack<MB, N>(x, po, ro);
    }
}

// ----------------------------------------------------------- lane units
//
// A wavefront owns a 1024-element chunk; each lane takes its elements in
// units of N consecutive elements: unit u of lane l is chunk elements
// 64 N u + N l + i (i < N), so every access instruction of the wavefront
// covers one contiguous block of each stream.  A 32-element quantization
// group is one unit of each of 32 / N adjacent lanes.  The per-variant N
// (unit_elems) follows from the access shape: a 16-byte access per lane
// streams best; a lane moving 64 contiguous bytes of one stream in four
// 16-byte accesses (fp32 moments with N = 16) streams at well under half the
// bandwidth, and 32 bytes (16-bit streams with N = 16) somewhat below.

// BYTES (4, 8, 16, 32 or 64) consecutive bytes at p into words, streaming.
template <int BYTES>
__device__ __forceinline__ void ld_words(const void *p, uint32_t *w)
{
    if constexpr (BYTES == 4) {
        w[0] = ld4s(p);
    } else if constexpr (BYTES == 8) {
        const u32x2 v = ld8s(p);
        w[0] = v.x; w[1] = v.y;
    } else {
#pragma unroll
        for (int k = 0; k < BYTES / 16; ++k) {
            const uint4 v = ld16s(p, k);
            w[4 * k] = v.x; w[4 * k + 1] = v.y; w[4 * k + 2] = v.z; w[4 * k + 3] = v.w;
        }
    }
}

template <int BYTES>
__device__ __forceinline__ void st_words(void *p, const uint32_t *w)
{
    if constexpr (BYTES == 4) {
        st4s(p, w[0]);
    } else if constexpr (BYTES == 8) {
        st8s(p, u32x2{w[0], w[1]});
    } else {
#pragma unroll
        for (int k = 0; k < BYTES / 16; ++k)
            st16s(p, make_uint4(w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]), k);
    }
}

// The first cnt of N elements of ESZ (1, 2 or 4) bytes at p into words,
// zeros beyond; and the matching masked store.
template <int ESZ, int N>
__device__ __forceinline__ void ld_elems(const void *p, int cnt, uint32_t *w)
{
#pragma unroll
    for (int i = 0; i < N * ESZ / 4; ++i) w[i] = 0u;
#pragma unroll
    for (int j = 0; j < N; ++j) {
        if (j < cnt) {
            if constexpr (ESZ == 1) w[j >> 2] |= static_cast<uint32_t>(((g_cu8 *)p)[j]) << (8 * (j & 3));
            if constexpr (ESZ == 2) w[j >> 1] |= static_cast<uint32_t>(((g_cu16 *)p)[j]) << (16 * (j & 1));
            if constexpr (ESZ == 4) w[j] = ((g_cu32 *)p)[j];
        }
    }
}

template <int ESZ, int N>
__device__ __forceinline__ void st_elems(void *p, int cnt, const uint32_t *w)
{
#pragma unroll
    for (int j = 0; j < N; ++j) {
        if (j < cnt) {
            if constexpr (ESZ == 1) ((g_u8 *)p)[j] = static_cast<uint8_t>(w[j >> 2] >> (8 * (j & 3)));
            if constexpr (ESZ == 2) ((g_u16 *)p)[j] = static_cast<uint16_t>(w[j >> 1] >> (16 * (j & 1)));
            if constexpr (ESZ == 4) ((g_u32 *)p)[j] = w[j];
        }
    }
}

// Elements per unit of each step variant: fp32 moments and fp32 parameters
// need N = 4 for 16-byte accesses; the quantized variants use N = 8 (16-bit streams in
// 16-byte accesses, a lane quad per group).  Measured on the 8.0B list
// against N = 16: 1.1% faster for the 24-bit master, 8.4% for the 32-bit
// master, 4.1% for the linear codec.
constexpr int unit_elems(int mb, int st) { return (st == kStatesFp32 || mb == kParamF32) ? 4 : 8; }

// One unit's inputs (arrays a variant does not use are removed by the
// compiler).
template <int MB, int ST, int N>
struct UnitIn {
    uint32_t pw[param_words(MB, N)], gw[param_words(MB, N)];
    uint32_t rw[rho_words(MB, N)];   // rho words, each value's sign bit flipped
    uint32_t mw[N / 4], vw[N / 4];   // codes (quantized states)
    uint32_t mf[N], vf[N];           // fp32 states, bit patterns
    uint32_t smb, svb;               // fp16 scale bits of the unit's group
};

// First element of unit u of a lane, relative to the chunk.
template <int N>
__device__ __forceinline__ uint32_t unit_first(int u, int lane)
{
    return static_cast<uint32_t>(64 * N * u + N * lane);
}

// Stream pointers at the start of one chunk, uniform across the wavefront
// (scalar registers), so that unit accesses take a scalar base plus a 32-bit
// lane offset; rem = elements of the chunk that exist, capped at 1024.
struct ChunkPtrs {
    uint16_t *param;
    const uint16_t *grad;
    uint32_t *param32;          // the same streams as fp32 (kParamF32)
    const uint32_t *grad32;
    uint8_t *rho8;
    uint16_t *rho16;
    uint8_t *mc, *vc;
    uint32_t *mf, *vf;
    uint16_t *ms, *vs;
    int rem;
};

// Pointers of chunk k of a tensor, in the per-tensor streams or, with a
// blocked state layout (L.bytes != 0), in the chunk's block of the state
// buffer at d.rho (uniform: scalar arithmetic).  Whether the chunk is full
// is decided on 32-bit chunk indices (scalar compares; gfx9 has no 64-bit
// scalar less-than).
__device__ __forceinline__ ChunkPtrs chunk_ptrs(const DevTensor &d, int32_t k, const StateLayout &L)
{
    const int64_t off = static_cast<int64_t>(k) * kChunkElems;
    ChunkPtrs c;
    c.param = d.param + off;
    c.grad = d.grad + off;
    c.param32 = reinterpret_cast<uint32_t *>(d.param) + off;
    c.grad32 = reinterpret_cast<const uint32_t *>(d.grad) + off;
    c.mf = reinterpret_cast<uint32_t *>(d.m_codes) + off;
    c.vf = reinterpret_cast<uint32_t *>(d.v_codes) + off;
    if (L.bytes != 0u) {
        uint8_t *b = static_cast<uint8_t *>(d.rho) + static_cast<int64_t>(k) * L.bytes;
        c.rho8 = b;
        c.rho16 = reinterpret_cast<uint16_t *>(b);
        c.mc = b + L.m;
        c.vc = b + L.v;
        c.ms = reinterpret_cast<uint16_t *>(b + L.ms);
        c.vs = reinterpret_cast<uint16_t *>(b + L.vs);
    } else {
        c.rho8 = static_cast<uint8_t *>(d.rho) + off;
        c.rho16 = static_cast<uint16_t *>(d.rho) + off;
        c.mc = reinterpret_cast<uint8_t *>(d.m_codes) + off;
        c.vc = d.v_codes + off;
        c.ms = d.m_scales + off / kGroup;
        c.vs = d.v_scales + off / kGroup;
    }
    const int32_t full = static_cast<int32_t>(d.numel / kChunkElems);
    c.rem = k < full ? kChunkElems : static_cast<int>(d.numel % kChunkElems);
    return c;
}

// Elements of the unit at chunk offset r that exist: N, fewer at a ragged
// end, or 0.
template <int N>
__device__ __forceinline__ int unit_count(const ChunkPtrs &c, uint32_t r)
{
    const int rem = c.rem - static_cast<int>(r);
    return rem >= N ? N : (rem > 0 ? rem : 0);
}

// Loads of one unit of every stream (the unit at chunk offset r).  FULL:
// straight-line streaming loads; otherwise element-masked loads with zeros
// for missing elements (and zero scales for a unit with none).
template <int MB, int ST, int N, bool FULL, bool V = true>
__device__ __forceinline__ void load_unit(const ChunkPtrs &c, uint32_t r, int cnt,
                                          UnitIn<MB, ST, N> &in)
{
    in.smb = 0u;
    in.svb = 0u;
    if (FULL) {
        if constexpr (MB == kParamF32) {
            ld_words<4 * N>(at(c.param32, r), in.pw);
            ld_words<4 * N>(at(c.grad32, r), in.gw);
        } else {
            ld_words<2 * N>(at(c.param, r), in.pw);
            ld_words<2 * N>(at(c.grad, r), in.gw);
        }
        if constexpr (MB == 24) ld_words<N>(c.rho8 + r, in.rw);
        if constexpr (MB == 32) ld_words<2 * N>(at(c.rho16, r), in.rw);
        if constexpr (ST == kStatesFp32) {
            ld_words<4 * N>(at(c.mf, r), in.mf);
            if constexpr (V) ld_words<4 * N>(at(c.vf, r), in.vf);
        } else {
            ld_words<N>(c.mc + r, in.mw);
            in.smb = ld_u16(c.ms + r / kGroup);
            if constexpr (V) {
                ld_words<N>(c.vc + r, in.vw);
                in.svb = ld_u16(c.vs + r / kGroup);
            }
        }
    } else {
        if constexpr (MB == kParamF32) {
            ld_elems<4, N>(c.param32 + r, cnt, in.pw);
            ld_elems<4, N>(c.grad32 + r, cnt, in.gw);
        } else {
            ld_elems<2, N>(c.param + r, cnt, in.pw);
            ld_elems<2, N>(c.grad + r, cnt, in.gw);
        }
        if constexpr (MB == 24) ld_elems<1, N>(c.rho8 + r, cnt, in.rw);
        if constexpr (MB == 32) ld_elems<2, N>(c.rho16 + r, cnt, in.rw);
        if constexpr (ST == kStatesFp32) {
            ld_elems<4, N>(c.mf + r, cnt, in.mf);
            if constexpr (V) ld_elems<4, N>(c.vf + r, cnt, in.vf);
        } else {
            ld_elems<1, N>(c.mc + r, cnt, in.mw);
            if constexpr (V) ld_elems<1, N>(c.vc + r, cnt, in.vw);
            if (cnt > 0) {
                in.smb = ld_u16(c.ms + r / kGroup);
                if constexpr (V) in.svb = ld_u16(c.vs + r / kGroup);
            }
        }
    }
    // offset-binary rho for reconstruct_perm
#pragma unroll
    for (int i = 0; i < rho_words(MB, N); ++i) in.rw[i] ^= (MB == 32 ? 0x80008000u : 0x80808080u);
}

// Master pattern of element j, (theta' << 16) + rho * 2^(16 - w), from the
// bf16 words and the offset-binary rho words (rho + 2^(w-1) as an unsigned
// field): one v_perm places theta' in the upper half and the rho field
// below it (24-bit: bits 8-15, low byte zero; 32-bit: bits 0-15), which is
// the pattern plus 2^15; the subtraction removes that in wrapping integer
// arithmetic.
template <int MB, int W, int R>
__device__ __forceinline__ float reconstruct_perm(const uint32_t (&pw)[W], const uint32_t (&rw)[R],
                                                  int j)
{
    const uint32_t hi = 4u + 2u * static_cast<uint32_t>(j & 1);   // theta' bytes in S0
    uint32_t sel;
    if constexpr (MB == 24) sel = 0x0Cu | (static_cast<uint32_t>(j & 3) << 8);
    else sel = (2u * static_cast<uint32_t>(j & 1)) | ((2u * static_cast<uint32_t>(j & 1) + 1u) << 8);
    sel |= (hi << 16) | ((hi + 1u) << 24);
    const uint32_t word = MB == 24 ? rw[j >> 2] : rw[j >> 1];
    return __uint_as_float(__builtin_amdgcn_perm(pw[j >> 1], word, sel) - 0x8000u);
}

// Element j of a unit: the master theta (reconstructed, or the bf16 value
// itself without a split), and the new moments m1 = b1 m0 + (1 - b1) g and
// v1 = b2 v0 + ((1 - b2) g) g from the dequantized (or fp32) old ones.
template <int MB, int ST, int N>
__device__ __forceinline__ void element_moments(const UnitIn<MB, ST, N> &in, int j,
                                                const StepScalars &sc, const float *s_mu,
                                                const float *s_vu, float ms, float vs,
                                                float &theta, float &m, float &v)
{
    float g;
    if constexpr (MB == kParamF32) {
        theta = __uint_as_float(in.pw[j]);
        g = __uint_as_float(in.gw[j]);
    } else {
        if constexpr (MB == 0) theta = (j & 1) ? bf16_hi(in.pw[j >> 1]) : bf16_lo(in.pw[j >> 1]);
        else theta = reconstruct_perm<MB>(in.pw, in.rw, j);
        g = (j & 1) ? bf16_hi(in.gw[j >> 1]) : bf16_lo(in.gw[j >> 1]);
    }
    float m0, v0;
    if constexpr (ST == kStatesFp32) {
        m0 = __uint_as_float(in.mf[j]);
        v0 = __uint_as_float(in.vf[j]);
    } else {
        m0 = s_mu[ubyte(in.mw, j)] * ms;
        const float a0 = s_vu[ubyte(in.vw, j)] * vs;
        v0 = ST == kStatesCompanded ? a0 * a0 : a0;
    }
    const float m_decay = sc.b1 * m0;
    const float m_new = sc.c1 * g;
    m = m_decay + m_new;
    const float v_decay = sc.b2 * v0;
    const float cg = sc.c2 * g;
    const float v_new = cg * g;
    v = v_decay + v_new;
}

// The generic recomputation of one unit's updated parameter (and momentum
// codes) for lanes outside the short sequences' domains (see step_finish):
// reload the unit's inputs, redo the element arithmetic with correctly
// rounded division and sqrt, and encode and split with the NaN-safe element
// routines.  The variance codes, fp32 moments and the group scales do not
// depend on these paths and are produced by the caller.
template <int MB, int ST, int N>
__device__ __forceinline__ void unit_exact(const ChunkPtrs &c, uint32_t r, int cnt,
                                           const StepScalars &sc, const float *s_mu,
                                           const float *s_vu, uint32_t sm,
                                           uint32_t (&mo)[N / 4], uint32_t (&po)[param_words(MB, N)],
                                           uint32_t (&ro)[rho_words(MB, N)])
{
    constexpr unsigned kMSpec =
        ST == kStatesCompanded ? FLASHOPT_SPEC_MOMENTUM : FLASHOPT_SPEC_MOMENTUM_LINEAR;
    // an opaque copy of the unit offset keeps the compiler from reusing the
    // common path's loads, whose values would then stay live up to here
    asm volatile("" : "+v"(r));
    UnitIn<MB, ST, N> in;
    load_unit<MB, ST, N, false>(c, r, cnt, in);
    const float ms = f16_value(in.smb);
    const float vs = f16_value(in.svb);
    float m1[N], th1[N];
#pragma unroll
    for (int j = 0; j < N; ++j) {
        float theta, m, v;
        element_moments<MB, ST, N>(in, j, sc, s_mu, s_vu, ms, vs, theta, m, v);
        const float thd = theta * sc.cwd;
        const float mhat = m / sc.bc1;
        const float vhat = v / sc.bc2;
        const float den = sqrtf(vhat) + sc.eps;
        const float num = sc.lr * mhat;
        th1[j] = thd - num / den;
        m1[j] = j < cnt ? m : 0.0f;
    }
    if constexpr (ST != kStatesFp32) encode<kMSpec, N>(m1, group_div(sm), mo);
    pack_theta<MB, true, N>(th1, po, ro);
}

// Variance codes (the sqrt spec) of N values of one group with fp16 scale
// bits s.  The chain quantizes rt = sqrt(v1): y = rt / d, p = y * 255.  The
// update has already formed sq = sqrt(vhat) 2^32 with vhat = v1 / bc2, so
// p is taken as sq cv with cv = kv / d per group and kv = 255 sqrt(bc2) 2^-32
// (host, rounded once): relative error at most 3.5 units of 2^-24 (vhat's
// rounding halved by the sqrt, sq, kv, cv; the product is exact inside the
// fma) against at most 3 for the chain (rt, y, p), so the two differ by less
// than 6.5 2^-24 255.2 < 9.9e-5 (p <= 255.2 below the clamp).  Each code is
// converted twice, at p + and - kVarianceBand = 1.5e-4 (each fma adds at most
// 2^-17); where the two bytes agree no rounding boundary lies within 9.9e-5
// of p and the byte is the chain's code.  Words that disagree, and all words
// when exact_all (some v1 outside the range where the update formed sq),
// take the chain.
template <int N>
__device__ __forceinline__ void variance_codes(const float (&sq)[N], const float (&v1)[N], uint32_t s,
                                               float kv, bool exact_all, uint32_t (&out)[N / 4])
{
    const GroupDiv gd = group_div(s);
    const float cv = math::div_by_recip(kv, gd.d, gd.r);    // 0 for an infinite scale: codes 0
    constexpr float up = math::kVarianceBand, dn = -math::kVarianceBand;
    bool amb[N / 4], any = exact_all;
#pragma unroll
    for (int k = 0; k < N / 4; ++k) {
        uint32_t hi = 0u, lo = 0u;
        hi = math::cvt_u8<0>(__builtin_fmaf(sq[4 * k], cv, up), hi);
        lo = math::cvt_u8<0>(__builtin_fmaf(sq[4 * k], cv, dn), lo);
        hi = math::cvt_u8<1>(__builtin_fmaf(sq[4 * k + 1], cv, up), hi);
        lo = math::cvt_u8<1>(__builtin_fmaf(sq[4 * k + 1], cv, dn), lo);
        hi = math::cvt_u8<2>(__builtin_fmaf(sq[4 * k + 2], cv, up), hi);
        lo = math::cvt_u8<2>(__builtin_fmaf(sq[4 * k + 2], cv, dn), lo);
        hi = math::cvt_u8<3>(__builtin_fmaf(sq[4 * k + 3], cv, up), hi);
        lo = math::cvt_u8<3>(__builtin_fmaf(sq[4 * k + 3], cv, dn), lo);
        out[k] = hi;
        amb[k] = exact_all || hi != lo;
        any |= amb[k];
    }
    if (any) {                                  // rare: the correctly rounded chain for those words
        GroupDiv g2 = gd;
        g2.d *= 0x1p32f;                        // rt / d = (rt 2^32) / (d 2^32), same rounding
        g2.r *= 0x1p-32f;
#pragma unroll
        for (int k = 0; k < N / 4; ++k) {
            if (!amb[k]) continue;
            float rt[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = v1[4 * k + i];
                rt[i] = __float_as_uint(v) < kSqrtFastEnd ? math::sqrt_x2p32_zero_tiny(v) : sqrtf(v) * 0x1p32f;
            }
            uint32_t w[1];
            encode<FLASHOPT_SPEC_VARIANCE, 4>(rt, g2, w);
            out[k] = w[0];
        }
    }
}

// Issue the loads of unit u of a chunk for one lane (its first element r and
// count cnt are returned): straight-line streaming accesses for a full
// chunk, accesses masked per element at the ragged end of a tensor (missing
// elements read as zero).
template <int MB, int ST, int N, bool V = true>
__device__ __forceinline__ void load_chunk_unit(const ChunkPtrs &c, int u, int lane, uint32_t &r,
                                                int &cnt, UnitIn<MB, ST, N> &in)
{
    r = unit_first<N>(u, lane);
    if (c.rem == kChunkElems) {
        cnt = N;
        load_unit<MB, ST, N, true, V>(c, r, cnt, in);
    } else {
        cnt = unit_count<N>(c, r);
        load_unit<MB, ST, N, false, V>(c, r, cnt, in);
    }
}

// The short route's update terms of one unit of one lane: th1 = thd -
// (lr2 mhat) / (sq + eps2) with sq = sqrt(vhat) 2^32, and the smallest key
// of the nonzero numerators (see step_finish).  Once a bias correction
// rounds to 1 in fp32, dividing by it is exact: BC1 takes mhat = m1 (from
// t = 165 with beta1 = 0.9), BC2 vhat = v1 (from t = 17321 with beta2 =
// 0.999; the short sqrt then takes v1 itself, subnormal values included).
// The BC1-only form converts v1 to fp64 opaquely: it then keeps its own
// copy of the quotient's sqrt, where the compiler would otherwise share the
// general form's and hold 16 more VGPRs (one wavefront per SIMD fewer).
template <int N, bool BC1, bool BC2>
__device__ __forceinline__ void update_terms(const float (&m1)[N], const float (&v1)[N],
                                             const float (&thd)[N], const StepScalars &sc,
                                             float (&th1)[N], float (&sq)[N], uint32_t &kmin)
{
#pragma unroll
    for (int j = 0; j < N; ++j) {
        const float mhat = BC1 ? m1[j] : math::div_markstein(m1[j], sc.bc1, sc.rbc1);
        sq[j] = BC2 ? math::sqrt_x2p32_zero_tiny(v1[j])
                    : math::sqrt_quot_x2p32<BC1>(v1[j], sc.inv_bc2s);
        const float den = sq[j] + sc.eps2;
        const float num = sc.lr2 * mhat;
        th1[j] = thd[j] - math::div_markstein(num, den, math::recip_cr(den));
        const uint32_t key = (__float_as_uint(num) << 1) - 1u;
        kmin = key < kmin ? key : kmin;
    }
}

// The rest of one unit of one lane, from its loaded inputs: dequantize m and
// v (or read them as fp32), rebuild the master (or widen the bf16
// parameter), apply AdamW, find the group maxima (DPP exchanges among the
// group's lanes), and write scales and codes (or fp32 moments) and the new
// parameter (re-split, or cast to bf16).  Every lane of the wavefront calls
// this for the same unit.  FULL units use straight-line streaming stores; at
// the ragged end of a tensor stores are masked per element and groups padded
// with zeros.
template <int MB, int ST, int N, bool FULL>
__device__ __forceinline__ void step_finish(const ChunkPtrs &c, uint32_t r, int cnt, int lane,
                                            const UnitIn<MB, ST, N> &in, const StepScalars &sc,
                                            const float *s_mu, const float *s_vu)
{
    constexpr bool kQuant = ST != kStatesFp32;
    constexpr bool kComp = ST == kStatesCompanded;
    constexpr unsigned kVSpec = kComp ? FLASHOPT_SPEC_VARIANCE : FLASHOPT_SPEC_VARIANCE_LINEAR;
    const float ms = f16_value(in.smb);
    const float vs = f16_value(in.svb);

    // ---- dequantize, reconstruct, moments
    float thd[N], m1[N], v1[N];
    uint32_t vbits = 0u;                    // unsigned max of the v1 bit patterns
#pragma unroll
    for (int j = 0; j < N; ++j) {
        float theta;
        element_moments<MB, ST, N>(in, j, sc, s_mu, s_vu, ms, vs, theta, m1[j], v1[j]);
        thd[j] = theta * sc.cwd;
        vbits = max(vbits, __float_as_uint(v1[j]));
    }
    if (!FULL && kQuant) {                  // zero pad of the ragged last group
#pragma unroll
        for (int j = 0; j < N; ++j)
            if (j >= cnt) { m1[j] = 0.0f; v1[j] = 0.0f; }
    }

    // ---- unit maximum of |m1| (the maxima start from the first element: a
    // group of NaNs only has a NaN maximum, as the IEEE maxNum reduction over
    // its elements gives)
    float am = fabsf(m1[0]);
#pragma unroll
    for (int j = 1; j < N; ++j) am = fmaxf(am, fabsf(m1[j]));

    // ---- the update in the page's order: mhat = m1 / bc1, vhat = v1 / bc2,
    // theta1 = thd - (lr mhat) / (sqrt(vhat) + eps).  mhat comes from
    // div_markstein with the correctly rounded 1 / bc1 (exact for the m1 the
    // checks below let through, with the host's bound on lr); sq = sqrt(vhat) 2^32 comes from
    // sqrt_quot_x2p32 (vhat formed inside it; a subnormal or zero vhat gives
    // sq below 2^-31 instead of its exact root, lost in sq + eps2 while
    // eps >= 2^-38), and the division runs on the
    // 2^32-scaled numerator lr2 mhat and denominator sq + eps2 (the same
    // quotient), through the short division where its domain holds: every v1
    // below v1_bound (vhat < 2^63, so the denominator stays below 2^64),
    // |m1| <= m1_max (numerators at most 2^100 eps2) and every nonzero
    // numerator at least 2^-61 (>= 2^-126 times any denominator, and the
    // unscaled product lr mhat is normal, so scaling it was exact)
    uint32_t kmin = 0xFFFFFFFFu;          // min over nonzero |num| of its doubled pattern - 1
    float th1[N], sq[N];
    if (sc.unit_bc == 3) update_terms<N, true, true>(m1, v1, thd, sc, th1, sq, kmin);
    else if (sc.unit_bc & 1) update_terms<N, true, false>(m1, v1, thd, sc, th1, sq, kmin);
    else update_terms<N, false, false>(m1, v1, thd, sc, th1, sq, kmin);
    // NaN-propagating maximum (v_maximum3_f32): NaN iff some th1 is NaN
    float tnan = th1[0];
#pragma unroll
    for (int j = 1; j < N; ++j) tnan = __builtin_elementwise_maximum(tnan, th1[j]);
    const bool any_nan = tnan != tnan;
    const bool vfast = vbits < sc.v1_bound;   // the update's and the short variance codes' v range
    const bool exact = sc.fast == 0 || !vfast || !(am <= sc.m1_max) || kmin < sc.num_key || any_nan;

    // ---- group maxima, scales, variance codes
    uint32_t mo[N / 4], vo[N / 4], po[param_words(MB, N)], ro[rho_words(MB, N)];
    uint32_t sm_out = 0u, sv_out = 0u;
    if constexpr (kQuant) {
        sm_out = f16_bits(group_max<32 / N>(am));
        if constexpr (kComp) {
            // the group's largest sqrt(v1), 2^32-scaled: sqrt of the largest
            // v1 (sqrt is monotone; v1 = 0 gives 2^-63, whose scale is 0)
            float rmax;
            if (vbits < kSqrtFastEnd) {
                rmax = math::sqrt_x2p32_zero_tiny(__uint_as_float(vbits));
            } else {                            // rare: some v1 outside [0, 2^64): maxNum of the sqrts
                rmax = sqrtf(v1[0]) * 0x1p32f;
#pragma unroll
                for (int j = 1; j < N; ++j) rmax = fmaxf(rmax, sqrtf(v1[j]) * 0x1p32f);
            }
            sv_out = f16_bits(group_max<32 / N>(rmax) * 0x1p-32f);
            variance_codes<N>(sq, v1, sv_out, sc.kv, !vfast, vo);
        } else {
            float av = v1[0];
#pragma unroll
            for (int j = 1; j < N; ++j) av = fmaxf(av, v1[j]);
            sv_out = f16_bits(group_max<32 / N>(av));
            encode<kVSpec, N>(v1, group_div(sv_out), vo);
        }
    }

    // ---- momentum codes and the new parameter
    if (!exact) {
        if constexpr (kComp) encode_s8_softsign_fast<N>(m1, sm_out, mo);
        else if constexpr (kQuant) encode_s8_finite<false, N>(m1, group_div(sm_out), mo);
        pack_theta<MB, false, N>(th1, po, ro);
    } else {
        // rare: a unit outside the short sequences' domains (tiny or huge
        // numerators, NaN or infinite m or theta, unusual hyper-parameters)
        // is recomputed from its inputs in memory with the generic
        // operations; nothing has been stored yet, and the group scales
        // above are already exact
        unit_exact<MB, ST, N>(c, r, cnt, sc, s_mu, s_vu, sm_out, mo, po, ro);
    }

    // ---- stores
    uint32_t mb[N], vb[N];
#pragma unroll
    for (int j = 0; j < N; ++j) { mb[j] = __float_as_uint(m1[j]); vb[j] = __float_as_uint(v1[j]); }
    if (FULL) {
        if constexpr (MB == kParamF32) st_words<4 * N>(at(c.param32, r), po);
        else st_words<2 * N>(at(c.param, r), po);
        if constexpr (MB == 24) st_words<N>(c.rho8 + r, ro);
        if constexpr (MB == 32) st_words<2 * N>(at(c.rho16, r), ro);
        if constexpr (kQuant) {
            st_words<N>(c.mc + r, mo);
            st_words<N>(c.vc + r, vo);
        } else {
            st_words<4 * N>(at(c.mf, r), mb);
            st_words<4 * N>(at(c.vf, r), vb);
        }
    } else {
        if constexpr (MB == kParamF32) st_elems<4, N>(c.param32 + r, cnt, po);
        else st_elems<2, N>(c.param + r, cnt, po);
        if constexpr (MB == 24) st_elems<1, N>(c.rho8 + r, cnt, ro);
        if constexpr (MB == 32) st_elems<2, N>(c.rho16 + r, cnt, ro);
        if constexpr (kQuant) {
            st_elems<1, N>(c.mc + r, cnt, mo);
            st_elems<1, N>(c.vc + r, cnt, vo);
        } else {
            st_elems<4, N>(c.mf + r, cnt, mb);
            st_elems<4, N>(c.vf + r, cnt, vb);
        }
    }
    // the group's first lane writes its scales
    if (kQuant && lane % (32 / N) == 0 && cnt > 0) {
        st_u16(c.ms + r / kGroup, static_cast<uint16_t>(sm_out));
        st_u16(c.vs + r / kGroup, static_cast<uint16_t>(sv_out));
    }
}

// ------------------------------------------------------------ FlashSGD

// The rest of one FlashSGD unit of one lane, from its loaded inputs (the
// loads as load_chunk_unit with V = false): SGD with momentum (the buffer set
// to the gradient at step 1, coupled weight decay, optional dampening and
// Nesterov), the momentum buffer stored as group-32 codes (or fp32), the
// master re-split.
// There is no division: only non-finite values need the element-wise
// NaN-safe encoders, which run on the same registers.
template <int MB, int ST, int N, bool FULL>
__device__ __forceinline__ void sgd_finish(const ChunkPtrs &c, uint32_t r, int cnt, int lane,
                                           const UnitIn<MB, ST, N> &in, const SgdScalars &sc,
                                           const float *s_mu)
{
    constexpr bool kQuant = ST != kStatesFp32;
    constexpr bool kComp = ST == kStatesCompanded;
    constexpr unsigned kMSpec = kComp ? FLASHOPT_SPEC_MOMENTUM : FLASHOPT_SPEC_MOMENTUM_LINEAR;
    const float ms = f16_value(in.smb);

    float th1[N], b1[N];
    bool bad = false;                        // a non-finite buffer value or a NaN result
#pragma unroll
    for (int j = 0; j < N; ++j) {
        float theta;
        if constexpr (MB == 0) theta = (j & 1) ? bf16_hi(in.pw[j >> 1]) : bf16_lo(in.pw[j >> 1]);
        else theta = reconstruct_perm<MB>(in.pw, in.rw, j);
        float d = (j & 1) ? bf16_hi(in.gw[j >> 1]) : bf16_lo(in.gw[j >> 1]);
        if (sc.has_wd) {
            const float decay = sc.wd * theta;
            d = d + decay;
        }
        float b;
        if (sc.first) {
            b = d;
        } else {
            const float b0 = kQuant ? s_mu[ubyte(in.mw, j)] * ms : __uint_as_float(in.mf[j]);
            const float kept = sc.mu * b0;
            const float added = sc.cd * d;
            b = kept + added;
        }
        float dir = b;
        if (sc.nesterov) {
            const float look = sc.mu * b;
            dir = d + look;
        }
        const float upd = sc.lr * dir;
        th1[j] = theta - upd;
        b1[j] = (!FULL && kQuant && j >= cnt) ? 0.0f : b;   // zero pad of a ragged group
        bad |= !(fabsf(b1[j]) <= 0x1.fffffep127f) || th1[j] != th1[j];
    }

    uint32_t mo[N / 4], po[N / 2], ro[rho_words(MB, N)];
    uint32_t sm_out = 0u;
    if constexpr (kQuant) {
        float am = fabsf(b1[0]);
#pragma unroll
        for (int j = 1; j < N; ++j) am = fmaxf(am, fabsf(b1[j]));
        sm_out = f16_bits(group_max<32 / N>(am));
        if (!bad) {
            if constexpr (kComp) encode_s8_softsign_fast<N>(b1, sm_out, mo);
            else encode_s8_finite<false, N>(b1, group_div(sm_out), mo);
        }
        else encode<kMSpec, N>(b1, group_div(sm_out), mo);
    }
    if (!bad) pack_theta<MB, false, N>(th1, po, ro);
    else pack_theta<MB, true, N>(th1, po, ro);

    uint32_t bb[N];
#pragma unroll
    for (int j = 0; j < N; ++j) bb[j] = __float_as_uint(b1[j]);
    if (FULL) {
        st_words<2 * N>(at(c.param, r), po);
        if constexpr (MB == 24) st_words<N>(c.rho8 + r, ro);
        if constexpr (MB == 32) st_words<2 * N>(at(c.rho16, r), ro);
        if constexpr (kQuant) st_words<N>(c.mc + r, mo);
        else st_words<4 * N>(c.mf + r, bb);
    } else {
        st_elems<2, N>(c.param + r, cnt, po);
        if constexpr (MB == 24) st_elems<1, N>(c.rho8 + r, cnt, ro);
        if constexpr (MB == 32) st_elems<2, N>(c.rho16 + r, cnt, ro);
        if constexpr (kQuant) st_elems<1, N>(c.mc + r, cnt, mo);
        else st_elems<4, N>(c.mf + r, cnt, bb);
    }
    if (kQuant && lane % (32 / N) == 0 && cnt > 0) st_u16(c.ms + r / kGroup, static_cast<uint16_t>(sm_out));
}

// ------------------------------------------------------------- kernels

// Workgroup index renumbered so that each of the 8 XCDs takes one contiguous
// eighth of the grid: the dispatcher hands workgroups to the XCDs round-robin
// by index, so workgroup b runs on XCD b % 8, and with this order every XCD's
// L2 streams through a single contiguous region of the chunk space.  A
// permutation of [0, gridDim.x): XCD x takes `per` (or, when the grid is not
// a multiple of 8 and x > nb % 8, per - 1) consecutive numbers.
__device__ __forceinline__ uint32_t xcd_contiguous_block()
{
    const uint32_t nb = gridDim.x, b = blockIdx.x, x = b % 8u;
    const uint32_t per = (nb + 7u) / 8u, full = nb % 8u;
    uint32_t lb = x * per + b / 8u;
    if (full != 0u && x > full) lb -= x - full;
    return lb;
}

// Grid: one wavefront per unit, W units to a chunk, for the chunks
// [chunk_base, chunk_end) of the list (a list too long for one launch takes
// several, see launch_units; wavefronts past chunk_end, from rounding the
// grid up to whole workgroups, have no unit); a chunk never straddles two
// tensors.  Wavefronts are numbered in xcd_contiguous_block() order.  A
// wavefront finds the tensor owning its chunk by binary search over the
// chunk table (scalar loads, uniform across the wavefront).
//
// One unit per wavefront rather than a whole chunk: a wavefront's loads wait
// for its own earlier stores (one counter covers both), so a second unit in
// the same wavefront would start only once the first unit's stores had
// drained.  Split across wavefronts, a unit's loads go out while other
// wavefronts' stores are still in flight.
//
// Order within a wavefront: locate the unit and issue its loads (load),
// then build the workgroup's LDS tables and meet its barrier (tables: every
// wavefront calls it exactly once, at this one point, with or without a
// unit), then finish the unit (finish).  With the loads in flight first, the
// table build and the barrier overlap their latency instead of delaying
// them.
template <int W, typename Load, typename Tables, typename Finish>
__device__ __forceinline__ void for_each_unit(const DevTensor *__restrict__ tensors,
                                              const int32_t *__restrict__ chunk_start,
                                              int n_tensors, int32_t chunk_base,
                                              int32_t chunk_end, const StateLayout &L, Load &&load,
                                              Tables &&tables, Finish &&finish)
{
    // a launch has at most 2^24 workgroups (its work-items fit in 32 bits);
    // every quantity here is uniform and stays in scalar registers
    const uint32_t wave = xcd_contiguous_block() * (kBlockThreads / kWaveLanes) +
                          (__builtin_amdgcn_readfirstlane(threadIdx.x) >> 6);
    const int unit = static_cast<int>(wave % W);
    // chunk_base + wave / W < 2^31 + 2^25 fits in 32 unsigned bits
    const uint32_t cu = static_cast<uint32_t>(chunk_base) + wave / W;
    const bool any = cu < static_cast<uint32_t>(chunk_end);
    ChunkPtrs cp{};
    if (any) {
        // chunk indices fit in int32 (the host caps the total), so the
        // search compares in scalar registers: the last tensor whose first
        // chunk is <= c
        const int32_t c = static_cast<int32_t>(cu);
        int lo = 0, hi = n_tensors - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (chunk_start[mid] <= c) lo = mid;
            else hi = mid - 1;
        }
        const int t = __builtin_amdgcn_readfirstlane(lo);
        cp = chunk_ptrs(tensors[t], c - chunk_start[t], L);
        load(cp, unit);
    }
    tables();
    if (any) finish(cp);
}

// The same for one tensor (no chunk table): chunk c starts at element 1024 c.
template <int W, typename Load, typename Tables, typename Finish>
__device__ __forceinline__ void for_each_unit_of(const DevTensor &d, int32_t chunk_base,
                                                 int32_t chunk_end, const StateLayout &L,
                                                 Load &&load, Tables &&tables, Finish &&finish)
{
    const int32_t wave = __builtin_amdgcn_readfirstlane(
        static_cast<int32_t>(blockIdx.x) * (kBlockThreads / kWaveLanes) +
        static_cast<int32_t>(threadIdx.x >> 6));
    const int unit = wave % W;
    const int64_t c64 = static_cast<int64_t>(chunk_base) + wave / W;
    const bool any = c64 < chunk_end;
    ChunkPtrs cp{};
    if (any) {
        cp = chunk_ptrs(d, static_cast<int32_t>(c64), L);
        load(cp, unit);
    }
    tables();
    if (any) finish(cp);
}

// This thread's entries of the workgroup's dequantization tables (momentum:
// q/127, companded / (2 - |.|); variance: q/255), loaded at the start of a
// step kernel; build_tables writes them to LDS and meets the workgroup
// barrier (neither for fp32 states, which use no tables).
struct TableEntries {
    float mu, vu;
};

template <int ST, bool V>
__device__ __forceinline__ TableEntries table_entries()
{
    TableEntries e{0.0f, 0.0f};
    if constexpr (ST != kStatesFp32) {
        constexpr unsigned kMSpec =
            ST == kStatesCompanded ? FLASHOPT_SPEC_MOMENTUM : FLASHOPT_SPEC_MOMENTUM_LINEAR;
        e.mu = kDequantTable<kMSpec>.v[threadIdx.x];
        if constexpr (V) e.vu = kDequantTable<0u>.v[threadIdx.x];
    }
    return e;
}

template <int ST, bool V>
__device__ __forceinline__ void build_tables(const TableEntries &e, float *s_mu, float *s_vu)
{
    if constexpr (ST != kStatesFp32) {
        s_mu[threadIdx.x] = e.mu;
        if constexpr (V) s_vu[threadIdx.x] = e.vu;
        __syncthreads();
    }
}

// The fused FlashAdamW step.  With quantized states each workgroup holds
// the two 256-entry dequantization tables in LDS.  The step's scalars are read from the
// staged table (scalar loads, uniform across the wavefront), not from the
// kernel arguments, so that a captured launch steps with whatever scalars
// were written there before it runs.
template <int MB, int ST>
__global__ void __launch_bounds__(kBlockThreads)
adamw_step_kernel(const StepScalars *__restrict__ scalars, const DevTensor *__restrict__ tensors,
                  const int32_t *__restrict__ chunk_start, int n_tensors, int32_t chunk_base,
                  int32_t chunk_end)
{
    const StepScalars sc = *scalars;
    constexpr int kN = unit_elems(MB, ST);
    constexpr int kUnits = kLaneElems / kN;
    __shared__ float s_mu[256];
    __shared__ float s_vu[256];
    const TableEntries te = table_entries<ST, true>();
    const int lane = threadIdx.x & (kWaveLanes - 1);
    UnitIn<MB, ST, kN> in;
    uint32_t r = 0u;
    int cnt = 0;
    for_each_unit<kUnits>(
        tensors, chunk_start, n_tensors, chunk_base, chunk_end, sc.blk,
        [&](const ChunkPtrs &cp, int u) { load_chunk_unit<MB, ST, kN>(cp, u, lane, r, cnt, in); },
        [&] { build_tables<ST, true>(te, s_mu, s_vu); },
        [&](const ChunkPtrs &cp) {
            if (cp.rem == kChunkElems) step_finish<MB, ST, kN, true>(cp, r, cnt, lane, in, sc, s_mu, s_vu);
            else step_finish<MB, ST, kN, false>(cp, r, cnt, lane, in, sc, s_mu, s_vu);
        });
}

// The fused FlashSGD step (same grid and tables, momentum only; scalars read
// from the staged table like the AdamW step's).
template <int MB, int ST>
__global__ void __launch_bounds__(kBlockThreads)
sgd_step_kernel(const SgdScalars *__restrict__ scalars, const DevTensor *__restrict__ tensors,
                const int32_t *__restrict__ chunk_start, int n_tensors, int32_t chunk_base,
                int32_t chunk_end)
{
    const SgdScalars sc = *scalars;
    constexpr int kN = unit_elems(MB, ST);
    constexpr int kUnits = kLaneElems / kN;
    __shared__ float s_mu[256];
    const TableEntries te = table_entries<ST, false>();
    const int lane = threadIdx.x & (kWaveLanes - 1);
    UnitIn<MB, ST, kN> in;
    uint32_t r = 0u;
    int cnt = 0;
    for_each_unit<kUnits>(
        tensors, chunk_start, n_tensors, chunk_base, chunk_end, sc.blk,
        [&](const ChunkPtrs &cp, int u) { load_chunk_unit<MB, ST, kN, false>(cp, u, lane, r, cnt, in); },
        [&] { build_tables<ST, false>(te, s_mu, nullptr); },
        [&](const ChunkPtrs &cp) {
            if (cp.rem == kChunkElems) sgd_finish<MB, ST, kN, true>(cp, r, cnt, lane, in, sc, s_mu);
            else sgd_finish<MB, ST, kN, false>(cp, r, cnt, lane, in, sc, s_mu);
        });
}

// Single-tensor forms (the descriptor travels in the kernel arguments, no
// chunk table).
template <int MB, int ST>
__global__ void __launch_bounds__(kBlockThreads)
adamw_tensor_kernel(DevTensor d, StepScalars sc, int32_t chunk_base, int32_t chunk_end)
{
    constexpr int kN = unit_elems(MB, ST);
    constexpr int kUnits = kLaneElems / kN;
    __shared__ float s_mu[256];
    __shared__ float s_vu[256];
    const TableEntries te = table_entries<ST, true>();
    const int lane = threadIdx.x & (kWaveLanes - 1);
    UnitIn<MB, ST, kN> in;
    uint32_t r = 0u;
    int cnt = 0;
    for_each_unit_of<kUnits>(
        d, chunk_base, chunk_end, sc.blk,
        [&](const ChunkPtrs &cp, int u) { load_chunk_unit<MB, ST, kN>(cp, u, lane, r, cnt, in); },
        [&] { build_tables<ST, true>(te, s_mu, s_vu); },
        [&](const ChunkPtrs &cp) {
            if (cp.rem == kChunkElems) step_finish<MB, ST, kN, true>(cp, r, cnt, lane, in, sc, s_mu, s_vu);
            else step_finish<MB, ST, kN, false>(cp, r, cnt, lane, in, sc, s_mu, s_vu);
        });
}

template <int MB, int ST>
__global__ void __launch_bounds__(kBlockThreads)
sgd_tensor_kernel(DevTensor d, SgdScalars sc, int32_t chunk_base, int32_t chunk_end)
{
    constexpr int kN = unit_elems(MB, ST);
    constexpr int kUnits = kLaneElems / kN;
    __shared__ float s_mu[256];
    const TableEntries te = table_entries<ST, false>();
    const int lane = threadIdx.x & (kWaveLanes - 1);
    UnitIn<MB, ST, kN> in;
    uint32_t r = 0u;
    int cnt = 0;
    for_each_unit_of<kUnits>(
        d, chunk_base, chunk_end, sc.blk,
        [&](const ChunkPtrs &cp, int u) { load_chunk_unit<MB, ST, kN, false>(cp, u, lane, r, cnt, in); },
        [&] { build_tables<ST, false>(te, s_mu, nullptr); },
        [&](const ChunkPtrs &cp) {
            if (cp.rem == kChunkElems) sgd_finish<MB, ST, kN, true>(cp, r, cnt, lane, in, sc, s_mu);
            else sgd_finish<MB, ST, kN, false>(cp, r, cnt, lane, in, sc, s_mu);
        });
}

// ------------------------------------------------------------- launching

unsigned grid_for(int64_t n)
{
    const int64_t per_block = static_cast<int64_t>(kBlockThreads) * kLaneElems;
    return static_cast<unsigned>((n + per_block - 1) / per_block);
}

int64_t launch_chunks(int units_per_chunk);

// Launches of a split or reconstruct kernel with U units per wavefront over
// n elements: one workgroup per block of 1024 U elements, at most
// launch_chunks(4) blocks per launch (in order on one stream); each launch
// gets its first block after the arguments passed through.
template <int U, typename Kernel, typename... Args>
hipError_t launch_flat(Kernel kernel, int64_t n, hipStream_t st, Args... args)
{
    const int64_t per_block = static_cast<int64_t>(kChunkElems) * U;
    const int64_t blocks = (n + per_block - 1) / per_block;
    const int64_t per = launch_chunks(kBlockThreads / kWaveLanes);
    for (int64_t base = 0; base < blocks; base += per) {
        const int64_t k = blocks - base < per ? blocks - base : per;
        hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(k)), dim3(kBlockThreads), 0, st,
                           args..., base);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <unsigned SPEC>
hipError_t quantize_spec(const float *x, int64_t n, void *codes, uint16_t *scales, hipStream_t st)
{
    hipLaunchKernelGGL(quantize_kernel<SPEC>, dim3(grid_for(n)), dim3(kBlockThreads), 0, st,
                       x, n, codes, scales);
    return hipGetLastError();
}

template <unsigned SPEC>
hipError_t dequantize_spec(const void *codes, const uint16_t *scales, int64_t n, float *out,
                           hipStream_t st)
{
    hipLaunchKernelGGL(dequantize_kernel<SPEC>, dim3(grid_for(n)), dim3(kBlockThreads), 0, st,
                       codes, scales, n, out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const float *x, int64_t n, unsigned spec, void *codes,
                           uint16_t *scales, hipStream_t st)
{
    switch (spec & 7u) {
    case 0: return quantize_spec<0>(x, n, codes, scales, st);
    case 1: return quantize_spec<1>(x, n, codes, scales, st);
    case 2: return quantize_spec<2>(x, n, codes, scales, st);
    case 3: return quantize_spec<3>(x, n, codes, scales, st);
    case 4: return quantize_spec<4>(x, n, codes, scales, st);
    case 5: return quantize_spec<5>(x, n, codes, scales, st);
    case 6: return quantize_spec<6>(x, n, codes, scales, st);
    default: return quantize_spec<7>(x, n, codes, scales, st);
    }
}

hipError_t launch_dequantize(const void *codes, const uint16_t *scales, int64_t n, unsigned spec,
                             float *out, hipStream_t st)
{
    switch (spec & 7u) {
    case 0: return dequantize_spec<0>(codes, scales, n, out, st);
    case 1: return dequantize_spec<1>(codes, scales, n, out, st);
    case 2: return dequantize_spec<2>(codes, scales, n, out, st);
    case 3: return dequantize_spec<3>(codes, scales, n, out, st);
    case 4: return dequantize_spec<4>(codes, scales, n, out, st);
    case 5: return dequantize_spec<5>(codes, scales, n, out, st);
    case 6: return dequantize_spec<6>(codes, scales, n, out, st);
    default: return dequantize_spec<7>(codes, scales, n, out, st);
    }
}

hipError_t launch_split(const float *master, int64_t n, int master_bits, uint16_t *param,
                        void *rho, hipStream_t st)
{
    if (master_bits == 32)
        return launch_flat<split_units(32, false)>(split_kernel<32>, n, st, master, n, param, rho);
    return launch_flat<split_units(24, false)>(split_kernel<24>, n, st, master, n, param, rho);
}

hipError_t launch_reconstruct(const uint16_t *param, const void *rho, int64_t n, int master_bits,
                              float *master, hipStream_t st)
{
    if (master_bits == 32)
        return launch_flat<split_units(32, true)>(reconstruct_kernel<32>, n, st, param, rho, n, master);
    return launch_flat<split_units(24, true)>(reconstruct_kernel<24>, n, st, param, rho, n, master);
}

namespace {

// Chunks per launch: as many as one dispatch's 32-bit count of work-items
// allows (2^24 - 1 workgroups of four wavefronts, one wavefront per unit),
// or fewer when FLASHOPT_LAUNCH_CHUNKS asks for it (a test hook that makes
// small lists take several launches).
int64_t launch_chunks(int units_per_chunk)
{
    int64_t n = (static_cast<int64_t>(UINT32_MAX) / kBlockThreads) * (kBlockThreads / kWaveLanes) /
                units_per_chunk;
    if (const char *env = getenv("FLASHOPT_LAUNCH_CHUNKS")) {
        const long long v = atoll(env);
        if (v >= 1 && v < n) n = v;
    }
    return n;
}

// Launches kernel K over chunks [0, total_chunks) of a list, in as many
// launches as launch_chunks requires (one on any list that fits in HBM), each
// given its chunk range after the arguments passed through.
template <int MB, int ST, typename Kernel, typename... Args>
hipError_t launch_units(Kernel kernel, int32_t total_chunks, hipStream_t st, Args... args)
{
    constexpr int units = kLaneElems / unit_elems(MB, ST);
    const int64_t per = launch_chunks(units);
    for (int64_t base = 0; base < total_chunks; base += per) {
        const int64_t n = total_chunks - base < per ? total_chunks - base : per;
        const int64_t waves = n * units;
        const unsigned grid = static_cast<unsigned>((waves + kBlockThreads / kWaveLanes - 1) /
                                                    (kBlockThreads / kWaveLanes));
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(kBlockThreads), 0, st, args...,
                           static_cast<int32_t>(base), static_cast<int32_t>(base + n));
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int MB, int ST>
hipError_t step_variant(const DevTensor *tensors, const int32_t *chunk_start, int n_tensors,
                        int32_t total_chunks, const StepScalars *scalars, hipStream_t st)
{
    return launch_units<MB, ST>(adamw_step_kernel<MB, ST>, total_chunks, st, scalars, tensors,
                                chunk_start, n_tensors);
}

template <int MB, int ST>
hipError_t sgd_variant(const DevTensor *tensors, const int32_t *chunk_start, int n_tensors,
                       int32_t total_chunks, const SgdScalars *scalars, hipStream_t st)
{
    return launch_units<MB, ST>(sgd_step_kernel<MB, ST>, total_chunks, st, scalars, tensors,
                                chunk_start, n_tensors);
}

// The (master_bits, states) instantiations of one step kernel family: nine,
// plus the three fp32-parameter ones where the family has them.
template <template <int, int> class K, typename Sc>
hipError_t dispatch(int master_bits, int states, const DevTensor *tensors,
                    const int32_t *chunk_start, int n_tensors, int32_t total_chunks,
                    const Sc &sc, hipStream_t st)
{
    switch (master_bits * 4 + states) {
    case 24 * 4 + kStatesCompanded: return K<24, kStatesCompanded>::run(tensors, chunk_start, n_tensors, total_chunks, sc, st);
    case 24 * 4 + kStatesLinear: return K<24, kStatesLinear>::run(tensors, chunk_start, n_tensors, total_chunks, sc, st);
    case 24 * 4 + kStatesFp32: return K<24, kStatesFp32>::run(tensors, chunk_start, n_tensors, total_chunks, sc, st);
    case 32 * 4 + kStatesCompanded: return K<32, kStatesCompanded>::run(tensors, chunk_start, n_tensors, total_chunks, sc, st);
    case 32 * 4 + kStatesLinear: return K<32, kStatesLinear>::run(tensors, chunk_start, n_tensors, total_chunks, sc, st);
    case 32 * 4 + kStatesFp32: return K<32, kStatesFp32>::run(tensors, chunk_start, n_tensors, total_chunks, sc, st);
    case kStatesCompanded: return K<0, kStatesCompanded>::run(tensors, chunk_start, n_tensors, total_chunks, sc, st);
    case kStatesLinear: return K<0, kStatesLinear>::run(tensors, chunk_start, n_tensors, total_chunks, sc, st);
    case kStatesFp32: return K<0, kStatesFp32>::run(tensors, chunk_start, n_tensors, total_chunks, sc, st);
    default: break;
    }
    if constexpr (K<0, kStatesFp32>::kFp32Params) {
        switch (master_bits * 4 + states) {
        case kParamF32 * 4 + kStatesCompanded: return K<kParamF32, kStatesCompanded>::run(tensors, chunk_start, n_tensors, total_chunks, sc, st);
        case kParamF32 * 4 + kStatesLinear: return K<kParamF32, kStatesLinear>::run(tensors, chunk_start, n_tensors, total_chunks, sc, st);
        case kParamF32 * 4 + kStatesFp32: return K<kParamF32, kStatesFp32>::run(tensors, chunk_start, n_tensors, total_chunks, sc, st);
        default: break;
        }
    }
    return hipErrorInvalidValue;
}

// List launches: the scalars are a device pointer into the staged table.
template <int MB, int ST>
struct AdamWLaunch {
    static constexpr bool kFp32Params = true;
    static hipError_t run(const DevTensor *t, const int32_t *cs, int n, int32_t total,
                          const StepScalars *scalars, hipStream_t st)
    {
        return step_variant<MB, ST>(t, cs, n, total, scalars, st);
    }
};

template <int MB, int ST>
struct SgdLaunch {
    static constexpr bool kFp32Params = false;
    static hipError_t run(const DevTensor *t, const int32_t *cs, int n, int32_t total,
                          const SgdScalars *scalars, hipStream_t st)
    {
        return sgd_variant<MB, ST>(t, cs, n, total, scalars, st);
    }
};

// Single-tensor launches: t points to a host descriptor passed by value.
template <int MB, int ST>
struct AdamWTensorLaunch {
    static constexpr bool kFp32Params = true;
    static hipError_t run(const DevTensor *t, const int32_t *, int, int32_t total,
                          const StepScalars &sc, hipStream_t st)
    {
        return launch_units<MB, ST>(adamw_tensor_kernel<MB, ST>, total, st, *t, sc);
    }
};

template <int MB, int ST>
struct SgdTensorLaunch {
    static constexpr bool kFp32Params = false;
    static hipError_t run(const DevTensor *t, const int32_t *, int, int32_t total,
                          const SgdScalars &sc, hipStream_t st)
    {
        return launch_units<MB, ST>(sgd_tensor_kernel<MB, ST>, total, st, *t, sc);
    }
};

}  // namespace

// ------------------------------------ scratch of the allocation-free step

// The scalar block and chunk table of flashopt_adamw_step_noalloc: a device
// array of this file instead of a caller's workspace.  Every GPU the library
// runs on holds its own copy until the process ends.  In host code the name
// stands for a host-side shadow, not a device address, so host code reaches
// the array only through the address hipGetSymbolAddress returns for the
// current device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_address(void **ptr)
{
    constexpr int kDevices = 64;
    static std::mutex mu;
    static void *addr[kDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_adamw_step(const StepScalars *scalars, const DevTensor *tensors,
                             const int32_t *chunk_start, int n_tensors, int32_t total_chunks,
                             int master_bits, int states, hipStream_t st)
{
    if (total_chunks <= 0) return hipSuccess;
    return dispatch<AdamWLaunch>(master_bits, states, tensors, chunk_start, n_tensors,
                                 total_chunks, scalars, st);
}

hipError_t launch_sgd_step(const SgdScalars *scalars, const DevTensor *tensors,
                           const int32_t *chunk_start, int n_tensors, int32_t total_chunks,
                           int master_bits, int states, hipStream_t st)
{
    if (total_chunks <= 0) return hipSuccess;
    return dispatch<SgdLaunch>(master_bits, states, tensors, chunk_start, n_tensors,
                               total_chunks, scalars, st);
}

hipError_t launch_adamw_tensor(const DevTensor &d, const StepScalars &sc, int master_bits,
                               int states, hipStream_t st)
{
    const int64_t chunks = (d.numel + kChunkElems - 1) / kChunkElems;
    if (chunks <= 0) return hipSuccess;
    return dispatch<AdamWTensorLaunch>(master_bits, states, &d, nullptr, 1,
                                       static_cast<int32_t>(chunks), sc, st);
}

hipError_t launch_sgd_tensor(const DevTensor &d, const SgdScalars &sc, int master_bits,
                             int states, hipStream_t st)
{
    const int64_t chunks = (d.numel + kChunkElems - 1) / kChunkElems;
    if (chunks <= 0) return hipSuccess;
    return dispatch<SgdTensorLaunch>(master_bits, states, &d, nullptr, 1,
                                     static_cast<int32_t>(chunks), sc, st);
}

}  // namespace flashopt
