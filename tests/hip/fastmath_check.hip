// GPU check of the short exact fp32 sequences in flashopt_math.h against the
// compiler's correctly rounded division and sqrt on the same device.  Built
// in-tree as libfastmath_check.so and driven by tests/test_gpu_fastmath.py.
// Each entry point runs one exhaustive (or large structured) sweep and returns
// the number of mismatching inputs, or -1 on a HIP error.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flashopt_math.h"

using namespace flashopt::math;

namespace {

// per-thread count, one atomic per thread at the end
__device__ void flush(unsigned long long *bad, unsigned long long c)
{
    if (c) atomicAdd(bad, c);
}

__device__ __forceinline__ bool same(float a, float b) { return __float_as_uint(a) == __float_as_uint(b); }

__global__ void k_sqrt(unsigned long long *bad)
{
    unsigned long long c = 0;
    // every x in [0, 2^64): patterns 0 .. 0x5F7FFFFF
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < 0x5F800000ull;
         i += (uint64_t)gridDim.x * blockDim.x) {
        const float x = __uint_as_float((uint32_t)i);
        c += !same(sqrt_cr(x), sqrtf(x));
        c += !same(sqrt_x2p32_zero_tiny(x), i == 0 ? 0x1p-63f : sqrt_cr_x2p32(x));
    }
    flush(bad, c);
}

__global__ void k_recip(unsigned long long *bad)
{
    unsigned long long c = 0;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (1ull << 23);
         i += (uint64_t)gridDim.x * blockDim.x) {
        // every significand in [1, 2), at three exponents
        const float d = __uint_as_float(0x3F800000u | (uint32_t)i);
        c += !same(recip_cr(d), 1.0f / d);
        c += !same(recip_cr(d * 0x1p-60f), 1.0f / (d * 0x1p-60f));
        c += !same(recip_cr(d * 0x1p60f), 1.0f / (d * 0x1p60f));
        if (i < 0x7C00u && i > 0u) {       // every positive finite fp16 value
            const float h = (float)__builtin_bit_cast(_Float16, (unsigned short)i);
            c += !same(recip_cr(h), 1.0f / h);
        }
    }
    flush(bad, c);
}

__global__ void k_div_by_recip(unsigned long long *bad)
{
    unsigned long long c = 0;
    // every fp16 divisor significand (10 bits) x every dividend significand
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (1ull << 33);
         i += (uint64_t)gridDim.x * blockDim.x) {
        const float d = __uint_as_float(0x3F800000u | ((uint32_t)(i >> 23) << 13));
        const float a = __uint_as_float(0x3F800000u | (uint32_t)(i & 0x7FFFFFu));
        c += !same(div_by_recip(a, d, recip_cr(d)), a / d);
    }
    flush(bad, c);
}

__global__ void k_softsign(unsigned long long *bad)
{
    unsigned long long c = 0;
    // every y in [0, 1.5] (the sequence is odd-symmetric in y)
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i <= 0x3FC00000ull;
         i += (uint64_t)gridDim.x * blockDim.x) {
        const float y = __uint_as_float((uint32_t)i);
        const float num = 2.0f * y;
        const float den = 1.0f + fabsf(y);
        c += !same(softsign(y), num / den);
        if (y != 0.0f) c += !same(softsign(-y), (-num) / den);
    }
    flush(bad, c);
}

__global__ void k_cvt_pk_u8(unsigned long long *bad)
{
    unsigned long long c = 0;
    // every fp32 pattern: v_cvt_pk_u8_f32 == clamp(rint(x), 0, 255), NaN -> 0
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (1ull << 32);
         i += (uint64_t)gridDim.x * blockDim.x) {
        const float x = __uint_as_float((uint32_t)i);
        const unsigned got = __builtin_amdgcn_cvt_pk_u8_f32(x, 2, 0u) >> 16;
        unsigned want = 0u;
        if (x == x) want = (unsigned)fminf(fmaxf(rintf(x), 0.0f), 255.0f);
        c += got != want;
    }
    flush(bad, c);
}

__device__ __forceinline__ uint32_t mix(uint64_t i, uint32_t k)
{
    uint32_t h = (uint32_t)i * 2654435761u + k * 0x9E3779B9u + (uint32_t)(i >> 32) * 0x85EBCA6Bu;
    h ^= h >> 15; h *= 0x2C1B3C6Du; h ^= h >> 12; h *= 0x297A2D39u; h ^= h >> 15;
    return h;
}

// a float with random sign and significand and exponent field e (1..254)
__device__ __forceinline__ float with_exp(uint32_t e, uint32_t h) { return __uint_as_float((h & 0x807FFFFFu) | (e << 23)); }

__global__ void k_div_markstein(unsigned long long *bad)
{
    unsigned long long c = 0;
    // den: exponent field in [27, 227) (2^-100 .. 2^100); num: zero, or an
    // exponent field in [max(25, e_den - 125), min(254, e_den + 99)], i.e.
    // max(2^-102, 2^-126 den) <= |num| <= 2^100 den
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (1ull << 32);
         i += (uint64_t)gridDim.x * blockDim.x) {
        const uint32_t h1 = mix(i, 1), h2 = mix(i, 2), h3 = mix(i, 3);
        const uint32_t ed = 27u + h1 % 200u;
        const float den = __uint_as_float((ed << 23) | (h2 & 0x7FFFFFu));
        const uint32_t lo = ed >= 150u ? ed - 125u : 25u;
        const uint32_t hi = ed + 99u < 254u ? ed + 99u : 254u;
        float num;
        if ((h1 >> 26) == 0u) num = (h3 >> 31) ? -0.0f : 0.0f;
        else num = with_exp(lo + (h1 >> 8) % (hi - lo + 1u), h3);
        c += !same(div_markstein(num, den, recip_cr(den)), num / den);
    }
    // every divisor significand, numerators at the edges of the domain
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (1ull << 23);
         i += (uint64_t)gridDim.x * blockDim.x) {
        const uint32_t sig = (uint32_t)i;
        const uint32_t eds[3] = {27u, 127u, 226u};
        for (int a = 0; a < 3; ++a) {
            const uint32_t ed = eds[a];
            const float den = __uint_as_float((ed << 23) | sig);
            const uint32_t lo = ed >= 150u ? ed - 125u : 25u;
            const uint32_t hi = ed + 99u < 254u ? ed + 99u : 254u;
            const float nums[4] = {with_exp(lo, mix(i, 7)), with_exp(lo, 0u), with_exp(hi, mix(i, 8)),
                                   with_exp(hi, 0x7FFFFFu)};
            for (int b = 0; b < 4; ++b) c += !same(div_markstein(nums[b], den, recip_cr(den)), nums[b] / den);
        }
    }
    flush(bad, c);
}

__global__ void k_magic_code(unsigned long long *bad)
{
    unsigned long long c = 0;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (1ull << 32);
         i += (uint64_t)gridDim.x * blockDim.x) {
        const float p = __uint_as_float((uint32_t)i);
        if (p != p) continue;
        const int want = (int)fminf(fmaxf(rintf(p), -127.0f), 127.0f);
        c += (int)(int8_t)(code_s8_magic(p) & 0xFFu) != want;
    }
    flush(bad, c);
}

// Group divisors for the code check: every positive fp16 subnormal and every
// fp16 significand at three exponents (2^-10, 2^0, 2^14): 4095 values.
__device__ __forceinline__ float code_divisor(uint32_t i)
{
    if (i < 1023u) return (float)__builtin_bit_cast(_Float16, (unsigned short)(i + 1u));
    const uint32_t j = i - 1023u;
    const uint32_t e = (j >> 10) == 0 ? 5u : ((j >> 10) == 1 ? 15u : 29u);   // fp16 exponent field
    return (float)__builtin_bit_cast(_Float16, (unsigned short)((e << 10) | (j & 1023u)));
}

// The correctly rounded chain's code (encode_s8_finite's sequence).
__device__ __forceinline__ int exact_code(float m, float d)
{
    const float y = softsign(div_by_recip(m, d, recip_cr(d)));
    return (int)(int8_t)(code_s8_magic(y * 127.0f) & 0xFFu);
}

// softsign_code_bytes against the exact chain wherever its two bytes agree
// (GUARDED), or its upper byte everywhere (to show that the sweep reaches
// inputs where the short form alone would differ): for every divisor,
// 2 x 2048 dividends around each of the 127 positive rounding boundaries
// p = k + 1/2 (the map is odd), then 2^18 hashed dividends over
// [-d, d] (normal fp16 divisors: |m / d| <= 1 + 2^-11, the caller's range;
// the subnormal ones over [-(1 + 2^-11) d, (1 + 2^-11) d] as well).
template <bool GUARDED>
__global__ void k_softsign_code(unsigned long long *bad)
{
    constexpr uint64_t kW = 2048, kTies = 4095ull * 127ull * 2ull * kW, kRand = 4095ull << 18;
    unsigned long long c = 0;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < kTies + kRand;
         i += (uint64_t)gridDim.x * blockDim.x) {
        float d, m;
        if (i < kTies) {
            d = code_divisor((uint32_t)(i / (127ull * 2ull * kW)));
            const double pk = (double)((i / (2ull * kW)) % 127ull) + 0.5;
            const float ms = (float)(pk * (double)d / (254.0 - pk));     // p(ms) = k + 1/2
            m = __uint_as_float(__float_as_uint(ms) + (uint32_t)(i % (2ull * kW)) - (uint32_t)kW);
        } else {
            const uint64_t j = i - kTies;
            d = code_divisor((uint32_t)(j >> 18));
            uint32_t h = (uint32_t)j * 2654435761u;
            h ^= h >> 15; h *= 2246822519u; h ^= h >> 13;
            m = d * ((float)(h >> 8) * 0x1p-23f - 1.0f) * (1.0f + 0x1p-11f);
        }
        if (!(fabsf(m) <= d * (1.0f + 0x1p-11f))) continue;
        uint32_t hi, lo;
        softsign_code_bytes(m, m, m, m, d * kInv254, hi, lo);
        const int code = (int)(hi & 0xFFu) - 128;
        if (!GUARDED || hi == lo) c += code != exact_code(m, d);
    }
    flush(bad, c);
}

// Divisor k of the fp64-reciprocal division check: the fp32 bias
// corrections 1 - beta^t of eight betas for t = 1 .. 512 (4096 values), then
// 4096 hashed significands at exponents 2^-20 .. 2^0.
__device__ __forceinline__ float bias_divisor(uint32_t k)
{
    if (k < 4096u) {
        const double betas[8] = {0.9, 0.95, 0.99, 0.8, 0.999, 0.9999, 0.98, 0.5};
        return (float)(1.0 - pow(betas[k >> 9], (double)((k & 511u) + 1u)));
    }
    const uint32_t h = mix(k, 11);
    return __uint_as_float(((107u + h % 21u) << 23) | (h >> 9));
}

// The bias-correction quotient m / bc of the step: div_markstein with the
// correctly rounded reciprocal of bc (recip_cr) against the correctly rounded
// division, for every divisor above x every dividend significand with both
// signs, at a hashed exponent per significand from 2^-102 up to 2^85 (the
// range where the step takes this route: |m| >= 2^-102 and |m| <= 2^99 bc,
// bc >= 1e-4 here), plus the range's two ends and zero.
__global__ void k_div_bias(unsigned long long *bad)
{
    unsigned long long c = 0;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (8192ull << 23);
         i += (uint64_t)gridDim.x * blockDim.x) {
        const float d = bias_divisor((uint32_t)(i >> 23));
        const float r = recip_cr(d);
        const uint32_t sig = (uint32_t)i & 0x7FFFFFu;
        const uint32_t e = 25u + mix(i, 7) % 188u;                  // biased exponent: 2^-102 .. 2^85
        const float a = __uint_as_float((e << 23) | sig);
        c += !same(div_markstein(a, d, r), a / d);
        c += !same(div_markstein(-a, d, r), (-a) / d);
        if (sig < 4096u) {
            const float lo = __uint_as_float((25u << 23) | (mix(i, 8) & 0x807FFFFFu));   // |a| in [2^-102, 2^-101)
            c += !same(div_markstein(lo, d, r), lo / d);
            const float hi = __uint_as_float((212u << 23) | (mix(i, 9) & 0x807FFFFFu));  // |a| in [2^85, 2^86)
            c += !same(div_markstein(hi, d, r), hi / d);
        }
        if (sig == 0u) {
            c += !same(div_markstein(0.0f, d, r), 0.0f / d);
            c += !same(div_markstein(-0.0f, d, r), -0.0f / d);
        }
    }
    flush(bad, c);
}

// sqrt_quot_x2p32 for 16 bias-correction divisors (bias_divisor: t = 1, 2,
// 3, 512 of four betas) over every v pattern in [0, 2^64): where fl(v / b) is
// normal and below 2^63 it must equal sqrt_cr_x2p32(fl(v / b)); where the
// quotient is zero or subnormal it must be finite and below 2^-31.  The
// form with the opaque conversion must give the same bits everywhere.
__global__ void k_sqrt_quot(unsigned long long *bad)
{
    unsigned long long c = 0;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (16ull * 0x5F800000ull);
         i += (uint64_t)gridDim.x * blockDim.x) {
        const uint32_t k = (uint32_t)(i / 0x5F800000ull);
        const uint32_t sel[4] = {0u, 1u, 2u, 511u};
        const float b = bias_divisor(((k >> 2) << 9) + sel[k & 3u]);
        const float v = __uint_as_float((uint32_t)(i % 0x5F800000ull));
        const float q = v / b;
        if (!(q < 0x1p63f)) continue;
        const float got = sqrt_quot_x2p32(v, 0x1p64 / (double)b);
        c += !same(got, sqrt_quot_x2p32<true>(v, 0x1p64 / (double)b));
        if (q >= 0x1p-126f) c += !same(got, sqrt_cr_x2p32(q));
        else c += !(got >= 0.0f && got < 0x1p-31f);
    }
    flush(bad, c);
}

template <typename K>
long long run(K kernel, unsigned grid)
{
    unsigned long long *d = nullptr, h = 0;
    if (hipMalloc(&d, sizeof(h)) != hipSuccess) return -1;
    if (hipMemset(d, 0, sizeof(h)) != hipSuccess) { (void)hipFree(d); return -1; }
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(256), 0, 0, d);
    const bool ok = hipGetLastError() == hipSuccess && hipDeviceSynchronize() == hipSuccess &&
                    hipMemcpy(&h, d, sizeof(h), hipMemcpyDeviceToHost) == hipSuccess;
    (void)hipFree(d);
    return ok ? (long long)h : -1;
}

}  // namespace

extern "C" {
long long fastmath_check_sqrt(void) { return run(k_sqrt, 65536); }
long long fastmath_check_recip(void) { return run(k_recip, 8192); }
long long fastmath_check_div_by_recip(void) { return run(k_div_by_recip, 65536); }
long long fastmath_check_softsign(void) { return run(k_softsign, 65536); }
long long fastmath_check_cvt_pk_u8(void) { return run(k_cvt_pk_u8, 65536); }
long long fastmath_check_div_markstein(void) { return run(k_div_markstein, 65536); }
long long fastmath_check_div_bias(void) { return run(k_div_bias, 65536); }
long long fastmath_check_sqrt_quot(void) { return run(k_sqrt_quot, 65536); }
long long fastmath_check_magic_code(void) { return run(k_magic_code, 65536); }
long long fastmath_check_softsign_code(void) { return run(k_softsign_code<true>, 65536); }
long long fastmath_softsign_code_unguarded(void) { return run(k_softsign_code<false>, 65536); }
}
