// HIP kernels of libflashopt.so for gfx950 (MI355X): the group-32 state codec,
// the bf16 + rho weight split, and the fused FlashAdamW step.
//
// Method pages: "code/flashsim/quantization.py" (Alg. 2/3: quantize(),
// dequantize()), "code/flashsim/flash_adamw_sim.py" (Alg. 4:
// FlashAdamWSim.step()), "code/gpu/equivalence.py" (bf16 parameter and
// correction bits, eq_ecc()).
//
// Layout of the work: a lane owns 16 consecutive elements, so each element
// stream is read and written with 16-byte vector accesses (two for 16-bit
// streams, four for fp32); the lane pair (2k, 2k+1) owns one 32-element
// group and finishes the group max with one DPP exchange; a wavefront owns a
// 1024-element chunk.  The step is elementwise and memory-bound, so there is
// no MFMA and no LDS staging of data; LDS holds only the per-tensor chunk
// table and two 256-entry dequantization tables.
//
// Arithmetic: fp32, one IEEE rounding per operation in the written order
// (built with -ffp-contract=off, correctly rounded / and sqrt, fp32 and fp16
// denormals preserved), so results match a plain CPU evaluation bit for bit.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "flashopt.h"
#include "flashopt_internal.h"

namespace flashopt {
namespace {

// ----------------------------------------------------------------- helpers

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
// else the scale itself (quantize(): `where(scales == 0, 1, scales)`).
__device__ __forceinline__ float group_divisor(uint32_t s)
{
    return (s & 0x7FFFu) ? f16_value(s) : 1.0f;
}

// Maximum with the partner lane (lane ^ 1): DPP quad_perm [1, 0, 3, 2].
// Every lane of the wavefront must be active.
__device__ __forceinline__ float pair_max(float x)
{
    const int y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false);
    return fmaxf(x, __int_as_float(y));
}

// Byte j of a 16-byte register block, zero- or sign-extended.
__device__ __forceinline__ uint32_t ubyte(const uint32_t (&w)[4], int j)
{
    return (w[j >> 2] >> (8 * (j & 3))) & 0xFFu;
}
__device__ __forceinline__ int32_t sbyte(const uint32_t (&w)[4], int j)
{
    return static_cast<int32_t>(w[j >> 2] << (24 - 8 * (j & 3))) >> 24;
}
__device__ __forceinline__ int32_t shalf(const uint32_t (&w)[8], int j)
{
    return static_cast<int32_t>(w[j >> 1] << (16 - 16 * (j & 1))) >> 16;
}

// Dequantization before the scale: y = q/127 or q/255, then the softsign
// inverse y / (2 - |y|) (dequantize()).  Built once per workgroup into LDS;
// the table entries are these exact fp32 operations.
template <unsigned SPEC>
__device__ __forceinline__ float dequant_unit(int c)
{
    constexpr bool kSigned = (SPEC & FLASHOPT_Q_SIGNED) != 0;
    const float q = kSigned ? static_cast<float>(static_cast<int8_t>(c))
                            : static_cast<float>(static_cast<uint8_t>(c));
    float y = q / (kSigned ? 127.0f : 255.0f);
    if (SPEC & FLASHOPT_Q_SOFTSIGN) {
        const float den = 2.0f - fabsf(y);
        y = y / den;
    }
    return y;
}

// Code of one element from y = a / d (quantize()): softsign companding if
// asked, then round half to even of y*127 (signed, clamp [-127, 127]) or
// y*255 (unsigned, clamp [0, 255]).  A NaN gets code 0.  Returns the byte.
template <unsigned SPEC>
__device__ __forceinline__ uint32_t code_byte(float y)
{
    if (SPEC & FLASHOPT_Q_SOFTSIGN) {
        const float num = 2.0f * y;
        const float den = 1.0f + fabsf(y);
        y = num / den;
    }
    if (SPEC & FLASHOPT_Q_SIGNED) {
        float r = rintf(y * 127.0f);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        const int32_t q = (y != y) ? 0 : static_cast<int32_t>(r);
        return static_cast<uint32_t>(q) & 0xFFu;
    } else {
        float r = rintf(y * 255.0f);
        r = fminf(fmaxf(r, 0.0f), 255.0f);
        return (y != y) ? 0u : static_cast<uint32_t>(r);
    }
}

// Weight split of one fp32 value: theta' = nearest bf16 with ties away from
// zero, D = pattern(x) - (pattern(theta') << 16) in [-32768, 32767];
// rho = D (32-bit master) or round-half-even(D / 256) clamped to 127 (24-bit).
// NaN keeps its upper half, quieted, with rho = 0.
template <int MB>
__device__ __forceinline__ void split_elem(float x, uint32_t &hi, uint32_t &rho)
{
    const uint32_t u = __float_as_uint(x);
    const uint32_t b = (u + 0x8000u) >> 16;
    const int32_t D = static_cast<int32_t>(u - (b << 16));
    int32_t r;
    if (MB == 32) {
        r = D;
    } else {
        int32_t q = D >> 8;                 // floor(D / 256)
        const int32_t frac = D & 255;
        q += (frac > 128) | ((frac == 128) & (q & 1));
        r = q < 127 ? q : 127;
    }
    const bool nan = (u & 0x7FFFFFFFu) > 0x7F800000u;
    hi = nan ? ((u >> 16) | 0x40u) : b;
    rho = nan ? 0u : (static_cast<uint32_t>(r) & (MB == 32 ? 0xFFFFu : 0xFFu));
}

// Inverse split: pattern = (theta' << 16) + rho * 2^(16 - w), wrapping.
template <int MB>
__device__ __forceinline__ float reconstruct_elem(uint32_t hi_shifted, int32_t rho)
{
    const uint32_t add = (MB == 24) ? (static_cast<uint32_t>(rho) << 8) : static_cast<uint32_t>(rho);
    return __uint_as_float(hi_shifted + add);
}

// The number of this lane's elements that exist: 16, a partial count at a
// ragged end, or 0 past it.
__device__ __forceinline__ int lane_count(int64_t n, int64_t e0)
{
    const int64_t rem = n - e0;
    return rem >= kLaneElems ? kLaneElems : (rem > 0 ? static_cast<int>(rem) : 0);
}

// 16 consecutive 16-bit elements -> 8 words (zero past cnt)
__device__ __forceinline__ void load_u16x16(const uint16_t *__restrict__ p, int cnt, uint32_t (&w)[8])
{
    if (cnt == kLaneElems) {
        const uint4 a = reinterpret_cast<const uint4 *>(p)[0];
        const uint4 b = reinterpret_cast<const uint4 *>(p)[1];
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = 0u;
#pragma unroll
        for (int j = 0; j < kLaneElems; ++j)
            if (j < cnt) w[j >> 1] |= static_cast<uint32_t>(p[j]) << (16 * (j & 1));
    }
}

__device__ __forceinline__ void store_u16x16(uint16_t *__restrict__ p, int cnt, const uint32_t (&w)[8])
{
    if (cnt == kLaneElems) {
        reinterpret_cast<uint4 *>(p)[0] = make_uint4(w[0], w[1], w[2], w[3]);
        reinterpret_cast<uint4 *>(p)[1] = make_uint4(w[4], w[5], w[6], w[7]);
    } else {
#pragma unroll
        for (int j = 0; j < kLaneElems; ++j)
            if (j < cnt) p[j] = static_cast<uint16_t>(w[j >> 1] >> (16 * (j & 1)));
    }
}

// 16 consecutive bytes -> 4 words (zero past cnt)
__device__ __forceinline__ void load_u8x16(const void *__restrict__ pv, int cnt, uint32_t (&w)[4])
{
    const uint8_t *p = static_cast<const uint8_t *>(pv);
    if (cnt == kLaneElems) {
        const uint4 a = *reinterpret_cast<const uint4 *>(p);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = 0u;
#pragma unroll
        for (int j = 0; j < kLaneElems; ++j)
            if (j < cnt) w[j >> 2] |= static_cast<uint32_t>(p[j]) << (8 * (j & 3));
    }
}

__device__ __forceinline__ void store_u8x16(void *__restrict__ pv, int cnt, const uint32_t (&w)[4])
{
    uint8_t *p = static_cast<uint8_t *>(pv);
    if (cnt == kLaneElems) {
        *reinterpret_cast<uint4 *>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
#pragma unroll
        for (int j = 0; j < kLaneElems; ++j)
            if (j < cnt) p[j] = static_cast<uint8_t>(w[j >> 2] >> (8 * (j & 3)));
    }
}

// 16 consecutive fp32 (zero past cnt)
__device__ __forceinline__ void load_f32x16(const float *__restrict__ p, int cnt, float (&x)[16])
{
    if (cnt == kLaneElems) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float4 v = reinterpret_cast<const float4 *>(p)[k];
            x[4 * k + 0] = v.x; x[4 * k + 1] = v.y; x[4 * k + 2] = v.z; x[4 * k + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < kLaneElems; ++j) x[j] = 0.0f;
#pragma unroll
        for (int j = 0; j < kLaneElems; ++j)
            if (j < cnt) x[j] = p[j];
    }
}

__device__ __forceinline__ void store_f32x16(float *__restrict__ p, int cnt, const float (&x)[16])
{
    if (cnt == kLaneElems) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            reinterpret_cast<float4 *>(p)[k] = make_float4(x[4 * k], x[4 * k + 1], x[4 * k + 2], x[4 * k + 3]);
    } else {
#pragma unroll
        for (int j = 0; j < kLaneElems; ++j)
            if (j < cnt) p[j] = x[j];
    }
}

// ------------------------------------------------------- standalone codec

template <unsigned SPEC>
__global__ void __launch_bounds__(kBlockThreads)
quantize_kernel(const float *__restrict__ x, int64_t n, void *__restrict__ codes,
                uint16_t *__restrict__ scales)
{
    constexpr bool kSigned = (SPEC & FLASHOPT_Q_SIGNED) != 0;
    const int64_t e0 = (static_cast<int64_t>(blockIdx.x) * kBlockThreads + threadIdx.x) * kLaneElems;
    const int cnt = lane_count(n, e0);

    float a[16];
    load_f32x16(x + e0, cnt, a);             // missing elements are the zero pad
    if (SPEC & FLASHOPT_Q_SQRT) {
#pragma unroll
        for (int j = 0; j < 16; ++j) a[j] = sqrtf(a[j]);
    }
    float amax = kSigned ? 0.0f : -__builtin_inff();
#pragma unroll
    for (int j = 0; j < 16; ++j) amax = fmaxf(amax, kSigned ? fabsf(a[j]) : a[j]);
    amax = pair_max(amax);
    const uint32_t s = f16_bits(amax);
    const float d = group_divisor(s);

    uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const float y = a[j] / d;
        out[j >> 2] |= code_byte<SPEC>(y) << (8 * (j & 3));
    }
    store_u8x16(static_cast<uint8_t *>(codes) + e0, cnt, out);
    if ((threadIdx.x & 1) == 0 && cnt > 0) scales[e0 / kGroup] = static_cast<uint16_t>(s);
}

template <unsigned SPEC>
__global__ void __launch_bounds__(kBlockThreads)
dequantize_kernel(const void *__restrict__ codes, const uint16_t *__restrict__ scales, int64_t n,
                  float *__restrict__ out)
{
    __shared__ float unit[256];
    unit[threadIdx.x] = dequant_unit<SPEC>(static_cast<int>(threadIdx.x));
    __syncthreads();

    const int64_t e0 = (static_cast<int64_t>(blockIdx.x) * kBlockThreads + threadIdx.x) * kLaneElems;
    const int cnt = lane_count(n, e0);
    if (cnt == 0) return;
    uint32_t w[4];
    load_u8x16(static_cast<const uint8_t *>(codes) + e0, cnt, w);
    const float s = f16_value(scales[e0 / kGroup]);
    float o[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        float v = unit[ubyte(w, j)] * s;
        if (SPEC & FLASHOPT_Q_SQRT) v = v * v;
        o[j] = v;
    }
    store_f32x16(out + e0, cnt, o);
}

// ------------------------------------------------------- standalone split

template <int MB>
__global__ void __launch_bounds__(kBlockThreads)
split_kernel(const float *__restrict__ master, int64_t n, uint16_t *__restrict__ param,
             void *__restrict__ rho)
{
    const int64_t e0 = (static_cast<int64_t>(blockIdx.x) * kBlockThreads + threadIdx.x) * kLaneElems;
    const int cnt = lane_count(n, e0);
    if (cnt == 0) return;
    float x[16];
    load_f32x16(master + e0, cnt, x);
    uint32_t pw[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    uint32_t rw[MB == 32 ? 8 : 4] = {};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        uint32_t hi, r;
        split_elem<MB>(x[j], hi, r);
        pw[j >> 1] |= hi << (16 * (j & 1));
        if constexpr (MB == 32) rw[j >> 1] |= r << (16 * (j & 1));
        else rw[j >> 2] |= r << (8 * (j & 3));
    }
    store_u16x16(param + e0, cnt, pw);
    if constexpr (MB == 32) store_u16x16(static_cast<uint16_t *>(rho) + e0, cnt, rw);
    else store_u8x16(static_cast<uint8_t *>(rho) + e0, cnt, rw);
}

template <int MB>
__global__ void __launch_bounds__(kBlockThreads)
reconstruct_kernel(const uint16_t *__restrict__ param, const void *__restrict__ rho, int64_t n,
                   float *__restrict__ master)
{
    const int64_t e0 = (static_cast<int64_t>(blockIdx.x) * kBlockThreads + threadIdx.x) * kLaneElems;
    const int cnt = lane_count(n, e0);
    if (cnt == 0) return;
    uint32_t pw[8], rw[MB == 32 ? 8 : 4];
    load_u16x16(param + e0, cnt, pw);
    if constexpr (MB == 32) load_u16x16(static_cast<const uint16_t *>(rho) + e0, cnt, rw);
    else load_u8x16(static_cast<const uint8_t *>(rho) + e0, cnt, rw);
    float x[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const uint32_t hs = (j & 1) ? (pw[j >> 1] & 0xFFFF0000u) : (pw[j >> 1] << 16);
        int32_t r;
        if constexpr (MB == 32) r = shalf(rw, j);
        else r = sbyte(rw, j);
        x[j] = reconstruct_elem<MB>(hs, r);
    }
    store_f32x16(master + e0, cnt, x);
}

// ---------------------------------------------------- fused FlashAdamW step

constexpr int kMaxLdsTensors = 4096;   // chunk table entries kept in LDS

// One persistent grid over all chunks of all tensors.  Wavefront w takes
// chunks w, w + W, w + 2W, ... (W = wavefronts in the grid); the owning
// tensor of a chunk is found by walking the chunk table forward from the
// previous one (chunks only increase).  Per lane and element, in order:
// dequantize m and v, rebuild the master, AdamW, then the group maxima,
// codes, scales and the re-split.
template <int MB, bool COMP>
__global__ void __launch_bounds__(kBlockThreads)
adamw_step_kernel(const DevTensor *__restrict__ tensors, const int32_t *__restrict__ chunk_start,
                  int n_tensors, int32_t total_chunks, StepScalars sc)
{
    constexpr unsigned kMSpec = COMP ? FLASHOPT_SPEC_MOMENTUM : FLASHOPT_SPEC_MOMENTUM_LINEAR;
    constexpr unsigned kVSpec = COMP ? FLASHOPT_SPEC_VARIANCE : FLASHOPT_SPEC_VARIANCE_LINEAR;

    extern __shared__ int32_t s_start[];
    __shared__ float s_mu[256];   // momentum: q/127 (companded: / (2 - |.|))
    __shared__ float s_vu[256];   // variance: q/255
    const bool table_in_lds = n_tensors < kMaxLdsTensors;
    if (table_in_lds)
        for (int i = threadIdx.x; i <= n_tensors; i += kBlockThreads) s_start[i] = chunk_start[i];
    s_mu[threadIdx.x] = dequant_unit<kMSpec>(static_cast<int>(threadIdx.x));
    s_vu[threadIdx.x] = dequant_unit<0u>(static_cast<int>(threadIdx.x));
    __syncthreads();

    const int lane = threadIdx.x & (kWaveLanes - 1);
    const int32_t wave_stride = static_cast<int32_t>(gridDim.x) * (kBlockThreads / kWaveLanes);
    int32_t c = __builtin_amdgcn_readfirstlane(
        static_cast<int32_t>(blockIdx.x) * (kBlockThreads / kWaveLanes) + (threadIdx.x >> 6));
    int t = 0;

    for (; c < total_chunks; c += wave_stride) {
        // owning tensor of chunk c (uniform across the wavefront)
        if (table_in_lds) {
            while (c >= s_start[t + 1]) ++t;
        } else {
            while (c >= chunk_start[t + 1]) ++t;
        }
        t = __builtin_amdgcn_readfirstlane(t);
        const int32_t first = table_in_lds ? s_start[t] : chunk_start[t];
        const DevTensor d = tensors[t];
        const int64_t e0 = static_cast<int64_t>(c - first) * kChunkElems + lane * kLaneElems;
        const int cnt = lane_count(d.numel, e0);

        // ---- loads (missing elements read as zero)
        uint32_t pw[8], gw[8], rw[MB == 32 ? 8 : 4], mw[4], vw[4];
        load_u16x16(d.param + e0, cnt, pw);
        load_u16x16(d.grad + e0, cnt, gw);
        if constexpr (MB == 32) load_u16x16(static_cast<const uint16_t *>(d.rho) + e0, cnt, rw);
        else load_u8x16(static_cast<const uint8_t *>(d.rho) + e0, cnt, rw);
        load_u8x16(d.m_codes + e0, cnt, mw);
        load_u8x16(d.v_codes + e0, cnt, vw);
        uint32_t smb = 0u, svb = 0u;
        if (cnt > 0) {
            smb = d.m_scales[e0 / kGroup];
            svb = d.v_scales[e0 / kGroup];
        }
        const float ms = f16_value(smb);
        const float vs = f16_value(svb);

        // ---- dequantize, reconstruct, AdamW
        float m1[16], q1[16], th1[16];      // q1: what the variance quantizer sees
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t hs = (j & 1) ? (pw[j >> 1] & 0xFFFF0000u) : (pw[j >> 1] << 16);
            int32_t r;
            if constexpr (MB == 32) r = shalf(rw, j);
            else r = sbyte(rw, j);
            const float theta = reconstruct_elem<MB>(hs, r);
            const float g = (j & 1) ? bf16_hi(gw[j >> 1]) : bf16_lo(gw[j >> 1]);

            const float m0 = s_mu[ubyte(mw, j)] * ms;
            const float a0 = s_vu[ubyte(vw, j)] * vs;
            const float v0 = COMP ? a0 * a0 : a0;

            const float thd = theta * sc.cwd;
            const float m_decay = sc.b1 * m0;
            const float m_new = sc.c1 * g;
            const float m = m_decay + m_new;
            const float v_decay = sc.b2 * v0;
            const float cg = sc.c2 * g;
            const float v_new = cg * g;
            const float v = v_decay + v_new;
            const float rt = sqrtf(v);
            const float den = rt * sc.k2 + sc.eps;
            const float num = sc.alpha * m;
            const float upd = num / den;
            th1[j] = thd - upd;
            m1[j] = m;
            q1[j] = COMP ? rt : v;
        }
        if (cnt < kLaneElems) {             // zero pad of the ragged last group
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (j >= cnt) { m1[j] = 0.0f; q1[j] = 0.0f; }
        }

        // ---- requantize m and v: group max over the lane pair
        float am = 0.0f, av = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            am = fmaxf(am, fabsf(m1[j]));
            av = fmaxf(av, q1[j]);
        }
        am = pair_max(am);
        av = pair_max(av);
        const uint32_t sm_out = f16_bits(am);
        const uint32_t sv_out = f16_bits(av);
        const float dm = group_divisor(sm_out);
        const float dv = group_divisor(sv_out);

        uint32_t mo[4] = {0u, 0u, 0u, 0u}, vo[4] = {0u, 0u, 0u, 0u};
        uint32_t po[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
        uint32_t ro[MB == 32 ? 8 : 4] = {};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            mo[j >> 2] |= code_byte<kMSpec>(m1[j] / dm) << (8 * (j & 3));
            vo[j >> 2] |= code_byte<kVSpec>(q1[j] / dv) << (8 * (j & 3));
            uint32_t hi, r;
            split_elem<MB>(th1[j], hi, r);
            po[j >> 1] |= hi << (16 * (j & 1));
            if constexpr (MB == 32) ro[j >> 1] |= r << (16 * (j & 1));
            else ro[j >> 2] |= r << (8 * (j & 3));
        }

        // ---- stores
        store_u16x16(d.param + e0, cnt, po);
        if constexpr (MB == 32) store_u16x16(static_cast<uint16_t *>(d.rho) + e0, cnt, ro);
        else store_u8x16(static_cast<uint8_t *>(d.rho) + e0, cnt, ro);
        store_u8x16(d.m_codes + e0, cnt, mo);
        store_u8x16(d.v_codes + e0, cnt, vo);
        if ((lane & 1) == 0 && cnt > 0) {
            d.m_scales[e0 / kGroup] = static_cast<uint16_t>(sm_out);
            d.v_scales[e0 / kGroup] = static_cast<uint16_t>(sv_out);
        }
    }
}

// ------------------------------------------------------------- launching

unsigned grid_for(int64_t n)
{
    const int64_t per_block = static_cast<int64_t>(kBlockThreads) * kLaneElems;
    return static_cast<unsigned>((n + per_block - 1) / per_block);
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
        hipLaunchKernelGGL(split_kernel<32>, dim3(grid_for(n)), dim3(kBlockThreads), 0, st,
                           master, n, param, rho);
    else
        hipLaunchKernelGGL(split_kernel<24>, dim3(grid_for(n)), dim3(kBlockThreads), 0, st,
                           master, n, param, rho);
    return hipGetLastError();
}

hipError_t launch_reconstruct(const uint16_t *param, const void *rho, int64_t n, int master_bits,
                              float *master, hipStream_t st)
{
    if (master_bits == 32)
        hipLaunchKernelGGL(reconstruct_kernel<32>, dim3(grid_for(n)), dim3(kBlockThreads), 0, st,
                           param, rho, n, master);
    else
        hipLaunchKernelGGL(reconstruct_kernel<24>, dim3(grid_for(n)), dim3(kBlockThreads), 0, st,
                           param, rho, n, master);
    return hipGetLastError();
}

namespace {

template <int MB, bool COMP>
hipError_t step_variant(const DevTensor *tensors, const int32_t *chunk_start, int n_tensors,
                        int32_t total_chunks, const StepScalars &sc, int blocks_per_cu, int cus,
                        hipStream_t st)
{
    const size_t lds = n_tensors < kMaxLdsTensors ? sizeof(int32_t) * (n_tensors + 1) : 0;
    const int64_t waves_per_block = kBlockThreads / kWaveLanes;
    const int64_t need = (total_chunks + waves_per_block - 1) / waves_per_block;
    int64_t grid = static_cast<int64_t>(blocks_per_cu) * cus;
    if (grid > need) grid = need;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL((adamw_step_kernel<MB, COMP>), dim3(static_cast<unsigned>(grid)),
                       dim3(kBlockThreads), lds, st, tensors, chunk_start, n_tensors,
                       total_chunks, sc);
    return hipGetLastError();
}

template <int MB, bool COMP>
int occupancy_blocks(int n_tensors)
{
    const size_t lds = n_tensors < kMaxLdsTensors ? sizeof(int32_t) * (n_tensors + 1) : 0;
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, adamw_step_kernel<MB, COMP>,
                                                     kBlockThreads, lds) != hipSuccess || nb < 1)
        nb = 1;
    return nb;
}

}  // namespace

hipError_t launch_adamw_step(const DevTensor *tensors, const int32_t *chunk_start, int n_tensors,
                             int32_t total_chunks, const StepScalars &sc, int master_bits,
                             bool companded, hipStream_t st)
{
    if (total_chunks <= 0) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;

    // Workgroups resident per CU: the occupancy limit, unless the tuning
    // variable FLASHOPT_BLOCKS_PER_CU asks for fewer (or more) of them.
    int bpc = 0;
    if (const char *env = getenv("FLASHOPT_BLOCKS_PER_CU")) bpc = atoi(env);
    const bool m32 = master_bits == 32;
    if (bpc <= 0) {
        if (m32) bpc = companded ? occupancy_blocks<32, true>(n_tensors) : occupancy_blocks<32, false>(n_tensors);
        else bpc = companded ? occupancy_blocks<24, true>(n_tensors) : occupancy_blocks<24, false>(n_tensors);
    }
    if (m32)
        return companded ? step_variant<32, true>(tensors, chunk_start, n_tensors, total_chunks, sc, bpc, cus, st)
                         : step_variant<32, false>(tensors, chunk_start, n_tensors, total_chunks, sc, bpc, cus, st);
    return companded ? step_variant<24, true>(tensors, chunk_start, n_tensors, total_chunks, sc, bpc, cus, st)
                     : step_variant<24, false>(tensors, chunk_start, n_tensors, total_chunks, sc, bpc, cus, st);
}

}  // namespace flashopt
