// afq_device.hpp -- device primitives for the gfx950 kernels: number
// formats, wavefront reductions and the three FP8 quantisers.
//
// Layout convention used by every kernel: a row is cut into 8-element
// chunks (16 bytes of bf16/fp16); lane t of a row owns chunks t, t+NT,
// t+2NT, ...  Consecutive lanes therefore own consecutive chunks, so every
// global access of a wavefront is one contiguous 1 KiB (16-B loads) or
// 512 B (8-B code stores) span, and a 32-element MXFP8 block is exactly
// 4 consecutive lanes, a 128-element group exactly 16 (one DPP row).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace afq {

// ------------------------------------------------------------ activations
// dtype tags (match afq.h)
constexpr int kBF16 = 0, kFP16 = 1, kFP32 = 2;
constexpr int kMX = 0, kB128 = 1, kPT = 2;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).  Integer form:
// add half an ulp of the kept part, plus the kept LSB to break ties evenly.
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ uint32_t f32_to_f16(float f)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f); // v_cvt_f16_f32, RNE
}

// Unpack 8 activations of dtype DT from a 16-byte chunk into fp32.
template <int DT>
__device__ __forceinline__ void unpack8(const uint4 &c, float (&v)[8])
{
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (DT == kBF16) {
            v[2 * i] = bf16_lo(w[i]);
            v[2 * i + 1] = bf16_hi(w[i]);
        } else {
            v[2 * i] = f16_bits_to_f32(w[i] & 0xFFFFu);
            v[2 * i + 1] = f16_bits_to_f32(w[i] >> 16);
        }
    }
}

// Round 8 fp32 values to dtype DT; returns the packed 16-byte chunk and the
// rounded values (as fp32) in `r`.
template <int DT>
__device__ __forceinline__ uint4 round_pack8(const float (&v)[8], float (&r)[8])
{
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t a, b;
        if constexpr (DT == kBF16) {
            a = f32_to_bf16(v[2 * i]);
            b = f32_to_bf16(v[2 * i + 1]);
            r[2 * i] = __uint_as_float(a << 16);
            r[2 * i + 1] = __uint_as_float(b << 16);
        } else {
            a = f32_to_f16(v[2 * i]);
            b = f32_to_f16(v[2 * i + 1]);
            r[2 * i] = f16_bits_to_f32(a);
            r[2 * i + 1] = f16_bits_to_f32(b);
        }
        w[i] = a | (b << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// ---------------------------------------------------------------- e4m3fn
// OCP e4m3fn code of v, round to nearest even; |v| <= 448 (the caller
// clamps).  Normal range (|v| >= 2^-6): drop 20 mantissa bits with RNE and
// rebias the exponent from 127 to 7 (the carry of a round-up moves into the
// exponent field by itself).  Below 2^-6 the code is the count of 2^-9
// steps, rounded to nearest even (|v| * 2^9 is exact).
__device__ __forceinline__ uint32_t e4m3_code(float v)
{
    const uint32_t bits = __float_as_uint(v);
    const uint32_t sign = (bits >> 24) & 0x80u;
    const uint32_t a = bits & 0x7FFFFFFFu;
    const uint32_t rn = a + 0x7FFFFu + ((a >> 20) & 1u);
    const uint32_t normal = (rn >> 20) - (120u << 3);
    const uint32_t sub = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    return sign | (a >= 0x3C800000u ? normal : sub);
}

__device__ __forceinline__ float clamp448(float v)
{
    return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f);
}

// 8 codes of one chunk packed little-endian into two 32-bit words.
__device__ __forceinline__ uint2 pack_codes(const uint32_t (&c)[8])
{
    return make_uint2(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                      c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24));
}

// --------------------------------------------------------------- reductions
// DPP controls (GFX9 encoding).
constexpr int kQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

// max over the 4 lanes of a quad (an MXFP8 block), unsigned integers
__device__ __forceinline__ uint32_t max_quad(uint32_t v)
{
    v = max(v, dpp<kQuadSwap1>(v));
    v = max(v, dpp<kQuadSwap2>(v));
    return v;
}
// max over the 16 lanes of a DPP row (a 1x128 group)
__device__ __forceinline__ uint32_t max_row16(uint32_t v)
{
    v = max_quad(v);
    v = max(v, dpp<kRowHalfMirror>(v));
    v = max(v, dpp<kRowMirror>(v));
    return v;
}
// sum over the 16 lanes of a DPP row; every lane ends with the same value
// (each step adds two equal-across-the-pair partials, and fp32 addition is
// commutative).
__device__ __forceinline__ float sum_row16(float v)
{
    v += __uint_as_float(dpp<kQuadSwap1>(__float_as_uint(v)));
    v += __uint_as_float(dpp<kQuadSwap2>(__float_as_uint(v)));
    v += __uint_as_float(dpp<kRowHalfMirror>(__float_as_uint(v)));
    v += __uint_as_float(dpp<kRowMirror>(__float_as_uint(v)));
    return v;
}

// Lane-group reduction over the NT lanes of a row when NT <= 64 (a row
// inside one wavefront: lane groups of 16, 32 or 64).  The cross-row steps
// read the four row results with ds_swizzle-free readlane-style shuffles.
template <int W>
__device__ __forceinline__ float sum_lanes(float v)
{
    static_assert(W == 16 || W == 32 || W == 64, "lane group");
    v = sum_row16(v);
    if constexpr (W >= 32) v += __shfl_xor(v, 16, 64);
    if constexpr (W >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}
template <int W>
__device__ __forceinline__ uint32_t max_lanes(uint32_t v)
{
    static_assert(W == 16 || W == 32 || W == 64, "lane group");
    v = max_row16(v);
    if constexpr (W >= 32) v = max(v, (uint32_t)__shfl_xor((int)v, 16, 64));
    if constexpr (W >= 64) v = max(v, (uint32_t)__shfl_xor((int)v, 32, 64));
    return v;
}

// ------------------------------------------------------------- quantisers
// MXFP8 block scale: E8M0 byte b = max(E - 8, 0) from the fp32 exponent
// field E of the block amax; the codes use u * 2^(127 - b), a power of two
// whose fp32 exponent field is 254 - b (b <= 246, so always normal).
__device__ __forceinline__ uint32_t e8m0_from_amax_bits(uint32_t amax_bits)
{
    const int E = (int)(amax_bits >> 23);
    return (uint32_t)max(E - 8, 0);
}
__device__ __forceinline__ float mx_inv_scale(uint32_t b)
{
    return __uint_as_float((254u - b) << 23);
}

// 8 MXFP8 codes of a chunk given the block's inverse scale.
__device__ __forceinline__ uint2 mx_codes8(const float (&u)[8], float inv_x)
{
    uint32_t c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = e4m3_code(clamp448(u[i] * inv_x));
    return pack_codes(c);
}

// Largest |u| of 8 values as fp32 bit patterns (non-negative floats order
// like their bit patterns, so an integer max is a float max).
__device__ __forceinline__ uint32_t amax_bits8(const float (&u)[8])
{
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, __float_as_uint(u[i]) & 0x7FFFFFFFu);
    return m;
}

// fp32 scale s = amax / 448 and the reciprocal used by the quotient below.
struct Fp32Scale {
    float s;    // stored scale
    float r;    // RN(1/s) when the fast quotient is valid
    bool fast;  // s normal and 1/s finite
    bool zero;  // all-zero group
};
__device__ __forceinline__ Fp32Scale fp32_scale(uint32_t amax_bits)
{
    Fp32Scale sc;
    const float A = __uint_as_float(amax_bits);
    sc.s = A / 448.0f;             // IEEE division
    sc.zero = (amax_bits == 0u);
    sc.r = 1.0f / sc.s;            // IEEE division, correctly rounded
    sc.fast = (sc.s >= 0x1p-126f) && (sc.r < 0x1p127f);
    return sc;
}

// fp32(u / s), correctly rounded.  With r = RN(1/s), q0 = RN(u r) is within
// one ulp of u/s, the remainder u - q0 s is exact under FMA, and one
// correction step q0 + rem * r rounds to the correctly rounded quotient
// (Markstein's theorem; no overflow since |u/s| <= 448(1+2^-23)).  Scales
// that are subnormal or whose reciprocal overflows take the IEEE division.
__device__ __forceinline__ float quotient(float u, const Fp32Scale &sc)
{
    float q;
    if (sc.fast) {
        const float q0 = u * sc.r;
        const float rem = __builtin_fmaf(-q0, sc.s, u);
        q = __builtin_fmaf(rem, sc.r, q0);
    } else {
        q = u / sc.s;
    }
    return __builtin_copysignf(q, u);
}

__device__ __forceinline__ uint2 fp32scale_codes8(const float (&u)[8], const Fp32Scale &sc)
{
    uint32_t c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = sc.zero ? 0u : e4m3_code(clamp448(quotient(u[i], sc)));
    return pack_codes(c);
}

// ---------------------------------------------------------------- memory
template <typename V>
__device__ __forceinline__ V ldg(const void *p)
{
    return *reinterpret_cast<const V *>(p);
}
template <typename V>
__device__ __forceinline__ void stg(void *p, const V &v)
{
    *reinterpret_cast<V *>(p) = v;
}

} // namespace afq
