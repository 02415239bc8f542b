// afq_device.hpp -- device primitives for the gfx950 kernels: number
// formats, wavefront reductions and the three FP8 quantisers.
//
// Layout convention used by every kernel: a row is cut into 8-element
// chunks (16 bytes of bf16/fp16); lane t of a row owns chunks t, t+NT,
// t+2NT, ...  Consecutive lanes therefore own consecutive chunks, so every
// global access of a wavefront is one contiguous 1 KiB (16-B loads) or
// 512 B (8-B code stores) span, and a 32-element MXFP8 block is exactly
// 4 consecutive lanes, a 128-element group exactly 16 (one DPP row).
//
// Conversions use the gfx950 packed instructions v_cvt_pk_bf16_f32 and
// v_cvt_pk_fp8_f32 (OCP e4m3fn).  Both round to nearest even, as the GPU
// tests check against the oracle's roundings: v_cvt_pk_fp8_f32 on every
// fp32 from 2^-10 (below it everything rounds to zero) to 464 of either
// sign, which covers all it is given (clamped values, or quotients of at
// most 448(1+2^-23)); v_cvt_pk_bf16_f32 on every rounding class of every
// bf16 neighbourhood.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace afq {

// dtype / mode tags (match afq.h)
constexpr int kBF16 = 0, kFP16 = 1, kFP32 = 2;
constexpr int kMX = 0, kB128 = 1, kPT = 2;
constexpr int kNone = 3; // copy only: the launch writes no codes or scales

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------ activations
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// two fp32 -> packed bf16 pair (low = a), round to nearest even
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}
// two fp32 -> packed fp16 pair (low = a), round to nearest even
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
}
__device__ __forceinline__ float f16_lo(uint32_t w)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// scalar fp32 -> bf16 bits, RNE (used off the hot path)
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.0f) & 0xFFFFu; }

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
            v[2 * i] = f16_lo(w[i]);
            v[2 * i + 1] = f16_hi(w[i]);
        }
    }
}

// Round 8 fp32 values to dtype DT; returns the packed 16-byte chunk.
template <int DT>
__device__ __forceinline__ uint4 pack8(const float (&v)[8])
{
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        w[i] = DT == kBF16 ? pack_bf16x2(v[2 * i], v[2 * i + 1]) : pack_f16x2(v[2 * i], v[2 * i + 1]);
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// One fp32 value rounded to dtype DT (to nearest even), as fp32.
template <int DT>
__device__ __forceinline__ float round_dt(float v)
{
    if constexpr (DT == kBF16) return bf16_lo(pack_bf16x2(v, 0.0f));
    else return f16_lo(pack_f16x2(v, 0.0f));
}

// Round 8 fp32 values to dtype DT in place (v becomes the rounded values);
// returns the packed chunk.
template <int DT>
__device__ __forceinline__ uint4 round8(float (&v)[8])
{
    const uint4 p = pack8<DT>(v);
    unpack8<DT>(p, v);
    return p;
}

// ---------------------------------------------------------------- e4m3fn
__device__ __forceinline__ float clamp448(float v)
{
    return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f);
}

// 8 already-clamped fp32 values -> 8 e4m3fn codes packed little-endian into
// two 32-bit words (v_cvt_pk_fp8_f32 writes two codes into one half).
__device__ __forceinline__ uint2 cvt8_e4m3(const float (&v)[8])
{
    // the first conversion of each word keeps the upper half of its `old`
    // operand, which the second overwrites: any register serves, and v[0] /
    // v[4] (read by the same instruction) save a move of a zero
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], __float_as_int(v[0]), false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], __float_as_int(v[4]), false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], w1, true);
    return make_uint2((uint32_t)w0, (uint32_t)w1);
}

// --------------------------------------------------------------- reductions
// DPP controls (GFX9 encoding).
constexpr int kQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dppf(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

template <int CTRL>
__device__ __forceinline__ uint32_t dppu(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

// Maxima of non-negative floats are taken on their bit patterns (which
// order like the values), as unsigned integer maxima: no NaN quieting is
// needed, so each step is a single DPP-modified v_max_u32.
// max over the 4 lanes of a quad (an MXFP8 block)
__device__ __forceinline__ float max_quad(float f)
{
    uint32_t v = __float_as_uint(f);
    v = max(v, dppu<kQuadSwap1>(v));
    v = max(v, dppu<kQuadSwap2>(v));
    return __uint_as_float(v);
}
// max over the 8 lanes of a half DPP row (an MXFP8 block at 4 values per
// lane): after the quad step every lane holds its quad's max, and the
// half-row mirror pairs each lane with one of the other quad
__device__ __forceinline__ float max_oct(float f)
{
    uint32_t v = __float_as_uint(max_quad(f));
    v = max(v, dppu<kRowHalfMirror>(v));
    return __uint_as_float(v);
}
// max over the 16 lanes of a DPP row (a 1x128 group)
__device__ __forceinline__ float max_row16(float f)
{
    uint32_t v = __float_as_uint(max_quad(f));
    v = max(v, dppu<kRowHalfMirror>(v));
    v = max(v, dppu<kRowMirror>(v));
    return __uint_as_float(v);
}
// sum over the 16 lanes of a DPP row; every lane ends with the same value
// (each step adds two partials that are equal across the pair, and fp32
// addition is commutative).
__device__ __forceinline__ float sum_row16(float v)
{
    v += dppf<kQuadSwap1>(v);
    v += dppf<kQuadSwap2>(v);
    v += dppf<kRowHalfMirror>(v);
    v += dppf<kRowMirror>(v);
    return v;
}
// Exchange with the lane 16 (32) positions away: v_permlane16_swap /
// v_permlane32_swap (gfx950) applied to two copies of v return, between
// them, v of this lane and v of its partner; their sum (max) is symmetric,
// so which copy is which does not matter.
__device__ __forceinline__ float sum_xor16(float v)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float sum_xor32(float v)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float max_xor16(float v)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(max((uint32_t)p[0], (uint32_t)p[1]));
}
__device__ __forceinline__ float max_xor32(float v)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(max((uint32_t)p[0], (uint32_t)p[1]));
}

// all-reduce over the 64 lanes of a wavefront (no LDS traffic)
__device__ __forceinline__ float sum_wave(float v) { return sum_xor32(sum_xor16(sum_row16(v))); }

// fp64 all-reduce over a wavefront: the same lane pairings as sum_wave,
// with each exchange applied to both 32-bit halves of the double (a lane
// permutation moves the two halves together).  Every lane ends with the
// same value: each step adds two partials that are equal across the pair.
__device__ __forceinline__ double join64(uint32_t lo, uint32_t hi)
{
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
template <int CTRL>
__device__ __forceinline__ double dppd(double v)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    return join64(dppu<CTRL>((uint32_t)b), dppu<CTRL>((uint32_t)(b >> 32)));
}
__device__ __forceinline__ double sum_wave_f64(double v)
{
    v += dppd<kQuadSwap1>(v);
    v += dppd<kQuadSwap2>(v);
    v += dppd<kRowHalfMirror>(v);
    v += dppd<kRowMirror>(v);
    uint64_t b = __builtin_bit_cast(uint64_t, v);
    auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)b, (uint32_t)b, false, false);
    auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(b >> 32), (uint32_t)(b >> 32), false, false);
    v = join64(lo[0], hi[0]) + join64(lo[1], hi[1]);
    b = __builtin_bit_cast(uint64_t, v);
    lo = __builtin_amdgcn_permlane32_swap((uint32_t)b, (uint32_t)b, false, false);
    hi = __builtin_amdgcn_permlane32_swap((uint32_t)(b >> 32), (uint32_t)(b >> 32), false, false);
    return join64(lo[0], hi[0]) + join64(lo[1], hi[1]);
}
__device__ __forceinline__ float max_wave(float v) { return max_xor32(max_xor16(max_row16(v))); }

// Cross-wavefront step of a row reduction.  Each of the row's n <= 16
// wavefronts has left its partial in LDS: p0[0..n) (and p1[0..n) for a
// second segment).  Lane i < n of the first DPP row reads p0[i], lane
// 16 + i reads p1[i], every other lane takes the identity; one 16-lane
// reduction per DPP row then leaves each row's total in all of its lanes,
// and lanes 0 and 16 hand the totals out as wavefront-uniform values.  All
// partials are read in one LDS access.
__device__ __forceinline__ float lane_pick(float v, int lane)
{
    return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), lane));
}
template <int NSEG>
__device__ __forceinline__ float lds_rows_sum(const float *p0, const float *p1, int n, float &t1)
{
    const int l = threadIdx.x & 63, i = l & 15;
    float v = 0.f;
    if (l < 16 * NSEG && i < n) v = (l & 16) ? p1[i] : p0[i];
    v = sum_row16(v);
    t1 = NSEG > 1 ? lane_pick(v, 16) : 0.f;
    return lane_pick(v, 0);
}
// the same for the largest of non-negative partials
template <int NSEG>
__device__ __forceinline__ float lds_rows_max(const float *p0, const float *p1, int n, float &t1)
{
    const int l = threadIdx.x & 63, i = l & 15;
    float v = 0.f;
    if (l < 16 * NSEG && i < n) v = (l & 16) ? p1[i] : p0[i];
    v = max_row16(v);
    t1 = NSEG > 1 ? lane_pick(v, 16) : 0.f;
    return lane_pick(v, 0);
}
// the same for fp64 partials (the 16-lane steps of sum_wave_f64)
template <int NSEG>
__device__ __forceinline__ double lds_rows_sum_f64(const double *p0, const double *p1, int n, double &t1)
{
    const int l = threadIdx.x & 63, i = l & 15;
    double v = 0.0;
    if (l < 16 * NSEG && i < n) v = (l & 16) ? p1[i] : p0[i];
    v += dppd<kQuadSwap1>(v);
    v += dppd<kQuadSwap2>(v);
    v += dppd<kRowHalfMirror>(v);
    v += dppd<kRowMirror>(v);
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)b, hi = (uint32_t)(b >> 32);
    t1 = NSEG > 1 ? join64(__builtin_amdgcn_readlane(lo, 16), __builtin_amdgcn_readlane(hi, 16)) : 0.0;
    return join64(__builtin_amdgcn_readlane(lo, 0), __builtin_amdgcn_readlane(hi, 0));
}

// Sum of a row's block totals, p0[0..nb) and p1[0..nb) for a second
// segment (one total per 64-chunk block of the row, nb <= 64), in a tree
// fixed by nb, a function of the row width alone: up to 16 blocks the
// 16-lane tree of lds_rows_sum (both segments in one pass), more blocks the
// 64-lane wavefront tree per segment.  Lanes past nb add zeros, which add
// exactly (the totals are sums of squares, never -0).
template <int NSEG>
__device__ __forceinline__ float lds_blocks_sum(const float *p0, const float *p1, int nb, float &t1)
{
    if (nb <= 16) return lds_rows_sum<NSEG>(p0, p1, nb, t1);
    const int l = threadIdx.x & 63;
    const float t0 = lane_pick(sum_wave(l < nb ? p0[l] : 0.f), 0);
    t1 = NSEG > 1 ? lane_pick(sum_wave(l < nb ? p1[l] : 0.f), 0) : 0.f;
    return t0;
}
__device__ __forceinline__ double lane_pick_f64(double v, int lane)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    return join64(__builtin_amdgcn_readlane((uint32_t)b, lane), __builtin_amdgcn_readlane((uint32_t)(b >> 32), lane));
}
template <int NSEG>
__device__ __forceinline__ double lds_blocks_sum_f64(const double *p0, const double *p1, int nb, double &t1)
{
    if (nb <= 16) return lds_rows_sum_f64<NSEG>(p0, p1, nb, t1);
    const int l = threadIdx.x & 63;
    const double t0 = lane_pick_f64(sum_wave_f64(l < nb ? p0[l] : 0.0), 0);
    t1 = NSEG > 1 ? lane_pick_f64(sum_wave_f64(l < nb ? p1[l] : 0.0), 0) : 0.0;
    return t0;
}

// Block barrier that orders only LDS: the waves exchange reduction
// partials through LDS, and their outstanding global stores need not
// complete before the barrier (a __syncthreads() would wait for them).
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// 1/sqrt(x) for x > 0: the hardware estimate and one Newton step.
__device__ __forceinline__ float rsqrt_nr(float x)
{
    const float y = __builtin_amdgcn_rsqf(x);
    return y * __builtin_fmaf(-0.5f * x, y * y, 1.5f);
}

// The inverse RMS of the fp32-direct norm: fl32(1 / sqrt(ss / cols + eps))
// with the division, the sum, the square root and the reciprocal each the
// IEEE fp64 operation (the formula evaluated as written in fp64), given
// rcols = RN64(1 / cols).  Those IEEE operations cost some thirty fp64
// instructions on the row's critical path; the fast path below needs about
// a third of that and gives the same fp32:
//   x = fl64(ss * rcols + eps) is within 2^-51 (relative) of the formula's
//   fp64 argument, and the formula's fp64 result within 2^-52 of the exact
//   1/sqrt of that argument.  z is the hardware estimate of 1/sqrt(x) after
//   two Newton steps; it is accepted only if the residual 1 - x z^2 (one
//   FMA, error about 2^-52) is below 2^-46 in magnitude, which bounds z to
//   within about 2^-47 of 1/sqrt(x) whatever the estimate's accuracy.  The
//   formula's result then lies in [z (1 - 2^-44), z (1 + 2^-44)], and if
//   both ends round to the same fp32, so does it (rounding is monotone).
// Otherwise -- a value within about 2^-44 of an fp32 rounding midpoint, one
// row in 10^6 or so, or anything non-finite -- the formula itself runs.
// `fast`, when given, reports which path gave the result.
__device__ __forceinline__ float inv_rms_f32q(double ss, int32_t cols, double rcols, float eps,
                                              bool *fast = nullptr)
{
    const double x = __builtin_fma(ss, rcols, (double)eps);
    const double hx = 0.5 * x;
    double z = __builtin_amdgcn_rsq(x);
#pragma unroll
    for (int i = 0; i < 2; ++i) z = __builtin_fma(z, __builtin_fma(-(hx * z), z, 0.5), z);
    const double e = __builtin_fma(-(x * z), z, 1.0);
    const float lo = (float)(z * (1.0 - 0x1p-44));
    const float hi = (float)(z * (1.0 + 0x1p-44));
    const bool ok = __builtin_fabs(e) < 0x1p-46 && lo == hi;
    if (fast) *fast = ok;
    if (__builtin_expect(ok, 1)) return lo;
    return (float)(1.0 / sqrt(ss / (double)cols + (double)eps));
}

// largest |u| of 8 values (v_max3_f32 with |.| source modifiers)
__device__ __forceinline__ float amax8(const float (&u)[8])
{
    float m = __builtin_fmaxf(__builtin_fabsf(u[0]), __builtin_fabsf(u[1]));
#pragma unroll
    for (int i = 2; i < 8; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(u[i]));
    return m;
}

// ------------------------------------------------------------- quantisers
// MXFP8 block scale: E8M0 byte b = max(E - 8, 0) from the fp32 exponent
// field E of the block amax; the codes use u * 2^(127 - b), a power of two
// whose fp32 exponent field is 254 - b (b <= 246, so always normal).
__device__ __forceinline__ uint32_t e8m0_of(float amax)
{
    const int E = (int)(__float_as_uint(amax) >> 23);
    return (uint32_t)max(E - 8, 0);
}
__device__ __forceinline__ float mx_inv_scale(uint32_t b)
{
    return __uint_as_float((254u - b) << 23);
}

// 8 MXFP8 codes of a chunk given the block's inverse scale (exact power
// of two: u * inv_x is exact), clamped to +-448.
__device__ __forceinline__ uint2 mx_codes8(const float (&u)[8], float inv_x)
{
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = clamp448(u[i] * inv_x);
    return cvt8_e4m3(v);
}

// fp32 scale s = amax / 448 and the reciprocal used by the quotient below.
struct Fp32Scale {
    float s;    // stored scale
    float r;    // RN(1/s), set when fast
    bool fast;  // fast scale and fast quotient valid (amax >= 2^-83)
    bool zero;  // s == 0: an all-zero group, or one whose amax / 448
                // underflows fp32; its codes are all 0x00
};
// Fast path, amax >= 2^-83: s = RN(amax/448) as a product with RN(1/448)
// plus one Markstein correction, and RN(1/s) as the hardware reciprocal plus
// one Newton correction.  Both equal the IEEE divisions on every fp32
// mantissa at every exponent from 2^-116 up (checked on the GPU over all
// 2^23 mantissas of every exponent field).  The bound 2^-83 is the
// quotient's: its remainder (below) is exact when it is no finer than the
// smallest subnormal, which for every quotient of 2^-11 or more (all that
// decide an e4m3 code) needs s >= 2^-92, i.e. amax >= 448 * 2^-92 ~ 2^-83.2;
// below that the remainder can round and the corrected quotient miss the
// correctly rounded one.  Smaller amax take the IEEE divisions.
__device__ __forceinline__ Fp32Scale fp32_scale(float amax)
{
    Fp32Scale sc;
    if (__builtin_expect(amax >= 0x1p-83f, 1)) {
        constexpr float kInv448 = 1.0f / 448.0f;
        const float s0 = amax * kInv448;
        sc.s = __builtin_fmaf(__builtin_fmaf(-s0, 448.0f, amax), kInv448, s0);
        const float r0 = __builtin_amdgcn_rcpf(sc.s);
        sc.r = __builtin_fmaf(__builtin_fmaf(-sc.s, r0, 1.0f), r0, r0);
        sc.fast = true;
        sc.zero = false;
    } else {
        sc.s = amax / 448.0f;      // IEEE division
        sc.r = 0.0f;
        sc.fast = false;
        sc.zero = (sc.s == 0.0f);
    }
    return sc;
}

// fp32(u / s), correctly rounded, for a scale with sc.fast set.  With
// r = RN(1/s), q0 = RN(u r) is within one ulp of u/s, so the remainder
// q0 s - u is exact under FMA (no finer than the smallest subnormal for
// every quotient that can decide a code: amax >= 2^-83), and one correction
// step q0 - (q0 s - u) r rounds to the correctly rounded quotient
// (Markstein's theorem; no overflow since |u/s| <= 448(1+2^-23)).  Taking the
// remainder as q0 s - u keeps the sign of a zero u (-0 gives -0): for u = -0
// the correction is -(+0) r + (-0) = -0.
__device__ __forceinline__ float quotient_fast(float u, const Fp32Scale &sc)
{
    const float q0 = u * sc.r;
    const float nrem = __builtin_fmaf(q0, sc.s, -u);
    return __builtin_fmaf(-nrem, sc.r, q0);
}

// 8 codes of a chunk under an fp32 scale.  With a fast scale the quotients
// are at most 448(1+2^-23) in magnitude, which v_cvt_pk_fp8_f32 rounds to
// 448 exactly as it rounds the clamped value (checked on the GPU over every
// fp32 in [448, 464] of either sign), so no clamp is applied.  Other scales
// take the IEEE division and the clamp; a zero scale gives zero codes (a
// select after the conversion, of whatever the division gave).  The choice
// is made once per chunk (it is uniform over a group).
__device__ __forceinline__ uint2 fp32scale_codes8(const float (&u)[8], const Fp32Scale &sc)
{
    float v[8];
    if (__builtin_expect(sc.fast, 1)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = quotient_fast(u[i], sc);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = clamp448(__builtin_copysignf(u[i] / sc.s, u[i]));
    }
    const uint2 q = cvt8_e4m3(v);
    return make_uint2(sc.zero ? 0u : q.x, sc.zero ? 0u : q.y);
}

// ---------------------------------------------------------------- memory
// Activations are read once and outputs written once: both go through the
// non-temporal forms (measured faster on every workload here, e.g. the
// hidden-6144 MXFP8 norm at M = 16384 from 5.5 to 5.8 TB/s).  The norm
// weight, re-read by every row, uses the ordinary cached load.
// Wait until every vector memory operation the wavefront has issued is
// complete: s_waitcnt vmcnt(0), with the expcnt (7) and lgkmcnt (15) fields
// at their maxima so that they do not wait (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <typename V>
__device__ __forceinline__ V ldg(const void *p)
{
    return *reinterpret_cast<const V *>(p);
}
__device__ __forceinline__ uint4 ldg_stream(const void *p)
{
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p)));
}
__device__ __forceinline__ void stg_stream(void *p, const uint4 &v)
{
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4 *>(p));
}
__device__ __forceinline__ void stg_stream(void *p, const uint2 &v)
{
    __builtin_nontemporal_store(__builtin_bit_cast(u32x2, v), reinterpret_cast<u32x2 *>(p));
}
__device__ __forceinline__ void stg_stream(void *p, uint32_t v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<uint32_t *>(p));
}
// The norm kernel's group scales (MXFP8 bytes, 1x128 fp32) take the
// non-temporal form as well: the 1x128 norm at hidden 4096, 4096 rows
// 21.6 -> 21.1 us, the MXFP8 norm at hidden 6144, 1024 to 4096 rows 2-3 %
// faster.  Per-row scales (per-token) and the SiLU kernels' scales keep
// plain stores: there the non-temporal form was slower (a per-token row
// ends with its one scale store, and the non-temporal store of a few bytes
// took about 0.9 us longer to complete: the two-segment per-token norm at 8
// rows 2.9 -> 3.8 us; SiLU-and-mul 1x128 at 4096 rows of 12288 40.4 ->
// 40.9 us).
__device__ __forceinline__ void stg_scale(float *p, float v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void stg_scale(uint8_t *p, uint32_t b) { __builtin_nontemporal_store((uint8_t)b, p); }
__device__ __forceinline__ uint2 ldg_stream8(const void *p)
{
    return __builtin_bit_cast(uint2, __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p)));
}

} // namespace afq
