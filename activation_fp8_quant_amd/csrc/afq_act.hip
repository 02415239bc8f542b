// afq_act.hip -- SiLU-and-mul and the clamped SwiGLU, fused with FP8
// quantisation.
//
// act_quant_kernel (SiLU-and-mul with MXFP8 or 1x128; the clamped SwiGLU
// with MXFP8) works on a flat chunk index (8 activations per chunk): a row
// has no cross-row work, so every lane is busy for any width I.
// HBM-bound elementwise work: no dense contraction, so no MFMA.

#include "afq_device.hpp"
#include "afq_internal.h"
#include "afq_launch.hpp"

#include <cmath>

namespace afq {

// activation kinds
constexpr int kSilu = 0, kSwigluOai = 1;

struct ActArgs {
    const uint8_t *gu;
    int64_t gu_pitch;
    uint8_t *values;
    uint8_t *scales;
    uint8_t *act;
    uint32_t total;   // chunks of this launch (rows * C), < 2^32
    int32_t C;        // chunks per row (I / 8)
    int32_t I;
    DivC dc;          // division by C
    // clamped SwiGLU only: alpha log2(e) = cHi + cLo with a 16-bit head
    float alpha, beta, limit;
    float cHi;        // alpha log2(e) to 16 significant bits
    float cLoLn2;     // (alpha log2(e) - cHi) ln 2
};

// silu(g) = g / (1 + e^-g) in fp32 for a bf16 gate g >= -80, within 2 ulp
// of the fp64 value (measured over every such gate).  log2(e) is split as
// kHi + kLo with a 16-bit head, so t = -g kHi is exact for a bf16 g and
// e^-g = 2^t e^y with y = -g kLo ln 2 (|y| < 4e-4 for |g| <= 80); the
// hardware exp2 gives 2^t and e^y is taken to first order, so that
// 1 + e^-g = 2^t (1 + y) + 1 is two FMAs.  For large positive g, 2^t is
// zero and the denominator is 1.  Then g times the hardware reciprocal.
__device__ __forceinline__ float silu_fast(float g)
{
    constexpr float kHi = 1.44268798828125f;    // log2(e) to 16 significant bits
    constexpr float kLoLn2 = 4.8884954e-06f;    // (log2(e) - kHi) ln 2
    const float t = g * -kHi;
    const float w = __builtin_fmaf(g, -kLoLn2, 1.0f);
    const float d = __builtin_fmaf(__builtin_amdgcn_exp2f(t), w, 1.0f);
    return g * __builtin_amdgcn_rcpf(d);
}

// silu in fp64 as a two-term value hi + lo: for |g| < 1/2 as g/2 + (g/2)
// tanh(g/2) (for tiny g the plain quotient collapses to exactly g/2, a
// possible rounding midpoint, and the second term keeps the g^2/4 that
// decides it); else g e^g / (1 + e^g) (g < 0, no overflow) or
// g / (1 + e^-g).  A zero gate returns itself (silu(-0) = -0).
__device__ __forceinline__ void silu_f64(float g, double &hi, double &lo)
{
    const double gd = (double)g;
    lo = 0.0;
    if (gd == 0.0) {
        hi = gd;
    } else if (__builtin_fabs(gd) < 0.5) {
        const double a = gd * 0.5, b = a * tanh(a);
        hi = a + b;
        lo = b - (hi - a);
    } else if (gd < 0.0) {
        const double e = exp(gd);
        hi = gd * e / (1.0 + e);
    } else {
        hi = gd / (1.0 + exp(-gd));
    }
}

__device__ __noinline__ float silu_f32_slow(float g)
{
    double hi, lo;
    silu_f64(g, hi, lo);
    return (float)(hi + lo);
}


// bf16(silu(g)) of the 8 bf16 gates of a chunk (bits in gb), exactly
// rounded, as fp32 values.  The fast fp32 value is within 2 ulp of silu(g)
// for every bf16 gate >= -80 (measured over all of them), so its bf16
// rounding is the exact one unless it sits within 3 fp32 ulps of a bf16
// rounding midpoint; such gates, and gates below -80 (e^-g beyond the fp32
// range), read the exact value from kSiluBf16Table (generated from the
// definition in decimal arithmetic by gen_silu_table.py).  The common path
// has no branch; a chunk holding a flagged gate takes one.  Gate 5.9375
// (bf16 0x40BE), whose fast value falls on a midpoint exactly, is by far the
// most frequent flagged gate in N(0, sigma^2) activations with sigma near 3
// (0.06 % of the gates, so about a quarter of the wavefronts): its exact
// value is an immediate, and the table is read only for the other flagged
// gates.
#include "silu_bf16_table.inc"

__device__ __forceinline__ void silu_bf16x8(const float (&g)[8], const uint4 &gb, float (&s)[8])
{
    float raw[8];
    uint32_t dmin = 0xFFFFFFFFu; // (low 16 bits) - (0x8000 - 3): <= 6 when within 3 ulps of a midpoint
    uint32_t gmax = 0u;          // largest gate bit pattern: above that of -80 for a gate below -80
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        raw[i] = s[i] = silu_fast(g[i]);
        dmin = min(dmin, (__float_as_uint(raw[i]) & 0xFFFFu) - (0x8000u - 3u));
        gmax = max(gmax, __float_as_uint(g[i]));
    }
    round8<kBF16>(s);
    if (__builtin_expect(dmin <= 6u || gmax > 0xC2A00000u, 0)) {
        const uint32_t w[4] = {gb.x, gb.y, gb.z, gb.w};
        bool need = false;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t bits = (w[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
            const bool fl = g[i] < -80.0f || ((__float_as_uint(raw[i]) & 0xFFFFu) - (0x8000u - 3u)) <= 6u;
            if (fl && bits == 0x40BEu) s[i] = __uint_as_float((uint32_t)kSiluBf16Table[0x40BE] << 16);
            need |= fl && bits != 0x40BEu;
        }
        if (need) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t bits = (w[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
                if (bits != 0x40BEu && (g[i] < -80.0f || ((__float_as_uint(raw[i]) & 0xFFFFu) - (0x8000u - 3u)) <= 6u))
                    s[i] = __uint_as_float((uint32_t)kSiluBf16Table[bits] << 16);
            }
        }
    }
}

// fp32 silu of N gates for the MXFP8 path: the fast form; gates below -80
// (e^-g beyond the fp32 range) are redone in fp64.
template <int N>
__device__ __forceinline__ void silu_f32xn(const float (&g)[N], float (&s)[N])
{
    uint32_t gmax = 0u; // largest gate bit pattern: above that of -80 for a gate below -80
#pragma unroll
    for (int i = 0; i < N; ++i) {
        s[i] = silu_fast(g[i]);
        gmax = max(gmax, __float_as_uint(g[i]));
    }
    if (gmax > 0xC2A00000u) {
#pragma unroll 1
        for (int i = 0; i < N; ++i)
            if (g[i] < -80.0f) s[i] = silu_f32_slow(g[i]);
    }
}

// Clamped SwiGLU, gate factor: glu = gc logistic(alpha gc) with gc =
// min(g, limit), in fp32.  As in silu_fast, e^(-alpha gc) = 2^t e^y with
// t = -cHi gc exact (a bf16 gc times a 16-bit head; for a limit that is not
// a bf16 value a clamped gate makes t inexact by at most half an ulp) and
// y = -cLo ln2 gc.  |cLo| <= 2^-16 |alpha log2(e)|, so |y| <= |t| 2^-16 ln2,
// below 1.6e-3 wherever 2^t is not negligible (t > -150); e^y is taken to
// second order (the cubic term is below 1e-9).  y is clamped to [-1, 1]
// first, which changes nothing where it matters and keeps y^2 finite for
// huge gates under an infinite limit (there 2^t is 0).  For alpha gc below
// about -80 (t above 115, 2^t near the top of the fp32 range) the factor is
// redone in fp64.
__device__ __noinline__ float swiglu_glu_slow(float gc, float alpha)
{
    const double z = (double)alpha * (double)gc;
    const double e = exp(z);
    return (float)((double)gc * e / (1.0 + e));
}

template <int N>
__device__ __forceinline__ void swiglu_act_xn(const ActArgs &a, const float (&g)[N], float (&v)[N])
{
    float glu[N];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float gc = __builtin_fminf(g[i], a.limit);
        const float t = gc * -a.cHi;
        const float y = __builtin_amdgcn_fmed3f(gc * -a.cLoLn2, -1.0f, 1.0f);
        const float w = __builtin_fmaf(y, __builtin_fmaf(y, 0.5f, 1.0f), 1.0f);
        const float d = __builtin_fmaf(__builtin_amdgcn_exp2f(t), w, 1.0f);
        glu[i] = gc * __builtin_amdgcn_rcpf(d);
        tmax = __builtin_fmaxf(tmax, t);
    }
    if (tmax > 115.0f) {
#pragma unroll 1
        for (int i = 0; i < N; ++i) {
            const float gc = __builtin_fminf(g[i], a.limit);
            if (gc * -a.cHi > 115.0f) glu[i] = swiglu_glu_slow(gc, a.alpha);
        }
    }
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] = glu[i] * (__builtin_amdgcn_fmed3f(v[i], -a.limit, a.limit) + a.beta);
}

// The fp32 activation of the MXFP8 path from the gates g and the up values
// v (overwritten): SiLU-and-mul fl32(fl32(silu(g)) * up), or the clamped
// SwiGLU fl32(glu * fl32(clamp(up, +-limit) + beta)).
template <int ACT, int N>
__device__ __forceinline__ void act_f32xn(const ActArgs &a, const float (&g)[N], float (&v)[N])
{
    if constexpr (ACT == kSwigluOai) {
        swiglu_act_xn<N>(a, g, v);
    } else {
        float sg[N];
        silu_f32xn<N>(g, sg);
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] *= sg[i];
    }
}

// 4 bf16 values of a packed 8-byte half chunk -> fp32, and back (RNE)
__device__ __forceinline__ void unpack4(const uint2 &c, float (&v)[4])
{
    v[0] = bf16_lo(c.x);
    v[1] = bf16_hi(c.x);
    v[2] = bf16_lo(c.y);
    v[3] = bf16_hi(c.y);
}
__device__ __forceinline__ uint2 pack4(const float (&v)[4])
{
    return make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}

// The 1x128 outputs of chunk f (the launch's flat chunk index) from
// s = bf16(silu(gate)) and the up values v (fp32, overwritten):
// a = bf16(s * up), the group scale amax|a| / 448 over the 16 lanes of the
// group, the codes, and the optional bf16 copy of a.  The outputs are dense
// [rows, I] (codes, copy) and [rows, I / 128] (scales), and a row has a
// multiple of 16 chunks, so chunk f's codes start at element 8 f and its
// group's scale is entry f / 16: no row index is needed.
__device__ __forceinline__ void b128_tail(const ActArgs &a, const float (&s)[8], float (&v)[8], uint32_t f)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] *= s[i];
    const uint4 ap = round8<kBF16>(v);
    const int64_t out_off = (int64_t)f * 8;
    if (a.act) stg_stream(a.act + out_off * 2, ap);
    const Fp32Scale sc = fp32_scale(max_row16(amax8(v)));
    const uint2 q = fp32scale_codes8(v, sc);
    if ((f & 15u) == 0) reinterpret_cast<float *>(a.scales)[f >> 4] = sc.s;
    stg_stream(a.values + out_off, q);
}

// ACT: kSilu, or kSwigluOai (MXFP8 only: the clamped SwiGLU).
// QBF16 (MXFP8 only): the bf16-first variant, which quantises the fp32
// activation rounded to bf16 (the value the unfused chain stores and then
// quantises) instead of the fp32 activation itself.  QUANT false: the
// SiLU-and-mul of the unfused chain, which writes only the bf16 activation
// (rounded as MODE's activation is) and no codes or scales.
template <int MODE, int CPL, bool QBF16, bool QUANT, int ACT>
__global__ void __launch_bounds__(256)
act_quant_kernel(const ActArgs a)
{
    const uint32_t base = blockIdx.x * (256u * CPL) + threadIdx.x;
    uint4 gv[CPL], uv[CPL];
    bool ok[CPL];
    // outputs are dense rows of C chunks: chunk f's outputs sit at f alone
    // (element 8 f, MX scale f / 4); only the input, whose rows have a
    // pitch, needs f's row and column
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const uint32_t f = base + k * 256u;
        ok[k] = f < a.total;
        if (ok[k]) {
            const uint32_t r = div_c(f, a.dc);
            const int32_t lc = (int32_t)(f - r * (uint32_t)a.C);
            const uint8_t *p = a.gu + (int64_t)r * a.gu_pitch + (int64_t)lc * 16;
            gv[k] = ldg_stream(p);
            uv[k] = ldg_stream(p + (int64_t)a.I * 2);
        }
    }
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        if (!ok[k]) continue; // uniform over every quant group
        const uint32_t f = base + k * 256u;
        const int64_t out_off = (int64_t)f * 8;
        float g[8], v[8];
        unpack8<kBF16>(gv[k], g);
        unpack8<kBF16>(uv[k], v);
        if constexpr (!QUANT) {
            // the unfused SiLU-and-mul: the activation alone
            if constexpr (MODE == kMX) {
                act_f32xn<ACT, 8>(a, g, v);
            } else {
                float sg[8];
                silu_bf16x8(g, gv[k], sg);
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] *= sg[i];
            }
            stg_stream(a.act + out_off * 2, pack8<kBF16>(v));
        } else if constexpr (MODE == kMX) {
            uint2 q;
            act_f32xn<ACT, 8>(a, g, v);
            const uint4 ap = QBF16 ? round8<kBF16>(v) : pack8<kBF16>(v);
            if (a.act) stg_stream(a.act + out_off * 2, ap);
            const uint32_t b = e8m0_of(max_quad(amax8(v)));
            q = mx_codes8(v, mx_inv_scale(b));
            if ((f & 3u) == 0) a.scales[f >> 2] = (uint8_t)b;
            stg_stream(a.values + out_off, q);
        } else {
            float sg[8];
            silu_bf16x8(g, gv[k], sg);
            b128_tail(a, sg, v, f);
        }
    }
}

// Decode-size form of the MXFP8 activation kernel (SiLU-and-mul or the
// clamped SwiGLU; same arithmetic, same codes and scales) for quantising
// launches without the bf16 copy: 4 activations per lane (8-byte loads of
// gate and up), so a 32-element block spans 8 lanes (one half DPP row) and
// a launch has twice the lanes.  At decode row counts the launch fills few
// SIMDs, each wavefront runs alone, and the launch lasts about as long as
// one wavefront's instruction chain; halving the work per lane shortens it.
// a.C and a.dc describe 4-element chunks here.
template <int ACT, bool QBF16>
__global__ void __launch_bounds__(256)
act_mx4_kernel(const ActArgs a)
{
    const uint32_t f = blockIdx.x * 256u + threadIdx.x;
    // a row has I / 4 chunks, a multiple of 8, and blocks start at multiples
    // of 256: every 8-lane block is either wholly inside the launch or
    // wholly outside it
    if (f >= a.total) return;
    const uint32_t r = div_c(f, a.dc);
    const int32_t lc = (int32_t)(f - r * (uint32_t)a.C);
    const uint8_t *p = a.gu + (int64_t)r * a.gu_pitch + (int64_t)lc * 8;
    const uint2 gv = ldg_stream8(p);
    const uint2 uv = ldg_stream8(p + (int64_t)a.I * 2);
    float g[4], v[4];
    unpack4(gv, g);
    unpack4(uv, v);
    act_f32xn<ACT, 4>(a, g, v);
    if constexpr (QBF16) {
        const uint2 ap = pack4(v);
        unpack4(ap, v); // quantise the bf16 activation
    }
    const uint32_t b = e8m0_of(max_oct(__builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(v[0]), __builtin_fabsf(v[1])),
                                                       __builtin_fmaxf(__builtin_fabsf(v[2]), __builtin_fabsf(v[3])))));
    const float ix = mx_inv_scale(b);
    const float q0 = clamp448(v[0] * ix);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(q0, clamp448(v[1] * ix), __float_as_int(q0), false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(v[2] * ix), clamp448(v[3] * ix), w, true);
    // dense outputs: chunk f's codes at element 4 f, its block's scale at f / 8
    if ((f & 7u) == 0) a.scales[f >> 3] = (uint8_t)b;
    stg_stream(a.values + (int64_t)f * 4, (uint32_t)w);
}

// ================================================================ launcher
template <int MODE, int CPL, bool QBF16, bool QUANT = true, int ACT = kSilu>
static hipError_t go_act(const ActArgs &a, hipStream_t st)
{
    const uint32_t blocks = (a.total + 256u * CPL - 1) / (256u * CPL);
    hipLaunchKernelGGL((act_quant_kernel<MODE, CPL, QBF16, QUANT, ACT>), dim3(blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

// the 4-per-lane MXFP8 form (quantising launches without the bf16 copy):
// a (total, C, dc) describe 8-element chunks on entry and are switched to
// 4-element chunks here
template <int ACT>
static hipError_t go_act_mx4(ActArgs a, bool qbf16, hipStream_t st)
{
    a.total *= 2;
    a.C *= 2;
    a.dc = divc((uint32_t)a.C);
    const uint32_t blocks = (a.total + 255u) / 256u;
    if (qbf16)
        hipLaunchKernelGGL((act_mx4_kernel<ACT, true>), dim3(blocks), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((act_mx4_kernel<ACT, false>), dim3(blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

// alpha log2(e) split into a 16-significant-bit head and the rest (times
// ln 2), so that the head times a bf16 gate is exact in fp32
static void swiglu_split(float alpha, float &hi, float &lo_ln2)
{
    const double c = (double)alpha * 1.4426950408889634;
    int e = 0;
    const double m = std::frexp(c, &e);
    const double h = std::ldexp(std::nearbyint(std::ldexp(m, 16)), e - 16);
    hi = (float)h;
    lo_ln2 = (float)((c - h) * 0.6931471805599453);
}

// Quantising MXFP8 launches with no bf16 copy and at most this many
// 8-element chunks take the 4-per-lane form (act_mx4_kernel).  Measured at
// I = 768, hot, graph-replayed: the launch alone is faster from 64 to 1024
// rows (clamped SwiGLU 1.95 -> 1.86 us at 64 rows, 1.98 -> 1.88 at 192,
// 2.24 -> 2.12 at 1024; SiLU-and-mul 1.90 -> 1.82 at 192), the same within
// noise at 8 rows, and slower from 2048 rows (196,608 chunks) on.  A kernel
// that reads the codes right after it runs as fast as after the 8-per-lane
// form; one that reads a bf16 activation written by the 4-per-lane form
// (8-byte stores) ran 0.3-0.4 us slower, so copy-only launches and launches
// that write the copy keep the 8-per-lane form.
#ifndef AFQ_MX4_MAX_CHUNKS
#define AFQ_MX4_MAX_CHUNKS 131072
#endif
constexpr int64_t kMx4MaxChunks = AFQ_MX4_MAX_CHUNKS;

int launch_act(const ActPlan &p, void *stream)
{
    hipStream_t st = (hipStream_t)stream;
    const int32_t C = p.I / 8;
    const int64_t step = flat_rows_per_launch(C);
    for (int64_t r0 = 0; r0 < p.M; r0 += step) {
        const int64_t rows = p.M - r0 < step ? p.M - r0 : step;
        ActArgs a;
        a.gu = p.gu + r0 * p.gu_pitch;
        a.gu_pitch = p.gu_pitch;
        a.values = offset_or_null(p.values, r0 * p.I);
        a.scales = offset_or_null(p.scales, r0 * scale_row_bytes(p.mode, p.I));
        a.act = offset_or_null(p.act, r0 * p.I * 2);
        a.C = C;
        a.I = p.I;
        a.total = (uint32_t)(rows * C);
        a.dc = divc((uint32_t)C);
        a.alpha = p.alpha;
        a.beta = p.beta;
        a.limit = p.limit;
        swiglu_split(p.alpha, a.cHi, a.cLoLn2);
        hipError_t e;
        if (p.mode == kMX && p.quant && !p.act && (int64_t)a.total <= kMx4MaxChunks)
            e = p.act_kind == kSwigluOai ? go_act_mx4<kSwigluOai>(a, p.qin == 2, st)
                                         : go_act_mx4<kSilu>(a, p.qin == 2, st);
        else if (p.act_kind == kSwigluOai) // MXFP8 only
            e = !p.quant       ? go_act<kMX, 1, false, false, kSwigluOai>(a, st)
                : p.qin == 2   ? go_act<kMX, 1, true, true, kSwigluOai>(a, st)
                               : go_act<kMX, 1, false, true, kSwigluOai>(a, st);
        else
            e = !p.quant      ? (p.mode == kMX ? go_act<kMX, 1, false, false>(a, st)
                                               : go_act<kB128, 1, false, false>(a, st))
                : p.mode != kMX ? go_act<kB128, 1, false>(a, st)
                : p.qin == 2    ? go_act<kMX, 1, true>(a, st)
                                : go_act<kMX, 1, false>(a, st);
        if (e != hipSuccess) return (int)e;
    }
    return 0;
}

} // namespace afq
