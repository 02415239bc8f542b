// afq_kernels.hip -- gfx950 kernels for fused activation FP8 quantisation.
//
// Three kernel families, all HBM-bound elementwise/row work (no MFMA: no
// dense contraction exists on this path):
//
//   norm_quant_kernel  one row (one or two segments) per NT lanes; residual
//                      add, fp32 sum of squares (DPP inside a wavefront, one
//                      LDS step across wavefronts), scale by the weight,
//                      round to the activation dtype, quantise.
//   act_quant_kernel   SiLU-and-mul + quantisation on a flat chunk index:
//                      no cross-row work, so every lane is busy for any I.
//   quant_flat_kernel  standalone 1x32 / 1x128 quantisation (flat), and
//   quant_row_kernel   standalone per-token quantisation (row reduction).
//
// Every lane issues all of its 16-byte loads before it does any arithmetic,
// so a row's whole input is in flight at once; stores are 16 B (dtype
// outputs) and 8 B (codes) per lane, contiguous across the wavefront.

#include "afq_device.hpp"
#include "afq_internal.h"

namespace afq {

// ===================================================================== norm
// Rows are NT lanes (a whole number of wavefronts, NT <= 1024); a block
// holds R rows (R > 1 only for NT of 64 or 128 lanes).  Both are launch
// parameters; the per-lane chunk count CPL and the segment count NSEG are
// template parameters (the loops over a lane's chunks are unrolled, and a
// single-segment row carries no segment selection).
constexpr int kMaxBlock = 1024;

struct NormArgs {
    NormSegPlan seg[2];
    const uint8_t *res_in;
    uint8_t *res_out;
    int64_t M;
    float eps;
    int32_t C0;        // chunks of segment 0
    int32_t C;         // chunks of both segments
    int32_t NT;        // lanes per row
    int32_t R;         // rows per block
    int32_t WPR;       // wavefronts per row
    int32_t wpr_shift; // log2(WPR) when R > 1
    float inv_cols0;   // 1 / cols of each segment (the mean of the squares)
    float inv_cols1;
};

// sum of squares of the 8 values of a packed chunk (v_dot2 on pairs)
template <int DT>
__device__ __forceinline__ float sumsq8(const uint4 &c, float acc)
{
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (DT == kBF16)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[i]),
                                                  __builtin_bit_cast(bf16x2, w[i]), acc, false);
        else
            acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w[i]),
                                         __builtin_bit_cast(f16x2, w[i]), acc, false);
    }
    return acc;
}

template <int DT, int MODE, bool GEMMA, int CPL, int NSEG>
__global__ void __launch_bounds__(kMaxBlock)
norm_quant_kernel(const NormArgs a)
{
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int rib = a.R == 1 ? 0 : (wave >> a.wpr_shift); // row within the block
    const int t = tid - rib * a.NT;                       // lane within the row
    const int64_t row = (int64_t)blockIdx.x * a.R + rib;
    const bool row_ok = row < a.M;
    const bool has_res = a.res_in != nullptr;

    // per-row bases
    const uint8_t *xrow0 = a.seg[0].x + row * a.seg[0].x_pitch;
    const uint8_t *xrow1 = NSEG > 1 ? a.seg[1].x + row * a.seg[1].x_pitch : xrow0;
    const int64_t rrow = row * a.C0 * 16;

    // ---- issue every load of the row
    uint4 xv[CPL], rv[CPL], wv[CPL];
    bool ok[CPL];
    int sg[CPL], lc[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const int c = t + k * a.NT;
        ok[k] = row_ok && c < a.C;
        if constexpr (NSEG == 1) {
            sg[k] = 0;
            lc[k] = c;
        } else {
            sg[k] = c >= a.C0 ? 1 : 0;
            lc[k] = c - (sg[k] ? a.C0 : 0);
        }
        if (ok[k]) {
            xv[k] = ldg_stream((sg[k] ? xrow1 : xrow0) + lc[k] * 16);
            wv[k] = ldg<uint4>((sg[k] ? a.seg[1].w : a.seg[0].w) + lc[k] * 16);
            if (has_res)
                rv[k] = ldg_stream(a.res_in + rrow + lc[k] * 16);
        }
    }

    // ---- residual add (h = round_dt(x + r), stored), sum of squares
    float h[CPL][8];
    float ss0 = 0.f, ss1 = 0.f;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        if (!ok[k]) continue;
        uint4 hp = xv[k];
        if (has_res) {
            float rf[8];
            unpack8<DT>(xv[k], h[k]);
            unpack8<DT>(rv[k], rf);
#pragma unroll
            for (int i = 0; i < 8; ++i) h[k][i] += rf[i];
            hp = pack8<DT>(h[k]);
            stg_stream(a.res_out + rrow + lc[k] * 16, hp);
        }
        unpack8<DT>(hp, h[k]);
        if (NSEG > 1 && sg[k]) ss1 = sumsq8<DT>(hp, ss1);
        else ss0 = sumsq8<DT>(hp, ss0);
    }

    // ---- row reduction: DPP/permlane inside the wavefront, one LDS step
    //      across the wavefronts of the row
    __shared__ float red[kMaxBlock / 64][2];
    __shared__ float redm[kMaxBlock / 64][2];
    ss0 = sum_wave(ss0);
    if constexpr (NSEG > 1) ss1 = sum_wave(ss1);
    if (a.WPR > 1) {
        if ((tid & 63) == 0) {
            red[wave][0] = ss0;
            if constexpr (NSEG > 1) red[wave][1] = ss1;
        }
        lds_barrier();
        ss0 = 0.f;
        ss1 = 0.f;
        for (int i = 0; i < a.WPR; ++i) {
            ss0 += red[rib * a.WPR + i][0];
            if constexpr (NSEG > 1) ss1 += red[rib * a.WPR + i][1];
        }
    }
    const float inv0 = rsqrt_nr(__builtin_fmaf(ss0, a.inv_cols0, a.eps));
    const float inv1 = NSEG > 1 ? rsqrt_nr(__builtin_fmaf(ss1, a.inv_cols1, a.eps)) : inv0;

    // ---- u = round_dt(h * inv * g), kept in place of h; optional copy.
    //      Gemma: g * inv = (1 + w) inv as one FMA.
    float am0 = 0.f, am1 = 0.f;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        if (!ok[k]) continue;
        const float inv = sg[k] ? inv1 : inv0;
        float wf[8];
        unpack8<DT>(wv[k], wf);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            h[k][i] *= GEMMA ? __builtin_fmaf(wf[i], inv, inv) : wf[i] * inv;
        const uint4 up = round8<DT>(h[k]);
        uint8_t *normed = sg[k] ? a.seg[1].normed : a.seg[0].normed;
        const int32_t cols = sg[k] ? a.seg[1].cols : a.seg[0].cols;
        if (normed)
            stg_stream(normed + (row * cols + (int64_t)lc[k] * 8) * 2, up);
        if constexpr (MODE == kPT) {
            const float m = amax8(h[k]);
            if (NSEG > 1 && sg[k]) am1 = __builtin_fmaxf(am1, m); else am0 = __builtin_fmaxf(am0, m);
        }
    }

    // ---- quantise
    if constexpr (MODE == kPT) {
        am0 = max_wave(am0);
        if constexpr (NSEG > 1) am1 = max_wave(am1);
        if (a.WPR > 1) {
            if ((tid & 63) == 0) {
                redm[wave][0] = am0;
                if constexpr (NSEG > 1) redm[wave][1] = am1;
            }
            lds_barrier();
            am0 = 0.f;
            am1 = 0.f;
            for (int i = 0; i < a.WPR; ++i) {
                am0 = __builtin_fmaxf(am0, redm[rib * a.WPR + i][0]);
                if constexpr (NSEG > 1) am1 = __builtin_fmaxf(am1, redm[rib * a.WPR + i][1]);
            }
        }
        const Fp32Scale sc0 = fp32_scale(am0);
        const Fp32Scale sc1 = NSEG > 1 ? fp32_scale(am1) : sc0;
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            if (!ok[k]) continue;
            const NormSegPlan &s = sg[k] ? a.seg[1] : a.seg[0];
            const uint2 q = fp32scale_codes8(h[k], sg[k] ? sc1 : sc0);
            stg_stream(s.values + row * s.cols + (int64_t)lc[k] * 8, q);
            if (lc[k] == 0) reinterpret_cast<float *>(s.scales)[row] = sg[k] ? sc1.s : sc0.s;
        }
    } else {
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            if (!ok[k]) continue; // uniform over every quant group
            const NormSegPlan &s = sg[k] ? a.seg[1] : a.seg[0];
            uint2 q;
            if constexpr (MODE == kMX) {
                const uint32_t b = e8m0_of(max_quad(amax8(h[k])));
                q = mx_codes8(h[k], mx_inv_scale(b));
                if ((lc[k] & 3) == 0) s.scales[row * (s.cols / 32) + lc[k] / 4] = (uint8_t)b;
            } else {
                const Fp32Scale sc = fp32_scale(max_row16(amax8(h[k])));
                q = fp32scale_codes8(h[k], sc);
                if ((lc[k] & 15) == 0)
                    reinterpret_cast<float *>(s.scales)[row * (s.cols / 128) + lc[k] / 16] = sc.s;
            }
            stg_stream(s.values + row * s.cols + (int64_t)lc[k] * 8, q);
        }
    }
}

// ============================================================ SiLU-and-mul
// Division of a flat 32-bit chunk index by the chunks per row C, by a
// multiplier computed on the host (round-up method): with l = ceil(log2 C)
// and m = floor(2^32 (2^l - C) / C) + 1, n / C = (mulhi(n, m) + n) >> l
// for every n < 2^32 (the sum is taken in 64 bits).
struct DivC {
    uint32_t m;
    uint32_t l;
};
static DivC divc(uint32_t C)
{
    uint32_t l = 0;
    while ((1ull << l) < C) ++l;
    DivC d;
    d.m = (uint32_t)(((1ull << 32) * ((1ull << l) - C)) / C + 1);
    d.l = l;
    return d;
}
__device__ __forceinline__ uint32_t div_c(uint32_t n, DivC d)
{
    return (uint32_t)(((uint64_t)__umulhi(n, d.m) + n) >> d.l);
}

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
};

// silu(g) = g / (1 + e^-g) in fp32 for a bf16 gate g >= -80, within 2 ulp
// of the fp64 value (measured over every such gate).  log2(e) is split as
// kHi + kLo with a 16-bit head, so t = -g kHi is exact for a bf16 g and
// e^-g = 2^t e^y with y = -g kLo ln 2 (|y| < 4e-4 for |g| <= 80); the
// hardware exp2 gives 2^t and e^y is taken to first order.  For large
// positive g, 2^t vanishes and y is clamped so that the product stays
// finite.  Then g times the hardware reciprocal of 1 + e^-g.
__device__ __forceinline__ float silu_fast(float g)
{
    constexpr float kHi = 1.44268798828125f;    // log2(e) to 16 significant bits
    constexpr float kLoLn2 = 4.8884954e-06f;    // (log2(e) - kHi) ln 2
    const float t = g * -kHi;
    const float y = __builtin_fmaxf(g * -kLoLn2, -0.01f);
    const float e0 = __builtin_amdgcn_exp2f(t);
    const float e = __builtin_fmaf(e0, y, e0);
    return g * __builtin_amdgcn_rcpf(1.0f + e);
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
// has no branch; a chunk holding a flagged gate takes one.
#include "silu_bf16_table.inc"

__device__ __forceinline__ void silu_bf16x8(const float (&g)[8], const uint4 &gb, float (&s)[8])
{
    float raw[8];
    uint32_t dmin = 0xFFFFFFFFu; // (low 16 bits) - (0x8000 - 3): <= 6 when within 3 ulps of a midpoint
    float gmin = g[0];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        raw[i] = s[i] = silu_fast(g[i]);
        dmin = min(dmin, (__float_as_uint(raw[i]) & 0xFFFFu) - (0x8000u - 3u));
        gmin = __builtin_fminf(gmin, g[i]);
    }
    round8<kBF16>(s);
    if (__builtin_expect(dmin <= 6u || gmin < -80.0f, 0)) {
        const uint32_t w[4] = {gb.x, gb.y, gb.z, gb.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (g[i] < -80.0f || ((__float_as_uint(raw[i]) & 0xFFFFu) - (0x8000u - 3u)) <= 6u) {
                const uint32_t bits = (w[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
                s[i] = __uint_as_float((uint32_t)kSiluBf16Table[bits] << 16);
            }
        }
    }
}

// fp32 silu of 8 gates for the MXFP8 path: the fast form; gates below -80
// (e^-g beyond the fp32 range) are redone in fp64.
__device__ __forceinline__ void silu_f32x8(const float (&g)[8], float (&s)[8])
{
    float gmin = g[0];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        s[i] = silu_fast(g[i]);
        gmin = __builtin_fminf(gmin, g[i]);
    }
    if (gmin < -80.0f) {
#pragma unroll 1
        for (int i = 0; i < 8; ++i)
            if (g[i] < -80.0f) s[i] = silu_f32_slow(g[i]);
    }
}

template <int MODE, int CPL>
__global__ void __launch_bounds__(256)
act_quant_kernel(const ActArgs a)
{
    const uint32_t base = blockIdx.x * (256u * CPL) + threadIdx.x;
    uint4 gv[CPL], uv[CPL];
    bool ok[CPL];
    int64_t rw[CPL];
    int32_t lc[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const uint32_t f = base + k * 256u;
        ok[k] = f < a.total;
        const uint32_t r = div_c(f, a.dc);
        rw[k] = r;
        lc[k] = (int32_t)(f - r * (uint32_t)a.C);
        if (ok[k]) {
            const uint8_t *p = a.gu + rw[k] * a.gu_pitch + (int64_t)lc[k] * 16;
            gv[k] = ldg_stream(p);
            uv[k] = ldg_stream(p + (int64_t)a.I * 2);
        }
    }
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        if (!ok[k]) continue; // uniform over every quant group
        float g[8], v[8];
        unpack8<kBF16>(gv[k], g);
        unpack8<kBF16>(uv[k], v);
        const int64_t out_off = rw[k] * a.I + (int64_t)lc[k] * 8;
        uint2 q;
        if constexpr (MODE == kMX) {
            float sg[8];
            silu_f32x8(g, sg);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] *= sg[i];
            if (a.act) stg_stream(a.act + out_off * 2, pack8<kBF16>(v));
            const uint32_t b = e8m0_of(max_quad(amax8(v)));
            q = mx_codes8(v, mx_inv_scale(b));
            if ((lc[k] & 3) == 0) a.scales[rw[k] * (a.I / 32) + lc[k] / 4] = (uint8_t)b;
        } else {
            float sg[8];
            silu_bf16x8(g, gv[k], sg);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] *= sg[i];
            const uint4 ap = round8<kBF16>(v);
            if (a.act) stg_stream(a.act + out_off * 2, ap);
            const Fp32Scale sc = fp32_scale(max_row16(amax8(v)));
            q = fp32scale_codes8(v, sc);
            if ((lc[k] & 15) == 0)
                reinterpret_cast<float *>(a.scales)[rw[k] * (a.I / 128) + lc[k] / 16] = sc.s;
        }
        stg_stream(a.values + out_off, q);
    }
}

// ======================================================= standalone quant
struct QuantArgs {
    const uint8_t *x;
    int64_t x_pitch;
    uint8_t *values;
    uint8_t *scales;
    uint32_t total;  // chunks of this launch (flat kernel), < 2^32
    int64_t M;
    int32_t C;       // chunks per row
    int32_t cols;
    DivC dc;         // division by C
    int32_t NT;      // lanes per row (row kernel)
    int32_t R;       // rows per block (row kernel)
    int32_t WPR;     // wavefronts per row (row kernel)
};

template <int DT>
__device__ __forceinline__ void load_chunk(const uint8_t *p, float (&v)[8])
{
    if constexpr (DT == kFP32) {
        const uint4 a = ldg_stream(p), b = ldg_stream(p + 16);
        v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
        v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
        v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
        v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
    } else {
        unpack8<DT>(ldg_stream(p), v);
    }
}

template <int DT, int MODE, int CPL>
__global__ void __launch_bounds__(256)
quant_flat_kernel(const QuantArgs a)
{
    constexpr int EB = DT == kFP32 ? 4 : 2;
    const uint32_t base = blockIdx.x * (256u * CPL) + threadIdx.x;
    float v[CPL][8];
    bool ok[CPL];
    int64_t rw[CPL];
    int32_t lc[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const uint32_t f = base + k * 256u;
        ok[k] = f < a.total;
        const uint32_t r = div_c(f, a.dc);
        rw[k] = r;
        lc[k] = (int32_t)(f - r * (uint32_t)a.C);
        if (ok[k]) load_chunk<DT>(a.x + rw[k] * a.x_pitch + (int64_t)lc[k] * 8 * EB, v[k]);
    }
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        if (!ok[k]) continue;
        const int64_t out_off = rw[k] * a.cols + (int64_t)lc[k] * 8;
        uint2 q;
        if constexpr (MODE == kMX) {
            const uint32_t b = e8m0_of(max_quad(amax8(v[k])));
            q = mx_codes8(v[k], mx_inv_scale(b));
            if ((lc[k] & 3) == 0) a.scales[rw[k] * (a.cols / 32) + lc[k] / 4] = (uint8_t)b;
        } else {
            const Fp32Scale sc = fp32_scale(max_row16(amax8(v[k])));
            q = fp32scale_codes8(v[k], sc);
            if ((lc[k] & 15) == 0)
                reinterpret_cast<float *>(a.scales)[rw[k] * (a.cols / 128) + lc[k] / 16] = sc.s;
        }
        stg_stream(a.values + out_off, q);
    }
}

template <int DT, int CPL>
__global__ void __launch_bounds__(kMaxBlock)
quant_row_kernel(const QuantArgs a)
{
    constexpr int EB = DT == kFP32 ? 4 : 2;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int rib = wave / a.WPR;
    const int t = tid - rib * a.NT;
    const int64_t row = (int64_t)blockIdx.x * a.R + rib;
    const bool row_ok = row < a.M;
    float v[CPL][8];
    bool ok[CPL];
    float am = 0.f;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const int c = t + k * a.NT;
        ok[k] = row_ok && c < a.C;
        if (ok[k]) load_chunk<DT>(a.x + row * a.x_pitch + (int64_t)c * 8 * EB, v[k]);
    }
#pragma unroll
    for (int k = 0; k < CPL; ++k)
        if (ok[k]) am = __builtin_fmaxf(am, amax8(v[k]));
    am = max_wave(am);
    __shared__ float redm[kMaxBlock / 64];
    if (a.WPR > 1) {
        if ((tid & 63) == 0) redm[wave] = am;
        lds_barrier();
        am = 0.f;
        for (int i = 0; i < a.WPR; ++i) am = __builtin_fmaxf(am, redm[rib * a.WPR + i]);
    }
    const Fp32Scale sc = fp32_scale(am);
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        if (!ok[k]) continue;
        const int c = t + k * a.NT;
        stg_stream(a.values + row * a.cols + (int64_t)c * 8, fp32scale_codes8(v[k], sc));
        if (c == 0) reinterpret_cast<float *>(a.scales)[row] = sc.s;
    }
}

// ================================================================ launchers
// Row shape for a row of C chunks.  Few rows (latency-bound: every lane of
// a row works through its chunks one after the other, so the row's time
// grows with the chunks per lane): as many lanes as chunks, up to 1024.
// Many rows (bandwidth-bound): two chunks per lane, which measured best or
// within a few % of best on every configured width (hidden 6144 MX + copy,
// 4096 1x128, the 1536 + 512 two-segment per-token rows).  NT is a whole
// number of wavefronts; rows of fewer than 256 lanes are packed several to
// a block.
struct RowShapeRt {
    int NT, CPL, R, WPR;
};
static RowShapeRt row_shape(int C, int64_t M)
{
    RowShapeRt s;
    int cpl = M <= 1024 ? 1 : 2;
    if ((C + cpl - 1) / cpl > 1024) cpl = (C + 1023) / 1024;
    int nt = (C + cpl - 1) / cpl;
    nt = (nt + 63) / 64 * 64;
    s.NT = nt;
    s.CPL = (C + nt - 1) / nt;
    s.R = (nt < 256 && 256 % nt == 0) ? 256 / nt : 1;
    s.WPR = nt / 64;
    return s;
}

template <int DT, int MODE, bool GEMMA, int CPL>
static hipError_t go_norm(const NormArgs &a, int nseg, hipStream_t st)
{
    const int64_t blocks = (a.M + a.R - 1) / a.R;
    if (nseg > 1)
        hipLaunchKernelGGL((norm_quant_kernel<DT, MODE, GEMMA, CPL, 2>), dim3((unsigned)blocks),
                           dim3(a.NT * a.R), 0, st, a);
    else
        hipLaunchKernelGGL((norm_quant_kernel<DT, MODE, GEMMA, CPL, 1>), dim3((unsigned)blocks),
                           dim3(a.NT * a.R), 0, st, a);
    return hipGetLastError();
}

template <int DT, int MODE, bool GEMMA>
static hipError_t go_norm_cpl(const NormArgs &a, int nseg, int CPL, hipStream_t st)
{
    switch (CPL) {
    case 1: return go_norm<DT, MODE, GEMMA, 1>(a, nseg, st);
    case 2: return go_norm<DT, MODE, GEMMA, 2>(a, nseg, st);
    case 3: return go_norm<DT, MODE, GEMMA, 3>(a, nseg, st);
    default: return go_norm<DT, MODE, GEMMA, 4>(a, nseg, st);
    }
}

template <int DT, int MODE>
static hipError_t go_norm_kind(const NormArgs &a, bool gemma, int nseg, int CPL, hipStream_t st)
{
    return gemma ? go_norm_cpl<DT, MODE, true>(a, nseg, CPL, st)
                 : go_norm_cpl<DT, MODE, false>(a, nseg, CPL, st);
}

template <int DT>
static hipError_t go_norm_mode(const NormArgs &a, int mode, bool gemma, int nseg, int CPL, hipStream_t st)
{
    switch (mode) {
    case kMX: return go_norm_kind<DT, kMX>(a, gemma, nseg, CPL, st);
    case kB128: return go_norm_kind<DT, kB128>(a, gemma, nseg, CPL, st);
    default: return go_norm_kind<DT, kPT>(a, gemma, nseg, CPL, st);
    }
}

int launch_norm(const NormPlan &p, void *stream)
{
    NormArgs a;
    a.seg[0] = p.seg[0];
    a.seg[1] = p.nseg > 1 ? p.seg[1] : p.seg[0];
    a.res_in = p.res_in;
    a.res_out = p.res_out;
    a.M = p.M;
    a.eps = p.eps;
    a.C0 = p.seg[0].chunks;
    a.C = p.seg[0].chunks + (p.nseg > 1 ? p.seg[1].chunks : 0);
    const RowShapeRt sh = row_shape(a.C, p.M);
    a.NT = sh.NT;
    a.R = sh.R;
    a.WPR = sh.WPR;
    a.wpr_shift = sh.WPR == 2 ? 1 : 0; // R > 1 only with one or two wavefronts per row
    a.inv_cols0 = 1.0f / (float)p.seg[0].cols;
    a.inv_cols1 = 1.0f / (float)(p.nseg > 1 ? p.seg[1].cols : p.seg[0].cols);
    hipStream_t st = (hipStream_t)stream;
    const bool gemma = p.kind == 1;
    hipError_t e = p.dtype == kFP16 ? go_norm_mode<kFP16>(a, p.mode, gemma, p.nseg, sh.CPL, st)
                                    : go_norm_mode<kBF16>(a, p.mode, gemma, p.nseg, sh.CPL, st);
    return (int)e;
}

template <int MODE, int CPL>
static hipError_t go_act(const ActArgs &a, hipStream_t st)
{
    const uint32_t blocks = (a.total + 256u * CPL - 1) / (256u * CPL);
    hipLaunchKernelGGL((act_quant_kernel<MODE, CPL>), dim3(blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

// Rows per launch of the flat kernels: the flat chunk index stays below
// 2^31 (larger M is covered by several launches over row slices).
static int64_t flat_rows_per_launch(int32_t C) { return ((int64_t)1 << 31) / C; }

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
        a.values = p.values + r0 * p.I;
        a.scales = p.scales + r0 * (p.mode == kMX ? p.I / 32 : 4 * (p.I / 128));
        a.act = p.act ? p.act + r0 * p.I * 2 : nullptr;
        a.C = C;
        a.I = p.I;
        a.total = (uint32_t)(rows * C);
        a.dc = divc((uint32_t)C);
        hipError_t e = p.mode == kMX ? go_act<kMX, 1>(a, st) : go_act<kB128, 1>(a, st);
        if (e != hipSuccess) return (int)e;
    }
    return 0;
}

template <int DT, int MODE, int CPL>
static hipError_t go_quant_flat(const QuantArgs &a, hipStream_t st)
{
    const uint32_t blocks = (a.total + 256u * CPL - 1) / (256u * CPL);
    hipLaunchKernelGGL((quant_flat_kernel<DT, MODE, CPL>), dim3(blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int DT, int CPL>
static hipError_t go_quant_row(const QuantArgs &a, hipStream_t st)
{
    const int64_t blocks = (a.M + a.R - 1) / a.R;
    hipLaunchKernelGGL((quant_row_kernel<DT, CPL>), dim3((unsigned)blocks), dim3(a.NT * a.R), 0, st, a);
    return hipGetLastError();
}

template <int DT>
static hipError_t go_quant(QuantArgs &a, int mode, hipStream_t st)
{
    if (mode == kPT) {
        const RowShapeRt sh = row_shape(a.C, a.M);
        a.NT = sh.NT;
        a.R = sh.R;
        a.WPR = sh.WPR;
        switch (sh.CPL) {
        case 1: return go_quant_row<DT, 1>(a, st);
        case 2: return go_quant_row<DT, 2>(a, st);
        case 3: return go_quant_row<DT, 3>(a, st);
        default: return go_quant_row<DT, 4>(a, st);
        }
    }
    // flat kernels over row slices of at most 2^31 chunks
    constexpr int EB = DT == kFP32 ? 4 : 2;
    const int64_t step = flat_rows_per_launch(a.C);
    const int64_t sbytes = mode == kMX ? a.cols / 32 : 4 * (a.cols / 128);
    QuantArgs b = a;
    b.dc = divc((uint32_t)a.C);
    for (int64_t r0 = 0; r0 < a.M; r0 += step) {
        const int64_t rows = a.M - r0 < step ? a.M - r0 : step;
        b.x = a.x + r0 * a.x_pitch;
        b.values = a.values + r0 * a.cols;
        b.scales = a.scales + r0 * sbytes;
        b.M = rows;
        b.total = (uint32_t)(rows * a.C);
        const hipError_t e = mode == kMX ? go_quant_flat<DT, kMX, 1>(b, st) : go_quant_flat<DT, kB128, 1>(b, st);
        if (e != hipSuccess) return e;
    }
    (void)EB;
    return hipSuccess;
}

int launch_quant(const QuantPlan &p, void *stream)
{
    QuantArgs a;
    a.x = p.x;
    a.x_pitch = p.x_pitch;
    a.values = p.values;
    a.scales = p.scales;
    a.M = p.M;
    a.C = p.cols / 8;
    a.cols = p.cols;
    a.total = 0;
    a.dc = DivC{0, 0};
    a.NT = a.R = a.WPR = 0;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e;
    if (p.dtype == kFP32) e = go_quant<kFP32>(a, p.mode, st);
    else if (p.dtype == kFP16) e = go_quant<kFP16>(a, p.mode, st);
    else e = go_quant<kBF16>(a, p.mode, st);
    return (int)e;
}

} // namespace afq
