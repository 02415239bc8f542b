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
template <int NT>
struct RowShape {
    static constexpr int BS = NT < 256 ? 256 : NT;   // threads per block
    static constexpr int R = BS / NT;                // rows per block
    static constexpr int WPR = NT / 64;              // wavefronts per row
};

struct NormArgs {
    NormSegPlan seg[2];
    const uint8_t *res_in;
    uint8_t *res_out;
    int64_t M;
    float eps;
    int32_t nseg;
    int32_t gemma;
    int32_t C0;      // chunks of segment 0
    int32_t C;       // chunks of both segments
};

template <int DT, int MODE, int NT, int CPL>
__global__ void __launch_bounds__(RowShape<NT>::BS)
norm_quant_kernel(const NormArgs a)
{
    using S = RowShape<NT>;
    static_assert(NT >= 64 && NT % 64 == 0, "rows are whole wavefronts");
    const int tid = threadIdx.x;
    const int rib = tid / NT;
    const int t = tid % NT;
    const int64_t row = (int64_t)blockIdx.x * S::R + rib;
    const bool row_ok = row < a.M;
    const bool has_res = a.res_in != nullptr;

    // ---- issue every load of the row
    uint4 xv[CPL], rv[CPL], wv[CPL];
    bool ok[CPL];
    int sg[CPL], lc[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const int c = t + k * NT;
        ok[k] = row_ok && c < a.C;
        sg[k] = c >= a.C0 ? 1 : 0;
        lc[k] = c - (sg[k] ? a.C0 : 0);
        if (ok[k]) {
            const NormSegPlan &s = sg[k] ? a.seg[1] : a.seg[0];
            xv[k] = ldg<uint4>(s.x + row * s.x_pitch + (int64_t)lc[k] * 16);
            wv[k] = ldg<uint4>(s.w + (int64_t)lc[k] * 16);
            if (has_res)
                rv[k] = ldg<uint4>(a.res_in + (row * a.C0 + lc[k]) * 16);
        }
    }

    // ---- residual add, sum of squares
    float h[CPL][8];
    float ss0 = 0.f, ss1 = 0.f;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        if (!ok[k]) continue;
        float xf[8];
        unpack8<DT>(xv[k], xf);
        if (has_res) {
            float rf[8], sum[8];
            unpack8<DT>(rv[k], rf);
#pragma unroll
            for (int i = 0; i < 8; ++i) sum[i] = xf[i] + rf[i];
            const uint4 hp = round_pack8<DT>(sum, h[k]);
            stg<uint4>(a.res_out + (row * a.C0 + lc[k]) * 16, hp);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) h[k][i] = xf[i];
        }
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) p = __builtin_fmaf(h[k][i], h[k][i], p);
        if (sg[k]) ss1 += p; else ss0 += p;
    }

    // ---- row reduction: DPP inside the wavefront, LDS across wavefronts
    ss0 = sum_lanes<64>(ss0);
    if (a.nseg > 1) ss1 = sum_lanes<64>(ss1);
    if constexpr (S::WPR > 1) {
        __shared__ float red[S::R][S::WPR][2];
        const int w = t / 64;
        if ((t & 63) == 0) {
            red[rib][w][0] = ss0;
            red[rib][w][1] = ss1;
        }
        __syncthreads();
        ss0 = 0.f;
        ss1 = 0.f;
#pragma unroll
        for (int i = 0; i < S::WPR; ++i) {
            ss0 += red[rib][i][0];
            ss1 += red[rib][i][1];
        }
    }
    const float inv0 = 1.0f / __builtin_sqrtf(ss0 / (float)a.seg[0].cols + a.eps);
    const float inv1 = a.nseg > 1 ? 1.0f / __builtin_sqrtf(ss1 / (float)a.seg[1].cols + a.eps) : 0.f;

    // ---- y = h * inv * g, rounded to the dtype (u, kept in place of h),
    //      optional copy
    float (&u)[CPL][8] = h;
    uint32_t am0 = 0, am1 = 0;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        if (!ok[k]) continue;
        const NormSegPlan &s = sg[k] ? a.seg[1] : a.seg[0];
        const float inv = sg[k] ? inv1 : inv0;
        float wf[8], y[8];
        unpack8<DT>(wv[k], wf);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float g = a.gemma ? 1.0f + wf[i] : wf[i];
            y[i] = (h[k][i] * inv) * g;
        }
        const uint4 up = round_pack8<DT>(y, u[k]);
        if (s.normed)
            stg<uint4>(s.normed + (row * s.cols + (int64_t)lc[k] * 8) * 2, up);
        if constexpr (MODE == kPT) {
            const uint32_t m = amax_bits8(u[k]);
            if (sg[k]) am1 = max(am1, m); else am0 = max(am0, m);
        }
    }

    // ---- quantise
    if constexpr (MODE == kPT) {
        am0 = max_lanes<64>(am0);
        if (a.nseg > 1) am1 = max_lanes<64>(am1);
        if constexpr (S::WPR > 1) {
            __shared__ uint32_t redm[S::R][S::WPR][2];
            const int w = t / 64;
            if ((t & 63) == 0) {
                redm[rib][w][0] = am0;
                redm[rib][w][1] = am1;
            }
            __syncthreads();
            am0 = 0;
            am1 = 0;
#pragma unroll
            for (int i = 0; i < S::WPR; ++i) {
                am0 = max(am0, redm[rib][i][0]);
                am1 = max(am1, redm[rib][i][1]);
            }
        }
        const Fp32Scale sc0 = fp32_scale(am0);
        const Fp32Scale sc1 = fp32_scale(am1);
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            if (!ok[k]) continue;
            const NormSegPlan &s = sg[k] ? a.seg[1] : a.seg[0];
            const uint2 q = fp32scale_codes8(u[k], sg[k] ? sc1 : sc0);
            stg<uint2>(s.values + row * s.cols + (int64_t)lc[k] * 8, q);
            if (lc[k] == 0) reinterpret_cast<float *>(s.scales)[row] = sg[k] ? sc1.s : sc0.s;
        }
    } else {
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            if (!ok[k]) continue; // uniform over every quant group
            const NormSegPlan &s = sg[k] ? a.seg[1] : a.seg[0];
            uint2 q;
            if constexpr (MODE == kMX) {
                const uint32_t am = max_quad(amax_bits8(u[k]));
                const uint32_t b = e8m0_from_amax_bits(am);
                q = mx_codes8(u[k], mx_inv_scale(b));
                if ((lc[k] & 3) == 0) s.scales[row * (s.cols / 32) + lc[k] / 4] = (uint8_t)b;
            } else {
                const uint32_t am = max_row16(amax_bits8(u[k]));
                const Fp32Scale sc = fp32_scale(am);
                q = fp32scale_codes8(u[k], sc);
                if ((lc[k] & 15) == 0)
                    reinterpret_cast<float *>(s.scales)[row * (s.cols / 128) + lc[k] / 16] = sc.s;
            }
            stg<uint2>(s.values + row * s.cols + (int64_t)lc[k] * 8, q);
        }
    }
}

// ============================================================ SiLU-and-mul
struct ActArgs {
    const uint8_t *gu;
    int64_t gu_pitch;
    uint8_t *values;
    uint8_t *scales;
    uint8_t *act;
    int64_t total;    // M * C chunks
    int32_t C;        // chunks per row (I / 8)
    int32_t I;
    double invC;      // 1 / C, for the row index of a flat chunk
};

// Row of flat chunk f: a float estimate corrected by at most one step.
__device__ __forceinline__ int64_t row_of(int64_t f, int32_t C, double invC)
{
    int64_t r = (int64_t)((double)f * invC);
    if (r * C > f) --r;
    else if ((r + 1) * C <= f) ++r;
    return r;
}

// silu(g) in fp32, within a few ulp for g >= -80 (exp and an IEEE
// division); below that e^-g leaves the fp32 range and the value is
// computed in fp64 instead.
__device__ __forceinline__ float silu_f32(float g)
{
    if (g < -80.0f) {
        const double gd = (double)g;
        return (float)(gd / (1.0 + exp(-gd)));
    }
    return g / (1.0f + expf(-g));
}

// bf16(silu(g)) for a bf16 gate, exactly rounded: the fp32 value is
// accurate to a few ulp, so its bf16 rounding is the exact one unless the
// value sits within 16 fp32 ulps of a bf16 rounding midpoint (or e^-g
// leaves the fp32 range); those rare cases are redone in fp64.
__device__ __forceinline__ uint32_t silu_bf16(float g)
{
    const float s = g / (1.0f + expf(-g));
    const uint32_t low = __float_as_uint(s) & 0xFFFFu;
    if (g < -80.0f || (low >= 0x8000u - 16u && low <= 0x8000u + 16u)) {
        const double gd = (double)g;
        const double sd = gd / (1.0 + exp(-gd));
        const uint32_t sign = sd < 0.0 ? 0x8000u : 0u;
        const double ad = __builtin_fabs(sd);
        if (ad < 0x1p-126) // bf16 subnormals: a count of 2^-133 steps, RNE
            return sign | (uint32_t)__builtin_rint(ad * 0x1p133);
        // fp64 keeps 52 mantissa bits, bf16 7: drop 45 with RNE (a carry
        // moves into the exponent field by itself)
        const uint64_t db = (uint64_t)__double_as_longlong(ad);
        const uint64_t rn = db + ((1ull << 44) - 1) + ((db >> 45) & 1ull);
        const uint32_t e8 = (uint32_t)((rn >> 52) - 1023 + 127);
        return sign | (e8 << 7) | (uint32_t)((rn >> 45) & 0x7Full);
    }
    return f32_to_bf16(s);
}

template <int MODE, int CPL>
__global__ void __launch_bounds__(256)
act_quant_kernel(const ActArgs a)
{
    const int64_t base = (int64_t)blockIdx.x * (256 * CPL) + threadIdx.x;
    uint4 gv[CPL], uv[CPL];
    bool ok[CPL];
    int64_t rw[CPL];
    int32_t lc[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const int64_t f = base + k * 256;
        ok[k] = f < a.total;
        rw[k] = row_of(f, a.C, a.invC);
        lc[k] = (int32_t)(f - rw[k] * a.C);
        if (ok[k]) {
            const uint8_t *p = a.gu + rw[k] * a.gu_pitch + (int64_t)lc[k] * 16;
            gv[k] = ldg<uint4>(p);
            uv[k] = ldg<uint4>(p + (int64_t)a.I * 2);
        }
    }
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        if (!ok[k]) continue; // uniform over every quant group
        float g[8], up[8], v[8];
        unpack8<kBF16>(gv[k], g);
        unpack8<kBF16>(uv[k], up);
        const int64_t out_off = rw[k] * a.I + (int64_t)lc[k] * 8;
        uint2 q;
        if constexpr (MODE == kMX) {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = silu_f32(g[i]) * up[i];
            if (a.act) {
                float dummy[8];
                stg<uint4>(a.act + out_off * 2, round_pack8<kBF16>(v, dummy));
            }
            const uint32_t am = max_quad(amax_bits8(v));
            const uint32_t b = e8m0_from_amax_bits(am);
            q = mx_codes8(v, mx_inv_scale(b));
            if ((lc[k] & 3) == 0) a.scales[rw[k] * (a.I / 32) + lc[k] / 4] = (uint8_t)b;
        } else {
            float sgm[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) sgm[i] = __uint_as_float(silu_bf16(g[i]) << 16) * up[i];
            const uint4 ap = round_pack8<kBF16>(sgm, v);
            if (a.act) stg<uint4>(a.act + out_off * 2, ap);
            const uint32_t am = max_row16(amax_bits8(v));
            const Fp32Scale sc = fp32_scale(am);
            q = fp32scale_codes8(v, sc);
            if ((lc[k] & 15) == 0)
                reinterpret_cast<float *>(a.scales)[rw[k] * (a.I / 128) + lc[k] / 16] = sc.s;
        }
        stg<uint2>(a.values + out_off, q);
    }
}

// ======================================================= standalone quant
struct QuantArgs {
    const uint8_t *x;
    int64_t x_pitch;
    uint8_t *values;
    uint8_t *scales;
    int64_t total;   // M * C chunks (flat kernel)
    int64_t M;
    int32_t C;       // chunks per row
    int32_t cols;
    double invC;
};

template <int DT>
__device__ __forceinline__ void load_chunk(const uint8_t *p, float (&v)[8])
{
    if constexpr (DT == kFP32) {
        const uint4 a = ldg<uint4>(p), b = ldg<uint4>(p + 16);
        v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
        v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
        v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
        v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
    } else {
        unpack8<DT>(ldg<uint4>(p), v);
    }
}

template <int DT, int MODE, int CPL>
__global__ void __launch_bounds__(256)
quant_flat_kernel(const QuantArgs a)
{
    constexpr int EB = DT == kFP32 ? 4 : 2;
    const int64_t base = (int64_t)blockIdx.x * (256 * CPL) + threadIdx.x;
    float v[CPL][8];
    bool ok[CPL];
    int64_t rw[CPL];
    int32_t lc[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const int64_t f = base + k * 256;
        ok[k] = f < a.total;
        rw[k] = row_of(f, a.C, a.invC);
        lc[k] = (int32_t)(f - rw[k] * a.C);
        if (ok[k]) load_chunk<DT>(a.x + rw[k] * a.x_pitch + (int64_t)lc[k] * 8 * EB, v[k]);
    }
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        if (!ok[k]) continue;
        const int64_t out_off = rw[k] * a.cols + (int64_t)lc[k] * 8;
        uint2 q;
        if constexpr (MODE == kMX) {
            const uint32_t b = e8m0_from_amax_bits(max_quad(amax_bits8(v[k])));
            q = mx_codes8(v[k], mx_inv_scale(b));
            if ((lc[k] & 3) == 0) a.scales[rw[k] * (a.cols / 32) + lc[k] / 4] = (uint8_t)b;
        } else {
            const Fp32Scale sc = fp32_scale(max_row16(amax_bits8(v[k])));
            q = fp32scale_codes8(v[k], sc);
            if ((lc[k] & 15) == 0)
                reinterpret_cast<float *>(a.scales)[rw[k] * (a.cols / 128) + lc[k] / 16] = sc.s;
        }
        stg<uint2>(a.values + out_off, q);
    }
}

template <int DT, int NT, int CPL>
__global__ void __launch_bounds__(RowShape<NT>::BS)
quant_row_kernel(const QuantArgs a)
{
    using S = RowShape<NT>;
    constexpr int EB = DT == kFP32 ? 4 : 2;
    const int tid = threadIdx.x;
    const int rib = tid / NT;
    const int t = tid % NT;
    const int64_t row = (int64_t)blockIdx.x * S::R + rib;
    const bool row_ok = row < a.M;
    float v[CPL][8];
    bool ok[CPL];
    uint32_t am = 0;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const int c = t + k * NT;
        ok[k] = row_ok && c < a.C;
        if (ok[k]) load_chunk<DT>(a.x + row * a.x_pitch + (int64_t)c * 8 * EB, v[k]);
    }
#pragma unroll
    for (int k = 0; k < CPL; ++k)
        if (ok[k]) am = max(am, amax_bits8(v[k]));
    am = max_lanes<64>(am);
    if constexpr (S::WPR > 1) {
        __shared__ uint32_t redm[S::R][S::WPR];
        if ((t & 63) == 0) redm[rib][t / 64] = am;
        __syncthreads();
        am = 0;
#pragma unroll
        for (int i = 0; i < S::WPR; ++i) am = max(am, redm[rib][i]);
    }
    const Fp32Scale sc = fp32_scale(am);
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        if (!ok[k]) continue;
        const int c = t + k * NT;
        stg<uint2>(a.values + row * a.cols + (int64_t)c * 8, fp32scale_codes8(v[k], sc));
        if (c == 0) reinterpret_cast<float *>(a.scales)[row] = sc.s;
    }
}

// ================================================================ launchers
// Threads per row and chunks per lane for a row of C chunks: the smallest
// whole number of wavefronts (power of two, 64..1024) that covers the row
// with at most 4 chunks per lane.
static void row_config(int C, int &NT, int &CPL)
{
    NT = 64;
    while (NT < 1024 && NT * 4 < C) NT *= 2;
    CPL = (C + NT - 1) / NT;
}

template <int DT, int MODE, int NT, int CPL>
static hipError_t go_norm(const NormArgs &a, hipStream_t st)
{
    using S = RowShape<NT>;
    const int64_t blocks = (a.M + S::R - 1) / S::R;
    hipLaunchKernelGGL((norm_quant_kernel<DT, MODE, NT, CPL>), dim3((unsigned)blocks),
                       dim3(S::BS), 0, st, a);
    return hipGetLastError();
}

template <int DT, int MODE, int NT>
static hipError_t go_norm_cpl(const NormArgs &a, int CPL, hipStream_t st)
{
    switch (CPL) {
    case 1: return go_norm<DT, MODE, NT, 1>(a, st);
    case 2: return go_norm<DT, MODE, NT, 2>(a, st);
    case 3: return go_norm<DT, MODE, NT, 3>(a, st);
    default: return go_norm<DT, MODE, NT, 4>(a, st);
    }
}

template <int DT, int MODE>
static hipError_t go_norm_nt(const NormArgs &a, int NT, int CPL, hipStream_t st)
{
    switch (NT) {
    case 64: return go_norm_cpl<DT, MODE, 64>(a, CPL, st);
    case 128: return go_norm_cpl<DT, MODE, 128>(a, CPL, st);
    case 256: return go_norm_cpl<DT, MODE, 256>(a, CPL, st);
    case 512: return go_norm_cpl<DT, MODE, 512>(a, CPL, st);
    default: return go_norm_cpl<DT, MODE, 1024>(a, CPL, st);
    }
}

template <int DT>
static hipError_t go_norm_mode(const NormArgs &a, int mode, int NT, int CPL, hipStream_t st)
{
    switch (mode) {
    case kMX: return go_norm_nt<DT, kMX>(a, NT, CPL, st);
    case kB128: return go_norm_nt<DT, kB128>(a, NT, CPL, st);
    default: return go_norm_nt<DT, kPT>(a, NT, CPL, st);
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
    a.nseg = p.nseg;
    a.gemma = p.kind;
    a.C0 = p.seg[0].chunks;
    a.C = p.seg[0].chunks + (p.nseg > 1 ? p.seg[1].chunks : 0);
    int NT, CPL;
    row_config(a.C, NT, CPL);
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = p.dtype == kFP16 ? go_norm_mode<kFP16>(a, p.mode, NT, CPL, st)
                                    : go_norm_mode<kBF16>(a, p.mode, NT, CPL, st);
    return (int)e;
}

// Chunks per lane of the flat kernels.
constexpr int kFlatCPL = 2;

int launch_act(const ActPlan &p, void *stream)
{
    ActArgs a;
    a.gu = p.gu;
    a.gu_pitch = p.gu_pitch;
    a.values = p.values;
    a.scales = p.scales;
    a.act = p.act;
    a.C = p.I / 8;
    a.I = p.I;
    a.total = p.M * (int64_t)a.C;
    a.invC = 1.0 / (double)a.C;
    const int64_t blocks = (a.total + 256 * kFlatCPL - 1) / (256 * kFlatCPL);
    hipStream_t st = (hipStream_t)stream;
    if (p.mode == kMX)
        hipLaunchKernelGGL((act_quant_kernel<kMX, kFlatCPL>), dim3((unsigned)blocks), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((act_quant_kernel<kB128, kFlatCPL>), dim3((unsigned)blocks), dim3(256), 0, st, a);
    return (int)hipGetLastError();
}

template <int DT>
static hipError_t go_quant(const QuantArgs &a, int mode, hipStream_t st)
{
    if (mode == kPT) {
        int NT, CPL;
        row_config(a.C, NT, CPL);
        // the row kernel covers up to 4 chunks per lane
        auto launch = [&](auto kern, int nt) {
            const int bs = nt < 256 ? 256 : nt;
            const int64_t R = bs / nt;
            hipLaunchKernelGGL(kern, dim3((unsigned)((a.M + R - 1) / R)), dim3(bs), 0, st, a);
        };
#define AFQ_QROW(NT_, CPL_) \
        if (NT == NT_ && CPL == CPL_) { launch(quant_row_kernel<DT, NT_, CPL_>, NT_); return hipGetLastError(); }
#define AFQ_QROW4(NT_) AFQ_QROW(NT_, 1) AFQ_QROW(NT_, 2) AFQ_QROW(NT_, 3) AFQ_QROW(NT_, 4)
        AFQ_QROW4(64) AFQ_QROW4(128) AFQ_QROW4(256) AFQ_QROW4(512) AFQ_QROW4(1024)
#undef AFQ_QROW4
#undef AFQ_QROW
        return hipErrorInvalidValue;
    }
    const int64_t blocks = (a.total + 256 * kFlatCPL - 1) / (256 * kFlatCPL);
    if (mode == kMX)
        hipLaunchKernelGGL((quant_flat_kernel<DT, kMX, kFlatCPL>), dim3((unsigned)blocks), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((quant_flat_kernel<DT, kB128, kFlatCPL>), dim3((unsigned)blocks), dim3(256), 0, st, a);
    return hipGetLastError();
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
    a.total = p.M * (int64_t)a.C;
    a.invC = 1.0 / (double)a.C;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e;
    if (p.dtype == kFP32) e = go_quant<kFP32>(a, p.mode, st);
    else if (p.dtype == kFP16) e = go_quant<kFP16>(a, p.mode, st);
    else e = go_quant<kBF16>(a, p.mode, st);
    return (int)e;
}

} // namespace afq
