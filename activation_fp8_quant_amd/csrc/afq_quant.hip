// afq_quant.hip -- the standalone row-wise FP8 quantisers (the separate
// quant kernel of the unfused chains):
//
//   quant_flat_kernel  1x32 / 1x128 quantisation on a flat chunk index
//   quant_row_kernel   per-token quantisation (one row reduction)

#include "afq_device.hpp"
#include "afq_internal.h"
#include "afq_launch.hpp"

namespace afq {

constexpr int kMaxBlock = 1024;

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
    // outputs are dense rows of C chunks (C a multiple of 4, of 16 for
    // 1x128): chunk f's codes start at element 8 f and its group's scale is
    // entry f / 4 (MX) or f / 16 (1x128); only the input, whose rows have a
    // pitch, needs f's row and column
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const uint32_t f = base + k * 256u;
        ok[k] = f < a.total;
        if (ok[k]) {
            const uint32_t r = div_c(f, a.dc);
            const int32_t lc = (int32_t)(f - r * (uint32_t)a.C);
            load_chunk<DT>(a.x + (int64_t)r * a.x_pitch + (int64_t)lc * 8 * EB, v[k]);
        }
    }
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        if (!ok[k]) continue;
        const uint32_t f = base + k * 256u;
        uint2 q;
        if constexpr (MODE == kMX) {
            const uint32_t b = e8m0_of(max_quad(amax8(v[k])));
            q = mx_codes8(v[k], mx_inv_scale(b));
            if ((f & 3u) == 0) a.scales[f >> 2] = (uint8_t)b;
        } else {
            const Fp32Scale sc = fp32_scale(max_row16(amax8(v[k])));
            q = fp32scale_codes8(v[k], sc);
            if ((f & 15u) == 0) reinterpret_cast<float *>(a.scales)[f >> 4] = sc.s;
        }
        stg_stream(a.values + (int64_t)f * 8, q);
    }
}

template <int DT, int CPL>
__global__ void __launch_bounds__(kMaxBlock)
quant_row_kernel(const QuantArgs a)
{
    constexpr int EB = DT == kFP32 ? 4 : 2;
    const int tid = threadIdx.x;
    // rows are whole wavefronts: the wavefront and its row are uniform
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rib = wave / a.WPR;
    const int t = tid - rib * a.NT;
    const int64_t row = (int64_t)blockIdx.x * a.R + rib;
    const bool row_ok = row < a.M;
    float v[CPL][8];
    bool ok[CPL];
    float am = 0.f;
    // Every lane loads, without a branch: a lane off the rows or past the
    // row's end reads an in-bounds chunk (the last row's, the row's last)
    // and leaves it out of the max and the stores.  Loads under a lane mask
    // made the compiler wait for each before issuing the next.
    const int64_t lrow = row_ok ? row : a.M - 1;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const int c = t + k * a.NT;
        ok[k] = row_ok && c < a.C;
        const int lc = c < a.C ? c : a.C - 1;
        load_chunk<DT>(a.x + lrow * a.x_pitch + (int64_t)lc * 8 * EB, v[k]);
    }
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const float m = amax8(v[k]);
        am = ok[k] ? __builtin_fmaxf(am, m) : am;
    }
    am = max_wave(am);
    __shared__ float redm[kMaxBlock / 64];
    if (a.WPR > 1) {
        if ((tid & 63) == 0) redm[wave] = am;
        lds_barrier();
        float unused;
        am = lds_rows_max<1>(&redm[rib * a.WPR], &redm[rib * a.WPR], a.WPR, unused);
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

// ================================================================ launcher
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
        const RowShapeRt sh = quant_row_shape(a.C, a.M, device_cus());
        a.NT = sh.NT;
        a.R = sh.R;
        a.WPR = sh.WPR;
        // one launch per row slice (a single one below ~2^31 / NT rows)
        const int64_t step = row_rows_per_launch(a.NT, a.R);
        QuantArgs b = a;
        for (int64_t r0 = 0; r0 < a.M; r0 += step) {
            b.M = a.M - r0 < step ? a.M - r0 : step;
            b.x = a.x + r0 * a.x_pitch;
            b.values = a.values + r0 * a.cols;
            b.scales = a.scales + r0 * 4;
            hipError_t e;
            switch (sh.CPL) {
            case 1: e = go_quant_row<DT, 1>(b, st); break;
            case 2: e = go_quant_row<DT, 2>(b, st); break;
            case 3: e = go_quant_row<DT, 3>(b, st); break;
            default: e = go_quant_row<DT, 4>(b, st); break;
            }
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    // flat kernels over row slices of at most 2^31 chunks
    const int64_t step = flat_rows_per_launch(a.C);
    const int64_t sbytes = scale_row_bytes(mode, a.cols);
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
