// afq_norm.hip -- residual add + RMSNorm fused with FP8 quantisation.
//
// norm_quant_kernel: one row (one or two segments) per NT lanes; residual
// add, fp32 sum of squares (DPP inside a wavefront, one LDS step across
// wavefronts), scale by the weight, round to the activation dtype,
// quantise.  HBM-bound row work: no dense contraction, so no MFMA.
//
// Every lane issues all of its 16-byte loads before it does any arithmetic,
// so a row's whole input is in flight at once; stores are 16 B (dtype
// outputs) and 8 B (codes) per lane, contiguous across the wavefront.

#include "afq_device.hpp"
#include "afq_internal.h"
#include "afq_launch.hpp"

#include <atomic>

namespace afq {

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
    double rcols0;     // RN64(1 / cols) of each segment (fp32-direct inverse RMS)
    double rcols1;
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

// The sum of squares is formed in an order fixed by the row width alone, so
// that a row's outputs do not depend on the launch's row shape (and through
// it on the row count): each chunk's 8 squares in a fixed chain, each
// aligned 64-chunk block of the row by the wavefront tree, the blocks by a
// tree over their index (lds_blocks_sum).  At one chunk per lane every
// wavefront of the row is one block, and the first program below forms
// that order directly (lanes past the row skip their loads and stores); at
// two to four chunks per lane the second reduces each of a wavefront's
// slots (one block each) separately and adds the blocks in LDS.  In the
// second, lanes off the row load the first chunk of the last row and
// compute like every lane, only their stores are skipped: no branch skips
// a load or its use, which keeps the compiler's waits on the vector memory
// counter exact (with a load it had to assume pending, it waited for every
// store in flight too).
//
// F32Q (1x128 / per-token): the fp32-direct variant.  The quantiser reads
// the fp32 normed value y = fl32(fl32(h * inv32) * g32) instead of its
// dtype rounding, with inv32 = fl32(1 / sqrt(mean(h^2) + eps)).  To make
// inv32 the correctly rounded value (so that y, and with it every scale and
// code, is reproducible) the sum of squares is accumulated in fp64 (each
// h^2 is exact there) and the square root and reciprocal are those of fp64
// IEEE operations rounded once to fp32 (inv_rms_f32q).
//
// SEGU (two segments only): the first segment's chunk count C0 is a
// multiple of 64, so the chunks of slot k of a wavefront (64 consecutive
// chunks starting at a multiple of 64) all lie in one segment; the segment
// of each slot is then known per wavefront (scalar registers), and a
// wavefront skips the reductions of a segment it holds no chunk of.
template <int DT, int MODE, bool GEMMA, int CPL, int NSEG, bool SEGU, bool F32Q>
__global__ void __launch_bounds__(kMaxBlock)
norm_quant_kernel(const NormArgs a)
{
    if constexpr (CPL == 1) {
        const int tid = threadIdx.x;
        // rows are whole wavefronts: the wavefront, its row and everything
        // derived from them are wavefront-uniform (kept in scalar registers)
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int rib = a.R == 1 ? 0 : (wave >> a.wpr_shift); // row within the block
        const int t = tid - rib * a.NT;                       // lane within the row
        const int tw = wave * 64 - rib * a.NT;                // t of the wavefront's lane 0
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
                sg[k] = (SEGU ? tw + k * a.NT : c) >= a.C0 ? 1 : 0;
                lc[k] = c - (sg[k] ? a.C0 : 0);
            }
            if (ok[k]) {
                xv[k] = ldg_stream((sg[k] ? xrow1 : xrow0) + lc[k] * 16);
                wv[k] = ldg<uint4>((sg[k] ? a.seg[1].w : a.seg[0].w) + lc[k] * 16);
                if (has_res)
                    rv[k] = ldg_stream(a.res_in + rrow + lc[k] * 16);
            }
        }
        // Every load of the row is needed before the first store, so wait for
        // them all here, before any branch.  Left to itself the compiler cannot
        // tell at the joins below which loads a wavefront issued, and waits on
        // the memory counter after the residual store, that is for the store
        // (headline 146.8 -> 146.3 us, the 1x128 norm at 4096 rows 22.1 ->
        // 21.6 us, its fp32-direct form 23.2 -> 21.9 us; launches of a few
        // rows 0.01-0.04 us slower).  The multi-chunk path below keeps the
        // compiler's per-slot waits: the same early wait there was slower
        // (width 6144 at 1024 rows 11.2 -> 12.1 us).
        wait_loads();

        // ---- residual add (h = round_dt(x + r), stored), sum of squares
        float h[CPL][8];
        float ss0 = 0.f, ss1 = 0.f;
        double sd0 = 0.0, sd1 = 0.0; // F32Q
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
            if constexpr (F32Q) {
                double sd = 0.0;
    #pragma unroll
                for (int i = 0; i < 8; ++i) sd = __builtin_fma((double)h[k][i], (double)h[k][i], sd);
                if (NSEG > 1 && sg[k]) sd1 += sd;
                else sd0 += sd;
            } else {
                if (NSEG > 1 && sg[k]) ss1 = sumsq8<DT>(hp, ss1);
                else ss0 = sumsq8<DT>(hp, ss0);
            }
        }

        // segments this wavefront holds chunks of (with SEGU a scalar fact; a
        // segment it does not hold contributes zeros, so its reduction is skipped)
        bool has0 = true, has1 = NSEG > 1;
        if constexpr (NSEG > 1 && SEGU) {
            has0 = false;
            has1 = false;
    #pragma unroll
            for (int k = 0; k < CPL; ++k) {
                if (sg[k]) has1 = true;
                else has0 = true;
            }
        }

        // ---- row reduction: DPP/permlane inside the wavefront, one LDS step
        //      across the wavefronts of the row
        // (LDS partials are segment-major: a row's partials are contiguous)
        const int p0 = rib * a.WPR;
        __shared__ float redm[2][kMaxBlock / 64];
        float inv0, inv1;
        if constexpr (F32Q) {
            __shared__ double redd[2][kMaxBlock / 64];
            if (has0) sd0 = sum_wave_f64(sd0);
            if constexpr (NSEG > 1)
                if (has1) sd1 = sum_wave_f64(sd1);
            if (a.WPR > 1) {
                if ((tid & 63) == 0) {
                    redd[0][wave] = sd0;
                    if constexpr (NSEG > 1) redd[1][wave] = sd1;
                }
                lds_barrier();
                sd0 = lds_rows_sum_f64<NSEG>(&redd[0][p0], &redd[1][p0], a.WPR, sd1);
            }
            inv0 = inv_rms_f32q(sd0, a.seg[0].cols, a.rcols0, a.eps);
            inv1 = NSEG > 1 ? inv_rms_f32q(sd1, a.seg[1].cols, a.rcols1, a.eps) : inv0;
        } else {
            __shared__ float red[2][kMaxBlock / 64];
            if (has0) ss0 = sum_wave(ss0);
            if constexpr (NSEG > 1)
                if (has1) ss1 = sum_wave(ss1);
            if (a.WPR > 1) {
                if ((tid & 63) == 0) {
                    red[0][wave] = ss0;
                    if constexpr (NSEG > 1) red[1][wave] = ss1;
                }
                lds_barrier();
                ss0 = lds_rows_sum<NSEG>(&red[0][p0], &red[1][p0], a.WPR, ss1);
            }
            inv0 = rsqrt_nr(__builtin_fmaf(ss0, a.inv_cols0, a.eps));
            inv1 = NSEG > 1 ? rsqrt_nr(__builtin_fmaf(ss1, a.inv_cols1, a.eps)) : inv0;
        }

        // ---- u = round_dt(h * inv * g), kept in place of h; optional copy.
        //      Gemma: g * inv = (1 + w) inv as one FMA.  F32Q: y = (h inv) g
        //      in that order is kept in place of h (the quantiser's input), and
        //      only the copy is rounded.
        float am0 = 0.f, am1 = 0.f;
    #pragma unroll
        for (int k = 0; k < CPL; ++k) {
            if (!ok[k]) continue;
            const float inv = sg[k] ? inv1 : inv0;
            float wf[8];
            unpack8<DT>(wv[k], wf);
            if constexpr (F32Q) {
    #pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float g = GEMMA ? 1.0f + wf[i] : wf[i];
                    h[k][i] = (h[k][i] * inv) * g;
                }
            } else {
    #pragma unroll
                for (int i = 0; i < 8; ++i)
                    h[k][i] *= GEMMA ? __builtin_fmaf(wf[i], inv, inv) : wf[i] * inv;
            }
            const uint4 up = F32Q ? pack8<DT>(h[k]) : round8<DT>(h[k]);
            uint8_t *normed = sg[k] ? a.seg[1].normed : a.seg[0].normed;
            const int32_t cols = sg[k] ? a.seg[1].cols : a.seg[0].cols;
            if (normed)
                stg_stream(normed + (row * cols + (int64_t)lc[k] * 8) * 2, up);
            if constexpr (MODE == kPT) {
                const float m = amax8(h[k]);
                if (NSEG > 1 && sg[k]) am1 = __builtin_fmaxf(am1, m); else am0 = __builtin_fmaxf(am0, m);
            }
        }

        // ---- quantise (nothing more for a copy-only launch)
        if constexpr (MODE == kNone) {
            return;
        } else if constexpr (MODE == kPT) {
            if (has0) am0 = max_wave(am0);
            if constexpr (NSEG > 1)
                if (has1) am1 = max_wave(am1);
            if (a.WPR > 1) {
                if ((tid & 63) == 0) {
                    redm[0][wave] = am0;
                    if constexpr (NSEG > 1) redm[1][wave] = am1;
                }
                lds_barrier();
                am0 = lds_rows_max<NSEG>(&redm[0][p0], &redm[1][p0], a.WPR, am1);
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
                    if ((lc[k] & 3) == 0) stg_scale(s.scales + row * (s.cols / 32) + lc[k] / 4, b);
                } else {
                    const Fp32Scale sc = fp32_scale(max_row16(amax8(h[k])));
                    q = fp32scale_codes8(h[k], sc);
                    if ((lc[k] & 15) == 0)
                        stg_scale(reinterpret_cast<float *>(s.scales) + row * (s.cols / 128) + lc[k] / 16, sc.s);
                }
                stg_stream(s.values + row * s.cols + (int64_t)lc[k] * 8, q);
            }
        }
    } else {
        const int tid = threadIdx.x;
        // rows are whole wavefronts: the wavefront, its row and everything
        // derived from them are wavefront-uniform (kept in scalar registers)
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int rib = a.R == 1 ? 0 : (wave >> a.wpr_shift); // row within the block
        const int t = tid - rib * a.NT;                       // lane within the row
        const int tw = wave * 64 - rib * a.NT;                // t of the wavefront's lane 0
        const int64_t row = (int64_t)blockIdx.x * a.R + rib;
        const bool row_ok = row < a.M;
        const bool has_res = a.res_in != nullptr;

        // per-row bases.  Lanes off the row (past its last chunk, or in a row
        // slot past M) load the first chunk of the last row instead and compute
        // on it like every lane; only their stores are skipped.  No branch then
        // skips a load or its use, so the compiler's waits on the vector memory
        // counter stay exact (a load it has to assume pending would make it
        // wait for every store in flight too).
        const int64_t lrow = row_ok ? row : a.M - 1; // a row that exists
        const uint8_t *xrow0 = a.seg[0].x + lrow * a.seg[0].x_pitch;
        const uint8_t *xrow1 = NSEG > 1 ? a.seg[1].x + lrow * a.seg[1].x_pitch : xrow0;
        const int64_t rrow = row * a.C0 * 16;  // stores (row_ok only)
        const int64_t rlrow = lrow * a.C0 * 16; // loads

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
                sg[k] = (SEGU ? tw + k * a.NT : c) >= a.C0 ? 1 : 0;
                lc[k] = c - (sg[k] ? a.C0 : 0);
            }
            const bool in = c < a.C;       // a chunk of the row (any row)
            const int ls = in ? lc[k] : 0; // the chunk this lane loads
            // ... and its segment: with SEGU the slot's (wavefront-uniform,
            // so the pointers are chosen in scalar registers; a lane past
            // the row loads chunk 0 of that segment)
            const bool s1 = NSEG > 1 && (SEGU ? sg[k] != 0 : (in && sg[k] != 0));
            xv[k] = ldg_stream((s1 ? xrow1 : xrow0) + ls * 16);
            wv[k] = ldg<uint4>((s1 ? a.seg[1].w : a.seg[0].w) + ls * 16);
            if (has_res) rv[k] = ldg_stream(a.res_in + rlrow + ls * 16);
        }

        // ---- residual add (h = round_dt(x + r), stored), squares.
        //      The mean square is summed in an order fixed by the row width
        //      alone, never by the launch's row shape, so that a row's outputs
        //      do not depend on the shape (and through it on the row count):
        //      each chunk's 8 squares in a fixed chain; each 64-chunk block of
        //      the row (one slot of one wavefront, in every shape) by the fixed
        //      wavefront tree; the blocks by a fixed tree over their index.
        float h[CPL][8];
        float sq[CPL];   // this lane's chunk of slot k: its sum of squares
        double sqd[CPL]; // F32Q: the same in fp64 (each square exact)
    #pragma unroll
        for (int k = 0; k < CPL; ++k) {
            uint4 hp = xv[k];
            if (has_res) {
                float rf[8];
                unpack8<DT>(xv[k], h[k]);
                unpack8<DT>(rv[k], rf);
    #pragma unroll
                for (int i = 0; i < 8; ++i) h[k][i] += rf[i];
                hp = pack8<DT>(h[k]);
                if (ok[k]) stg_stream(a.res_out + rrow + lc[k] * 16, hp);
            }
            unpack8<DT>(hp, h[k]);
            sq[k] = 0.f;
            sqd[k] = 0.0;
            if constexpr (F32Q) {
                double d = 0.0;
    #pragma unroll
                for (int i = 0; i < 8; ++i) d = __builtin_fma((double)h[k][i], (double)h[k][i], d);
                sqd[k] = ok[k] ? d : 0.0;
            } else {
                const float f = sumsq8<DT>(hp, 0.f);
                sq[k] = ok[k] ? f : 0.f;
            }
        }

        // ---- row reduction.  Slot k of this wavefront is the aligned block
        //      (tw + k NT) / 64 of the row.  Every block total goes to LDS at its
        //      block index (0 for a segment the block holds no chunk of) and,
        //      after one barrier, the blocks of each segment are added by
        //      lds_blocks_sum.  With SEGU a slot lies in one segment, and the
        //      other segment's reduction is skipped.
        const int NB = (a.C + 63) >> 6; // blocks of the row (a function of the width)
        const int pb = rib * NB;        // this row's first LDS entry
        __shared__ float redm[2][kMaxBlock / 64];
        float inv0, inv1;
        auto slot_seg = [&](int k, int s) -> bool { // may slot k hold chunks of segment s
            if constexpr (NSEG == 1) return s == 0;
            else if constexpr (SEGU) return sg[k] == s;
            else return true;
        };
        if constexpr (F32Q) {
            __shared__ double redd[2][64];
            double t0, t1;
    #pragma unroll
            for (int k = 0; k < CPL; ++k) {
                const int b = (tw + k * a.NT) >> 6;
                if (b >= NB) continue; // wavefront-uniform
                double b0 = 0.0, b1 = 0.0;
                if constexpr (NSEG == 1) {
                    b0 = sum_wave_f64(sqd[k]);
                } else {
                    if (slot_seg(k, 0)) b0 = sum_wave_f64(sg[k] ? 0.0 : sqd[k]);
                    if (slot_seg(k, 1)) b1 = sum_wave_f64(sg[k] ? sqd[k] : 0.0);
                }
                if ((tid & 63) == 0) {
                    redd[0][pb + b] = b0;
                    if constexpr (NSEG > 1) redd[1][pb + b] = b1;
                }
            }
            lds_barrier();
            t0 = lds_blocks_sum_f64<NSEG>(&redd[0][pb], &redd[1][pb], NB, t1);
            inv0 = inv_rms_f32q(t0, a.seg[0].cols, a.rcols0, a.eps);
            inv1 = NSEG > 1 ? inv_rms_f32q(t1, a.seg[1].cols, a.rcols1, a.eps) : inv0;
        } else {
            __shared__ float red[2][64];
            float t0, t1;
    #pragma unroll
            for (int k = 0; k < CPL; ++k) {
                const int b = (tw + k * a.NT) >> 6;
                if (b >= NB) continue; // wavefront-uniform
                float b0 = 0.f, b1 = 0.f;
                if constexpr (NSEG == 1) {
                    b0 = sum_wave(sq[k]);
                } else {
                    if (slot_seg(k, 0)) b0 = sum_wave(sg[k] ? 0.f : sq[k]);
                    if (slot_seg(k, 1)) b1 = sum_wave(sg[k] ? sq[k] : 0.f);
                }
                if ((tid & 63) == 0) {
                    red[0][pb + b] = b0;
                    if constexpr (NSEG > 1) red[1][pb + b] = b1;
                }
            }
            lds_barrier();
            t0 = lds_blocks_sum<NSEG>(&red[0][pb], &red[1][pb], NB, t1);
            inv0 = rsqrt_nr(__builtin_fmaf(t0, a.inv_cols0, a.eps));
            inv1 = NSEG > 1 ? rsqrt_nr(__builtin_fmaf(t1, a.inv_cols1, a.eps)) : inv0;
        }

        // ---- u = round_dt(h * inv * g), kept in place of h; optional copy.
        //      Gemma: g * inv = (1 + w) inv as one FMA.  F32Q: y = (h inv) g
        //      in that order is kept in place of h (the quantiser's input), and
        //      only the copy is rounded.
        float am0 = 0.f, am1 = 0.f;
    #pragma unroll
        for (int k = 0; k < CPL; ++k) {
            const float inv = sg[k] ? inv1 : inv0;
            float wf[8];
            unpack8<DT>(wv[k], wf);
            if constexpr (F32Q) {
    #pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float g = GEMMA ? 1.0f + wf[i] : wf[i];
                    h[k][i] = (h[k][i] * inv) * g;
                }
            } else {
    #pragma unroll
                for (int i = 0; i < 8; ++i)
                    h[k][i] *= GEMMA ? __builtin_fmaf(wf[i], inv, inv) : wf[i] * inv;
            }
            const uint4 up = F32Q ? pack8<DT>(h[k]) : round8<DT>(h[k]);
            uint8_t *normed = sg[k] ? a.seg[1].normed : a.seg[0].normed;
            const int32_t cols = sg[k] ? a.seg[1].cols : a.seg[0].cols;
            if (normed && ok[k])
                stg_stream(normed + (row * cols + (int64_t)lc[k] * 8) * 2, up);
            if constexpr (MODE == kPT) {
                const float m = ok[k] ? amax8(h[k]) : 0.f;
                if (NSEG > 1 && sg[k]) am1 = __builtin_fmaxf(am1, m); else am0 = __builtin_fmaxf(am0, m);
            }
        }

        // ---- quantise (nothing more for a copy-only launch)
        if constexpr (MODE == kNone) {
            return;
        } else if constexpr (MODE == kPT) {
            // segments this wavefront holds chunks of (with SEGU a scalar fact; a
            // segment it does not hold contributes zeros, so its max is skipped)
            bool has0 = true, has1 = NSEG > 1;
            if constexpr (NSEG > 1 && SEGU) {
                has0 = false;
                has1 = false;
    #pragma unroll
                for (int k = 0; k < CPL; ++k) {
                    if (sg[k]) has1 = true;
                    else has0 = true;
                }
            }
            if (has0) am0 = max_wave(am0);
            if constexpr (NSEG > 1)
                if (has1) am1 = max_wave(am1);
            const int p0 = rib * a.WPR; // this row's first wavefront in the block
            if (a.WPR > 1) {
                if ((tid & 63) == 0) {
                    redm[0][wave] = am0;
                    if constexpr (NSEG > 1) redm[1][wave] = am1;
                }
                lds_barrier();
                am0 = lds_rows_max<NSEG>(&redm[0][p0], &redm[1][p0], a.WPR, am1);
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
            uint2 q[CPL];
            uint32_t b[CPL];
            Fp32Scale sc[CPL];
    #pragma unroll
            for (int k = 0; k < CPL; ++k) { // lanes off the row: their own groups only
                if constexpr (MODE == kMX) {
                    b[k] = e8m0_of(max_quad(amax8(h[k])));
                    q[k] = mx_codes8(h[k], mx_inv_scale(b[k]));
                } else {
                    sc[k] = fp32_scale(max_row16(amax8(h[k])));
                    q[k] = fp32scale_codes8(h[k], sc[k]);
                }
            }
    #pragma unroll
            for (int k = 0; k < CPL; ++k) {
                if (!ok[k]) continue;
                const NormSegPlan &s = sg[k] ? a.seg[1] : a.seg[0];
                if constexpr (MODE == kMX) {
                    if ((lc[k] & 3) == 0) stg_scale(s.scales + row * (s.cols / 32) + lc[k] / 4, b[k]);
                } else {
                    if ((lc[k] & 15) == 0)
                        stg_scale(reinterpret_cast<float *>(s.scales) + row * (s.cols / 128) + lc[k] / 16, sc[k].s);
                }
                stg_stream(s.values + row * s.cols + (int64_t)lc[k] * 8, q[k]);
            }
        }
    }
}

// ============================================ per-token, one wavefront a row
// Two per-wavefront reductions at once.  v_permlane16_swap(a, b) trades the
// odd 16-lane rows of a with the even rows of b, so after it a holds rows
// (a0, b0, a2, b2) and b rows (a1, b1, a3, b3), and their sum is
// (a0+a1, b0+b1, a2+a3, b2+b3); v_permlane32_swap(x, y) then pairs the lower
// halves with the upper ones.  With every 16-lane row of the inputs uniform
// (after sum_row16 / max_row16) this forms the wavefront tree of sum_wave /
// max_wave -- (r0 + r1) + (r2 + r3) over the row values r -- for two (or
// four) values at once, operand for operand.
__device__ __forceinline__ float sum_pair16(float a, float b)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float sum_pair32(float a, float b)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float max_pair16(float a, float b)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(max((uint32_t)p[0], (uint32_t)p[1]));
}
__device__ __forceinline__ float max_pair32(float a, float b)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(max((uint32_t)p[0], (uint32_t)p[1]));
}

// Per-token rows of 65..256 chunks (widths 520..2048, one or two segments)
// on one wavefront each, CPL = 2..4 chunks per lane, R = 256 / 64 rows per
// block.  Everything a row needs stays inside its wavefront: no LDS and no
// barrier, and the per-row work (two sums of squares, two maxima, the
// reciprocal square roots and the scales) is done once per row instead of
// once per wavefront of it.  The numerics are those of norm_quant_kernel at
// every shape: slot k of the lane is the aligned 64-chunk block k, each
// block is summed by the wavefront tree and the blocks by the tree of
// lds_blocks_sum, which for at most four blocks is (b0 + b1) + (b2 + b3)
// (a missing block adds an exact zero); the block trees of slots 0-1 and
// 2-3 are formed pairwise (sum_pair16 / sum_pair32), which leaves block k's
// total in 16-lane row k, and the segment totals come from the same pairing
// applied to the rows of each segment.  Lanes off the row load chunk 0 of
// the row's segment and compute on it; only their stores are skipped.
//
// KB: 0 for one segment; for two segments whose boundary lies on a 64-chunk
// line, the first slot of the second segment (1..3), so that every slot's
// segment, scale and pointers are known at compile time; -1 for two
// segments with the boundary inside a slot (segment chosen per lane).
template <int DT, bool GEMMA, int CPL, int NSEG, int KB>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8, 8)))
norm_pt_wave_kernel(const NormArgs a)
{
    static_assert(CPL >= 2 && CPL <= 4, "one wavefront holds at most 4 blocks of 64 chunks");
    static_assert((NSEG == 1) == (KB == 0) && KB >= -1 && KB < CPL, "segment boundary slot");
    constexpr bool SEGU = KB > 0;
    const int t = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t row = (int64_t)blockIdx.x * a.R + wave;
    if (row >= a.M) return; // the whole wavefront: nothing waits for it
    const bool has_res = NSEG == 1 && a.res_in != nullptr; // two segments take no residual
    const uint8_t *xrow0 = a.seg[0].x + row * a.seg[0].x_pitch;
    const uint8_t *xrow1 = NSEG > 1 ? a.seg[1].x + row * a.seg[1].x_pitch : xrow0;
    const int64_t rrow = row * a.C0 * 16;

    // ---- issue every load of the row
    uint4 xv[CPL], rv[CPL], wv[CPL];
    bool ok[CPL];
    int sg[CPL], lc[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const int c = t + 64 * k;
        ok[k] = c < a.C;
        if constexpr (NSEG == 1) {
            sg[k] = 0;
            lc[k] = c;
        } else if constexpr (SEGU) {
            sg[k] = k >= KB ? 1 : 0;
            lc[k] = k >= KB ? t + 64 * (k - KB) : c;
        } else {
            sg[k] = c >= a.C0 ? 1 : 0;
            lc[k] = c - (sg[k] ? a.C0 : 0);
        }
        const int ls = ok[k] ? lc[k] : 0;
        const bool s1 = NSEG > 1 && (SEGU ? sg[k] != 0 : (ok[k] && sg[k] != 0));
        xv[k] = ldg_stream((s1 ? xrow1 : xrow0) + ls * 16);
        wv[k] = ldg<uint4>((s1 ? a.seg[1].w : a.seg[0].w) + ls * 16);
        if (has_res) rv[k] = ldg_stream(a.res_in + rrow + ls * 16);
    }

    // ---- residual add (h = round_dt(x + r), stored), squares per chunk.
    //      Rows stay packed in the dtype (hp) between the steps, which keeps
    //      the kernel within 64 VGPRs: eight wavefronts per SIMD, so that a
    //      round of the GPU holds 32 rows per compute unit.
    uint4 hp[CPL];
    float sq[CPL];            // this lane's chunk of slot k: its sum of squares
    float sq0[CPL], sq1[CPL]; // the same split by segment (two segments, unaligned)
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        hp[k] = xv[k];
        if (has_res) {
            float hf[8], rf[8];
            unpack8<DT>(xv[k], hf);
            unpack8<DT>(rv[k], rf);
#pragma unroll
            for (int i = 0; i < 8; ++i) hf[i] += rf[i];
            hp[k] = pack8<DT>(hf);
            if (ok[k]) stg_stream(a.res_out + rrow + lc[k] * 16, hp[k]);
        }
        sq[k] = ok[k] ? sumsq8<DT>(hp[k], 0.f) : 0.f;
        sq0[k] = sg[k] ? 0.f : sq[k];
        sq1[k] = sg[k] ? sq[k] : 0.f;
    }

    // ---- block totals: block k's in 16-lane row k (blocks past the row are 0)
    auto block_rows = [](const float (&v)[CPL]) -> float {
        float r[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) r[k] = k < CPL ? sum_row16(v[k]) : 0.f;
        return sum_pair32(sum_pair16(r[0], r[1]), sum_pair16(r[2], r[3]));
    };
    // ---- segment totals: (b0 + b1) + (b2 + b3) over the blocks of a segment
    float t0, t1 = 0.f;
    if constexpr (NSEG == 1) {
        const float b = block_rows(sq);
        const float p = sum_pair16(b, b); // rows: b0+b1, b0+b1, b2+b3, b2+b3
        t0 = lane_pick(sum_pair32(p, p), 0);
    } else if constexpr (SEGU) {
        // a block lies in one segment: split the block totals by rows
        const float b = block_rows(sq);
        const bool in1 = (t >> 4) >= KB; // this lane's 16-lane row holds block t >> 4
        const float p = sum_pair16(in1 ? 0.f : b, in1 ? b : 0.f); // rows: s0(01), s1(01), s0(23), s1(23)
        const float q = sum_pair32(p, p);                         // rows: s0, s1, s0, s1
        t0 = lane_pick(q, 0);
        t1 = lane_pick(q, 16);
    } else {
        const float b0 = block_rows(sq0), b1 = block_rows(sq1);
        const float p = sum_pair16(b0, b1);
        const float q = sum_pair32(p, p);
        t0 = lane_pick(q, 0);
        t1 = lane_pick(q, 16);
    }
    const float inv0 = rsqrt_nr(__builtin_fmaf(t0, a.inv_cols0, a.eps));
    const float inv1 = NSEG > 1 ? rsqrt_nr(__builtin_fmaf(t1, a.inv_cols1, a.eps)) : inv0;

    // ---- u = round_dt(h * inv * g), kept packed; optional copy.  The row
    //      maximum is taken of |h * inv * g| before the rounding and rounded
    //      once: rounding to nearest is monotone and symmetric, so that is
    //      the largest |u|.
    uint4 up[CPL];
    float am0 = 0.f, am1 = 0.f;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const float inv = sg[k] ? inv1 : inv0;
        float hf[8], wf[8];
        unpack8<DT>(hp[k], hf);
        unpack8<DT>(wv[k], wf);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            hf[i] *= GEMMA ? __builtin_fmaf(wf[i], inv, inv) : wf[i] * inv;
        up[k] = pack8<DT>(hf);
        uint8_t *normed = sg[k] ? a.seg[1].normed : a.seg[0].normed;
        const int32_t cols = sg[k] ? a.seg[1].cols : a.seg[0].cols;
        if (normed && ok[k]) stg_stream(normed + (row * cols + (int64_t)lc[k] * 8) * 2, up[k]);
        const float m = ok[k] ? amax8(hf) : 0.f;
        if (NSEG > 1 && sg[k]) am1 = __builtin_fmaxf(am1, m); else am0 = __builtin_fmaxf(am0, m);
    }
    if constexpr (NSEG == 1) {
        am0 = lane_pick(max_wave(am0), 0);
    } else {
        const float p = max_pair16(max_row16(am0), max_row16(am1)); // rows: m0(01), m1(01), m0(23), m1(23)
        const float q = max_pair32(p, p);                           // rows: m0, m1, m0, m1
        am0 = lane_pick(q, 0);
        am1 = lane_pick(q, 16);
    }
    const Fp32Scale sc0 = fp32_scale(round_dt<DT>(am0));
    const Fp32Scale sc1 = NSEG > 1 ? fp32_scale(round_dt<DT>(am1)) : sc0;

    // ---- quantise, store.  The fast/slow choice is made once for the row
    //      (both segments fast: the common case) rather than per chunk.
    uint2 qv[CPL];
    if (sc0.fast && sc1.fast) {
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            float u[8];
            unpack8<DT>(up[k], u);
            const Fp32Scale &sc = sg[k] ? sc1 : sc0;
#pragma unroll
            for (int i = 0; i < 8; ++i) u[i] = quotient_fast(u[i], sc);
            qv[k] = cvt8_e4m3(u);
        }
    } else {
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            float u[8];
            unpack8<DT>(up[k], u);
            qv[k] = fp32scale_codes8(u, sg[k] ? sc1 : sc0);
        }
    }
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const NormSegPlan &s = sg[k] ? a.seg[1] : a.seg[0];
        if (!ok[k]) continue;
        stg_stream(s.values + row * s.cols + (int64_t)lc[k] * 8, qv[k]);
        if (lc[k] == 0) reinterpret_cast<float *>(s.scales)[row] = sg[k] ? sc1.s : sc0.s;
    }
}

// ================================================================ launcher
template <int DT, int MODE, bool GEMMA, int CPL, bool F32Q>
static hipError_t go_norm(const NormArgs &a, int nseg, hipStream_t st)
{
    const int64_t blocks = (a.M + a.R - 1) / a.R;
    const dim3 grid((unsigned)blocks), block(a.NT * a.R);
    if (nseg == 1)
        hipLaunchKernelGGL((norm_quant_kernel<DT, MODE, GEMMA, CPL, 1, false, F32Q>), grid, block, 0, st, a);
    else if (a.C0 % 64 == 0)
        hipLaunchKernelGGL((norm_quant_kernel<DT, MODE, GEMMA, CPL, 2, true, F32Q>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((norm_quant_kernel<DT, MODE, GEMMA, CPL, 2, false, F32Q>), grid, block, 0, st, a);
    return hipGetLastError();
}

template <int DT, int MODE, bool GEMMA, bool F32Q>
static hipError_t go_norm_cpl(const NormArgs &a, int nseg, int CPL, hipStream_t st)
{
    switch (CPL) {
    case 1: return go_norm<DT, MODE, GEMMA, 1, F32Q>(a, nseg, st);
    case 2: return go_norm<DT, MODE, GEMMA, 2, F32Q>(a, nseg, st);
    case 3: return go_norm<DT, MODE, GEMMA, 3, F32Q>(a, nseg, st);
    default: return go_norm<DT, MODE, GEMMA, 4, F32Q>(a, nseg, st);
    }
}

template <int DT, int MODE, bool F32Q>
static hipError_t go_norm_kind(const NormArgs &a, bool gemma, int nseg, int CPL, hipStream_t st)
{
    return gemma ? go_norm_cpl<DT, MODE, true, F32Q>(a, nseg, CPL, st)
                 : go_norm_cpl<DT, MODE, false, F32Q>(a, nseg, CPL, st);
}

template <int DT, bool GEMMA, int CPL>
static hipError_t go_norm_pt_wave(const NormArgs &a, int nseg, hipStream_t st)
{
    const int64_t blocks = (a.M + a.R - 1) / a.R;
    const dim3 grid((unsigned)blocks), block(64 * a.R);
    // two segments with the boundary on a 64-chunk line: its slot, 1..CPL-1
    // (the first segment holds at least one block, the second at least one
    // chunk of the last slot)
    const int kb = (nseg == 2 && a.C0 % 64 == 0) ? a.C0 / 64 : 0;
    if (nseg == 1)
        hipLaunchKernelGGL((norm_pt_wave_kernel<DT, GEMMA, CPL, 1, 0>), grid, block, 0, st, a);
    else if (kb == 1)
        hipLaunchKernelGGL((norm_pt_wave_kernel<DT, GEMMA, CPL, 2, 1>), grid, block, 0, st, a);
    else if (kb == 2 && CPL > 2)
        hipLaunchKernelGGL((norm_pt_wave_kernel<DT, GEMMA, CPL, 2, (CPL > 2 ? 2 : 1)>), grid, block, 0, st, a);
    else if (kb == 3 && CPL > 3)
        hipLaunchKernelGGL((norm_pt_wave_kernel<DT, GEMMA, CPL, 2, (CPL > 3 ? 3 : 1)>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((norm_pt_wave_kernel<DT, GEMMA, CPL, 2, -1>), grid, block, 0, st, a);
    return hipGetLastError();
}

template <int DT>
static hipError_t go_norm_pt_wave_cpl(const NormArgs &a, bool gemma, int nseg, int CPL, hipStream_t st)
{
    switch (CPL) {
    case 2: return gemma ? go_norm_pt_wave<DT, true, 2>(a, nseg, st) : go_norm_pt_wave<DT, false, 2>(a, nseg, st);
    case 3: return gemma ? go_norm_pt_wave<DT, true, 3>(a, nseg, st) : go_norm_pt_wave<DT, false, 3>(a, nseg, st);
    default: return gemma ? go_norm_pt_wave<DT, true, 4>(a, nseg, st) : go_norm_pt_wave<DT, false, 4>(a, nseg, st);
    }
}

// The fp32-direct variant exists for the 1x128 and per-token modes only
// (the C ABI rejects it with MXFP8).
template <int DT>
static hipError_t go_norm_mode(const NormArgs &a, int mode, bool f32q, bool gemma, int nseg, int CPL,
                               hipStream_t st)
{
    switch (mode) {
    case kNone: return go_norm_kind<DT, kNone, false>(a, gemma, nseg, CPL, st);
    case kMX: return go_norm_kind<DT, kMX, false>(a, gemma, nseg, CPL, st);
    case kB128:
        return f32q ? go_norm_kind<DT, kB128, true>(a, gemma, nseg, CPL, st)
                    : go_norm_kind<DT, kB128, false>(a, gemma, nseg, CPL, st);
    default:
        return f32q ? go_norm_kind<DT, kPT, true>(a, gemma, nseg, CPL, st)
                    : go_norm_kind<DT, kPT, false>(a, gemma, nseg, CPL, st);
    }
}

// Compute units of the current device (the device the binding and the C
// callers launch on), read once per device: the row-shape rules count whole
// rows per CU, and a partitioned MI355X exposes fewer than 256 per device.
int64_t device_cus()
{
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices]; // 0: not read yet
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
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
    const int mode = p.quant ? p.mode : kNone;
    const bool copy = p.seg[0].normed != nullptr || (p.nseg > 1 && p.seg[1].normed != nullptr);
    const bool f32q = p.qin == 1;
    // per-token rows of up to 256 rows on one wavefront: when the
    // one-wavefront kernel serves the launch (not the fp32-direct form) and
    // the row has no residual or at most 128 chunks
    const bool small_one_wave = mode == kPT && !f32q && (p.nseg > 1 || p.res_in == nullptr || a.C <= 128);
    const RowShapeRt sh = norm_row_shape(a.C, p.M, mode == kPT, mode == kMX && copy, device_cus(), small_one_wave);
    a.NT = sh.NT;
    a.R = sh.R;
    a.WPR = sh.WPR;
    a.wpr_shift = sh.WPR == 2 ? 1 : 0; // R > 1 only with one or two wavefronts per row
    a.inv_cols0 = 1.0f / (float)p.seg[0].cols;
    a.inv_cols1 = 1.0f / (float)(p.nseg > 1 ? p.seg[1].cols : p.seg[0].cols);
    a.rcols0 = 1.0 / (double)p.seg[0].cols;
    a.rcols1 = 1.0 / (double)(p.nseg > 1 ? p.seg[1].cols : p.seg[0].cols);
    hipStream_t st = (hipStream_t)stream;
    const bool gemma = p.kind == 1;
    // per-token rows on one wavefront at two to four chunks per lane: the
    // kernel without LDS or barrier (the fp32-direct form keeps the general
    // kernel, whose fp64 reduction it has)
    const bool pt_wave = mode == kPT && !f32q && sh.WPR == 1 && sh.CPL >= 2;
    // one launch per row slice (a single one below ~2^31 / NT rows)
    const int64_t step = row_rows_per_launch(a.NT, a.R);
    NormArgs b = a;
    for (int64_t r0 = 0; r0 < p.M; r0 += step) {
        b.M = p.M - r0 < step ? p.M - r0 : step;
        for (int s = 0; s < 2; ++s) {
            const NormSegPlan &g = a.seg[s];
            b.seg[s].x = g.x + r0 * g.x_pitch;
            b.seg[s].values = offset_or_null(g.values, r0 * g.cols);
            b.seg[s].scales = offset_or_null(g.scales, r0 * scale_row_bytes(mode, g.cols));
            b.seg[s].normed = offset_or_null(g.normed, r0 * g.cols * 2);
        }
        b.res_in = a.res_in ? a.res_in + r0 * a.C0 * 16 : nullptr;
        b.res_out = a.res_out ? a.res_out + r0 * a.C0 * 16 : nullptr;
        hipError_t e;
        if (pt_wave)
            e = p.dtype == kFP16 ? go_norm_pt_wave_cpl<kFP16>(b, gemma, p.nseg, sh.CPL, st)
                                 : go_norm_pt_wave_cpl<kBF16>(b, gemma, p.nseg, sh.CPL, st);
        else
            e = p.dtype == kFP16 ? go_norm_mode<kFP16>(b, mode, f32q, gemma, p.nseg, sh.CPL, st)
                                 : go_norm_mode<kBF16>(b, mode, f32q, gemma, p.nseg, sh.CPL, st);
        if (e != hipSuccess) return (int)e;
    }
    return 0;
}

} // namespace afq
