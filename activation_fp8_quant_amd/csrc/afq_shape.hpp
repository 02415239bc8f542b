// afq_shape.hpp -- the launch-shape rules, host code only (plain C++, no
// HIP): the row shape of the row kernels, the rows per launch of the flat
// and row kernels, and the multiplier of the flat kernels' division by the
// chunks per row.  Kept apart from the device code so that the rules can be
// built and checked on a host compiler alone.
#pragma once

#include <stdint.h>

namespace afq {

// Division of a flat 32-bit chunk index by the chunks per row C, by a
// multiplier computed on the host (round-up method): with l = ceil(log2 C)
// and m = floor(2^32 (2^l - C) / C) + 1, n / C = (mulhi(n, m) + n) >> l
// for every n < 2^32 (the sum is taken in 64 bits).
struct DivC {
    uint32_t m;
    uint32_t l;
};
static inline DivC divc(uint32_t C)
{
    uint32_t l = 0;
    while ((1ull << l) < C) ++l;
    DivC d;
    d.m = (uint32_t)(((1ull << 32) * ((1ull << l) - C)) / C + 1);
    d.l = l;
    return d;
}

// Row shapes of the row kernels.  A row of C chunks runs on NT lanes (a
// whole number of wavefronts, at most 1024), CPL = ceil(C / NT) chunks per
// lane; rows of fewer than 256 lanes are packed several to a block.
struct RowShapeRt {
    int NT, CPL, R, WPR;
};
static inline int row_lanes(int C, int cpl)
{
    const int nt = (C + cpl - 1) / cpl;
    return (nt + 63) / 64 * 64;
}
static inline RowShapeRt shape_at(int C, int cpl)
{
    if ((C + cpl - 1) / cpl > 1024) cpl = (C + 1023) / 1024;
    RowShapeRt s;
    const int nt = row_lanes(C, cpl);
    s.NT = nt;
    s.CPL = (C + nt - 1) / nt;
    s.R = (nt < 256 && 256 % nt == 0) ? 256 / nt : 1;
    s.WPR = nt / 64;
    return s;
}

// Rows of a row kernel that one round of the GPU holds in the row shape
// shape_at(C, cpl): `cus` compute units (256 on a whole MI355X), `slots`
// wavefront slots per CU, whole rows per CU.
static inline int64_t rows_per_round(int C, int cpl, int slots, int64_t cus)
{
    return cus * (slots / shape_at(C, cpl).WPR);
}

// The standalone per-token quantiser's row shape (its kernel runs 8
// wavefronts per SIMD, 32 per CU, at one to four chunks per lane), chosen
// from a sweep (graph replay, rotated buffers, widths 2048 / 4096 / 6144 /
// 8192, 1 to 8192 rows, one to four chunks per lane): two chunks per lane,
// or three when a round at two chunks per lane cannot hold every row.  Over
// the sweep's 40 launches this takes 243 us, against 242 us for the best
// shape of each launch (at most 3.4 % slower in any one) and 248 us for
// one chunk per lane up to 256 rows at widths up to 4096 and wherever a
// round at one chunk per lane has rows to spare (the rule this replaced:
// up to 20 % slower than two, e.g. width 4096 at 512 rows 3.85 -> 3.21 us).
static inline RowShapeRt quant_row_shape(int C, int64_t M, int64_t cus)
{
    return shape_at(C, rows_per_round(C, 2, 32, cus) >= M ? 2 : 3);
}

// Rows of the norm kernel that one round of the GPU holds in the row shape
// shape_at(C, cpl) (the shape that runs: rows wider than 1024 chunks take
// more chunks per lane than asked): `cus` compute units (256 on a whole
// MI355X), each with 32 wavefront slots (8 per SIMD; 7 at four chunks per
// lane, where the kernel needs more than 64 VGPRs), whole rows per CU.
static inline int64_t norm_rows_per_round(int C, int cpl, int64_t cus)
{
    return rows_per_round(C, cpl, shape_at(C, cpl).CPL >= 4 ? 28 : 32, cus);
}

// Whether M rows in the row shape s fill at most 90 % of the wavefront
// slots of `cus` compute units (the norm kernel's 32 per CU, 28 at four
// chunks per lane).
static inline bool norm_round_has_room(const RowShapeRt &s, int64_t M, int64_t cus)
{
    return 10 * M * s.WPR <= 9 * cus * (s.CPL >= 4 ? 28 : 32);
}

// The norm kernel's row shape, chosen from sweeps (rotated buffers, widths
// 2048 to 8192, 1 to 4096 rows, one to four chunks per lane):
//  * per-token (two row reductions, each an LDS exchange across the row's
//    wavefronts): rows of 65 to 256 chunks on one wavefront (ceil(C / 64)
//    chunks per lane: the kernel that keeps a row in one wavefront, with no
//    LDS exchange) above 256 rows, and up to 256 rows when `small_one_wave`
//    says so (the launcher sets it when the one-wavefront kernel serves the
//    launch and the row has no residual or at most 128 chunks: the
//    two-segment 1536 + 512 launch at 8192 rows 12.3 -> 11.4 us, at 8 rows
//    2.79 -> 2.67 us, width 1024 with the residual at 8 rows 2.51 -> 2.43
//    us; with the residual at 192 to 256 chunks one wavefront's chain is
//    the longer, width 2048 at 192 rows 2.75 -> 3.38 us); other rows up to
//    256 rows on 256 to 512 lanes (two chunks per lane for rows wider than
//    2048; 7-23 % faster at widths 4096-8192, 8 rows), above 256 rows the
//    fewest chunks per lane from two up whose row is a whole divisor of a
//    CU's 32 wavefront slots (13-44 % faster than one chunk per lane from
//    512 rows: at width 6144, 4096 rows, 27.6 -> 15.4 us at three chunks
//    per lane);
//  * MXFP8 with the copy: the base shape (one chunk per lane; two or more
//    for rows wider than 1024 chunks) when one round of it holds every row
//    with at most 90 % of the GPU's wavefront slots filled; otherwise, up
//    to three rounds of rows at the base shape, the fewest chunks per lane
//    whose round does, shapes with no idle chunk slot (NT * CPL = C) first,
//    then any.  A round that fills every slot is slow: width 2048 at 2048
//    rows 8.64 us at one chunk per lane, 7.83 at two; width 4096 at 1024
//    rows 8.60 -> 7.83; width 8192 at 1024 rows 14.81 us at two, 14.15 at
//    four.  Rounds left partly empty cost little (width 6144 at 512 rows,
//    three quarters of the slots: one chunk per lane is the fastest).  Over
//    a sweep of widths 2048 / 4096 / 6144 / 7168 / 8192 at 256 to 4096 rows
//    the rule is at most 2.5 % off the best shape of any launch (the rule it
//    replaced, which went to more chunks per lane only above one round:
//    10.5 %), and at most 7.5 % at widths 3072 / 5120 / 10240 / 12288 /
//    16384, which it was not fitted on.  At decode sizes (8 to 192 rows)
//    one chunk per lane is the fastest by 0.1-0.7 us.  Above three rounds
//    one chunk per lane (the launch is bandwidth-bound, and longer lane
//    work only costs);
//  * everything else (1x128, copy-only, MXFP8 without the copy): one chunk
//    per lane, which the same sweep found best for 1x128 at every size.
static inline RowShapeRt norm_row_shape(int C, int64_t M, bool per_token, bool mx_copy, int64_t cus,
                                        bool small_one_wave)
{
    int cpl = 1;
    if (per_token) {
        if (C > 64 && C <= 256 && (M > 256 || small_one_wave)) {
            cpl = (C + 63) / 64;
        } else if (M <= 256) {
            cpl = C > 256 ? 2 : 1;
        } else {
            cpl = 2;
            for (int c = 2; c <= 4; ++c)
                if (32 % shape_at(C, c).WPR == 0) {
                    cpl = c;
                    break;
                }
        }
    } else if (mx_copy && M <= 3 * norm_rows_per_round(C, 1, cus) &&
               !(M <= norm_rows_per_round(C, 1, cus) && norm_round_has_room(shape_at(C, 1), M, cus))) {
        for (int pass = 0; pass < 2; ++pass)
            for (int c = 1; c <= 4; ++c) {
                const RowShapeRt s = shape_at(C, c);
                if (pass == 0 && s.NT * s.CPL != C) continue;
                if (norm_rows_per_round(C, c, cus) >= M && norm_round_has_room(s, M, cus)) return s;
            }
    }
    return shape_at(C, cpl);
}

// Rows per launch of the flat kernels: the flat chunk index stays below
// 2^31 (larger M is covered by several launches over row slices).
static inline int64_t flat_rows_per_launch(int32_t C) { return ((int64_t)1 << 31) / C; }

// Rows per launch of the row kernels (NT lanes per row, R rows per block):
// a launch stays below 2^31 work-items (a dispatch's grid size is a 32-bit
// count of work-items), a whole number of blocks; larger M is covered by
// several launches over row slices.
static inline int64_t row_rows_per_launch(int NT, int R)
{
    return (((int64_t)1 << 31) / NT) / R * R;
}

} // namespace afq
