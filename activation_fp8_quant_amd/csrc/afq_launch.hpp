// afq_launch.hpp -- launch-shape helpers shared by the kernel launchers:
// the row shape of the row kernels, the rows per launch of the flat
// kernels, and the flat kernels' division of a chunk index by the chunks
// per row (multiplier made on the host, applied on the device).
#pragma once

#include <hip/hip_runtime.h>
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
__device__ __forceinline__ uint32_t div_c(uint32_t n, DivC d)
{
    return (uint32_t)(((uint64_t)__umulhi(n, d.m) + n) >> d.l);
}

// Row shape for a row of C chunks: one chunk per lane (as many lanes as
// chunks, up to 1024), so that a row's loads are all in flight at once and
// the per-lane work is shortest.  Per-token rows of a bandwidth-bound
// launch (M > 1024) take two chunks per lane instead: they need two row
// reductions (sum of squares, then amax), each an LDS exchange across the
// row's wavefronts, and halving the wavefronts per row pays for the longer
// lane work (measured at M = 8192, H = 2048..8192: per-token 4-14% faster
// at two chunks; MXFP8 1-3% and 1x128 within 1% faster at one).  NT is a
// whole number of wavefronts; rows of fewer than 256 lanes are packed
// several to a block.
struct RowShapeRt {
    int NT, CPL, R, WPR;
};
static inline RowShapeRt row_shape(int C, int64_t M, bool per_token)
{
    RowShapeRt s;
    int cpl = (per_token && M > 1024) ? 2 : 1;
    if ((C + cpl - 1) / cpl > 1024) cpl = (C + 1023) / 1024;
    int nt = (C + cpl - 1) / cpl;
    nt = (nt + 63) / 64 * 64;
    s.NT = nt;
    s.CPL = (C + nt - 1) / nt;
    s.R = (nt < 256 && 256 % nt == 0) ? 256 / nt : 1;
    s.WPR = nt / 64;
    return s;
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

// Bytes of scales per row of `cols` elements in quant mode `mode`.
static inline int64_t scale_row_bytes(int mode, int32_t cols)
{
    return mode == kMX ? cols / 32 : mode == kB128 ? 4 * (cols / 128) : mode == kPT ? 4 : 0;
}

// p + off for a buffer that may be absent (nullptr stays nullptr).
template <typename T>
static inline T *offset_or_null(T *p, int64_t off) { return p ? p + off : nullptr; }

} // namespace afq
