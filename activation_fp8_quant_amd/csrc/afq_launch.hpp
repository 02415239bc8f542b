// afq_launch.hpp -- launch helpers shared by the kernel launchers: the
// launch-shape rules (afq_shape.hpp), the device half of the flat kernels'
// division of a chunk index by the chunks per row, and buffer offsets.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "afq_shape.hpp"

namespace afq {

// The flat kernels' division of a chunk index by C: the multiplier and
// shift come from divc() on the host (afq_shape.hpp).
__device__ __forceinline__ uint32_t div_c(uint32_t n, DivC d)
{
    return (uint32_t)(((uint64_t)__umulhi(n, d.m) + n) >> d.l);
}

// Compute units of the current device, read once per device (afq_norm.hip).
int64_t device_cus();

// Bytes of scales per row of `cols` elements in quant mode `mode`.
static inline int64_t scale_row_bytes(int mode, int32_t cols)
{
    return mode == kMX ? cols / 32 : mode == kB128 ? 4 * (cols / 128) : mode == kPT ? 4 : 0;
}

// p + off for a buffer that may be absent (nullptr stays nullptr).
template <typename T>
static inline T *offset_or_null(T *p, int64_t off) { return p ? p + off : nullptr; }

} // namespace afq
