// afq_internal.h -- plain structs passed from the validated C ABI to the
// kernel launchers.  No HIP types: the ABI translation unit is plain C++.
#pragma once

#include <stdint.h>

namespace afq {

struct NormSegPlan {
    const uint8_t *x;      // segment base
    int64_t x_pitch;       // bytes between rows
    const uint8_t *w;      // weight
    uint8_t *values;       // codes [M, cols]
    uint8_t *scales;       // scales, row-major
    uint8_t *normed;       // optional copy [M, cols] in dtype, or nullptr
    int32_t cols;          // elements
    int32_t chunks;        // cols / 8
};

struct NormPlan {
    NormSegPlan seg[2];
    const uint8_t *res_in;  // [M, cols0] or nullptr
    uint8_t *res_out;       // [M, cols0] or nullptr
    int64_t M;
    float eps;
    int32_t nseg;
    int32_t kind;           // 0 standard, 1 Gemma
    int32_t dtype;          // 0 bf16, 1 fp16
    int32_t mode;           // 0 MX, 1 B128, 2 PT
    int32_t qin;            // 0 dtype-rounded row, 1 fp32 normed value (B128 / PT)
    int32_t quant;          // 1 quantise; 0 copy only (values, scales nullptr)
};

struct ActPlan {
    const uint8_t *gu;      // [M, 2I] bf16
    int64_t gu_pitch;       // bytes
    uint8_t *values;        // [M, I]
    uint8_t *scales;
    uint8_t *act;           // optional bf16 [M, I]
    int64_t M;
    int32_t I;
    int32_t mode;           // also the activation's rounding when copy only
    int32_t qin;            // 0 mode default, 2 bf16-rounded activation (MX)
    int32_t quant;          // 1 quantise; 0 copy only (values, scales nullptr)
    int32_t act_kind;       // 0 SiLU-and-mul, 1 clamped SwiGLU (MX only)
    float alpha, beta, limit; // clamped SwiGLU parameters
};

struct QuantPlan {
    const uint8_t *x;
    int64_t x_pitch;        // bytes
    uint8_t *values;
    uint8_t *scales;
    int64_t M;
    int32_t cols;
    int32_t dtype;          // 0 bf16, 1 fp16, 2 fp32
    int32_t mode;
};

// Enqueue on `stream` (a hipStream_t).  Return 0 or the hipError_t code.
int launch_norm(const NormPlan &p, void *stream);
int launch_act(const ActPlan &p, void *stream);
int launch_quant(const QuantPlan &p, void *stream);

} // namespace afq
