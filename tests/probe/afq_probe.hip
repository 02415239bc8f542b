// afq_probe.hip -- test-only probe kernels (not part of libafq.so).
//
// Each kernel applies one of the library's device primitives (from
// afq_device.hpp, the header the product kernels use) element-wise, so that
// the tests can compare the primitive with IEEE arithmetic and with the
// oracle's roundings on the host, over exhaustive input sets:
//   afqp_scale     fp32_scale(amax): the stored scale s, the reciprocal r
//                  and the fast-path flag
//   afqp_quotient  the quotient a quantiser forms for u under amax's scale
//                  (quotient_fast on the fast path, IEEE division otherwise)
//   afqp_cvt8_e4m3 cvt8_e4m3 on 8 values at a time (v_cvt_pk_fp8_f32, both
//                  word halves), no clamp
//   afqp_e4m3_range the same on every fp32 bit pattern base .. base + n - 1,
//                  generated in the kernel
//   afqp_pack_bf16 pack8<bf16> on 8 values at a time (v_cvt_pk_bf16_f32)
//   afqp_inv_rms   inv_rms_f32q(ss, cols, RN64(1/cols), eps): the
//                  fp32-direct inverse RMS, and which path gave it
//   afqp_issue     an issue-rate kernel: every lane runs 8 independent
//                  chains of one instruction kind (fp32 FMA, exp2, rcp,
//                  bf16 and e4m3 pair conversions, a three-input bitwise
//                  op, integer add, fp64 FMA, bf16 dot2) over registers
//                  only, for the caller to time
//
// Every kernel is guarded by its element count; the host wrappers reject
// counts above 2^31, counts that are not a multiple of 8 where 8 values go
// to one lane, and buffers not 16-byte aligned, before launching.
#include "afq_device.hpp"

using namespace afq;

namespace {

constexpr int kBlock = 256;

__global__ void __launch_bounds__(kBlock) k_scale(const float *amax, float *s, float *r, uint8_t *fast, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= n) return;
    const Fp32Scale sc = fp32_scale(amax[i]);
    s[i] = sc.s;
    r[i] = sc.r;
    fast[i] = sc.fast ? 1 : 0;
}

__global__ void __launch_bounds__(kBlock) k_quotient(const float *u, const float *amax, float *q, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= n) return;
    const Fp32Scale sc = fp32_scale(amax[i]);
    q[i] = sc.fast ? quotient_fast(u[i], sc) : u[i] / sc.s;
}

__global__ void __launch_bounds__(kBlock) k_cvt8(const float *v, uint8_t *codes, int64_t n8)
{
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= n8) return;
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = v[i * 8 + k];
    *reinterpret_cast<uint2 *>(codes + i * 8) = cvt8_e4m3(x);
}

__global__ void __launch_bounds__(kBlock) k_e4m3_range(uint32_t base, uint8_t *codes, int64_t n8)
{
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= n8) return;
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = __uint_as_float(base + (uint32_t)(i * 8 + k));
    *reinterpret_cast<uint2 *>(codes + i * 8) = cvt8_e4m3(x);
}

__global__ void __launch_bounds__(kBlock) k_pack_bf16(const float *v, uint16_t *out, int64_t n8)
{
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= n8) return;
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = v[i * 8 + k];
    *reinterpret_cast<uint4 *>(out + i * 8) = pack8<kBF16>(x);
}

__global__ void __launch_bounds__(kBlock) k_inv_rms(const double *ss, int32_t cols, double rcols, float eps,
                                                    float *inv, uint8_t *fast, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= n) return;
    bool f = false;
    inv[i] = inv_rms_f32q(ss[i], cols, rcols, eps, &f);
    fast[i] = f ? 1 : 0;
}

// threads needed for n work items, or -1 when n is out of range
int64_t grid_for(int64_t n)
{
    if (n < 0 || n > ((int64_t)1 << 31)) return -1;
    return (n + kBlock - 1) / kBlock;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Issue-rate kernel OP: 8 independent chains a lane of one instruction kind
// for n iterations, on registers only (the empty asm statements keep every
// chain live without touching memory); one word a lane is stored.
template <int OP>
__global__ void __launch_bounds__(kBlock) k_issue(uint32_t *out, int32_t n, float seed)
{
    const uint32_t gid = blockIdx.x * kBlock + threadIdx.x;
    float x[8];
    uint32_t u[8];
    double d[4];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        x[j] = 0.25f + seed * (float)((gid * 8 + j) & 1023);
        u[j] = __float_as_uint(x[j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) d[j] = (double)x[j];
    for (int32_t i = 0; i < n; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if constexpr (OP == 0) x[j] = __builtin_fmaf(x[j], 1.0000001f, 0.5f);
            else if constexpr (OP == 1) x[j] = __builtin_amdgcn_exp2f(x[j]);
            else if constexpr (OP == 2) x[j] = __builtin_amdgcn_rcpf(x[j]);
            else if constexpr (OP == 3) u[j] = pack_bf16x2(__uint_as_float(u[j]), x[j]);
            else if constexpr (OP == 4) u[j] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(u[j]), x[j], (int)u[j], false);
            else if constexpr (OP == 5) u[j] = (u[j] & 0xFFFF0001u) ^ 0x3F800000u;
            else if constexpr (OP == 6) u[j] = u[j] + 0x9E3779B9u;
            else if constexpr (OP == 7) { if (j < 4) d[j] = __builtin_fma(d[j], 1.0000001, 0.5); }
            else x[j] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u[j]), __builtin_bit_cast(bf16x2, u[j]), x[j], false);
        }
        asm volatile("" : "+v"(u[0]), "+v"(u[1]), "+v"(u[2]), "+v"(u[3]), "+v"(u[4]), "+v"(u[5]), "+v"(u[6]), "+v"(u[7]));
        asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]));
        asm volatile("" : "+v"(d[0]), "+v"(d[1]), "+v"(d[2]), "+v"(d[3]));
    }
    uint32_t r = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) r ^= u[j] ^ __float_as_uint(x[j]);
#pragma unroll
    for (int j = 0; j < 4; ++j) r ^= (uint32_t)__double_as_longlong(d[j]);
    out[gid] = r;
}

} // namespace

extern "C" {

// All pointers are device pointers; n counts elements.  Returns 0, -1 for a
// rejected count, or the HIP error of the launch.
int afqp_scale(const float *amax, float *s, float *r, uint8_t *fast, int64_t n, void *stream)
{
    const int64_t g = grid_for(n);
    if (g < 0) return -1;
    if (g == 0) return 0;
    hipLaunchKernelGGL(k_scale, dim3((unsigned)g), dim3(kBlock), 0, (hipStream_t)stream, amax, s, r, fast, n);
    return (int)hipGetLastError();
}

int afqp_quotient(const float *u, const float *amax, float *q, int64_t n, void *stream)
{
    const int64_t g = grid_for(n);
    if (g < 0) return -1;
    if (g == 0) return 0;
    hipLaunchKernelGGL(k_quotient, dim3((unsigned)g), dim3(kBlock), 0, (hipStream_t)stream, u, amax, q, n);
    return (int)hipGetLastError();
}

// n must be a multiple of 8; codes holds n bytes
int afqp_cvt8_e4m3(const float *v, uint8_t *codes, int64_t n, void *stream)
{
    if (n % 8 || !aligned16(v) || !aligned16(codes)) return -1;
    const int64_t g = grid_for(n / 8);
    if (g < 0) return -1;
    if (g == 0) return 0;
    hipLaunchKernelGGL(k_cvt8, dim3((unsigned)g), dim3(kBlock), 0, (hipStream_t)stream, v, codes, n / 8);
    return (int)hipGetLastError();
}

// codes[i] = e4m3 of the fp32 with bit pattern base + i, i < n; n a multiple
// of 8 and base + n <= 2^32
int afqp_e4m3_range(uint32_t base, uint8_t *codes, int64_t n, void *stream)
{
    if (n % 8 || (int64_t)base + n > ((int64_t)1 << 32) || !aligned16(codes)) return -1;
    const int64_t g = grid_for(n / 8);
    if (g < 0) return -1;
    if (g == 0) return 0;
    hipLaunchKernelGGL(k_e4m3_range, dim3((unsigned)g), dim3(kBlock), 0, (hipStream_t)stream, base, codes, n / 8);
    return (int)hipGetLastError();
}

// n must be a multiple of 8; out holds n bf16 bit patterns
// inv[i] = inv_rms_f32q(ss[i], cols, RN64(1/cols), eps); fast[i] = 1 where
// the fast path gave it.  cols must be positive.
int afqp_inv_rms(const double *ss, int32_t cols, float eps, float *inv, uint8_t *fast, int64_t n, void *stream)
{
    const int64_t g = grid_for(n);
    if (g < 0 || cols <= 0) return -1;
    if (g == 0) return 0;
    hipLaunchKernelGGL(k_inv_rms, dim3((unsigned)g), dim3(kBlock), 0, (hipStream_t)stream, ss, cols,
                       1.0 / (double)cols, eps, inv, fast, n);
    return (int)hipGetLastError();
}

int afqp_pack_bf16(const float *v, uint16_t *out, int64_t n, void *stream)
{
    if (n % 8 || !aligned16(v) || !aligned16(out)) return -1;
    const int64_t g = grid_for(n / 8);
    if (g < 0) return -1;
    if (g == 0) return 0;
    hipLaunchKernelGGL(k_pack_bf16, dim3((unsigned)g), dim3(kBlock), 0, (hipStream_t)stream, v, out, n / 8);
    return (int)hipGetLastError();
}

// The issue-rate kernel of instruction kind op (0 fp32 FMA, 1 exp2, 2 rcp,
// 3 bf16 pair conversion, 4 e4m3 pair conversion, 5 three-input bitwise op,
// 6 integer add, 7 fp64 FMA (4 chains a lane), 8 bf16 dot2) on blocks
// blocks of 256 lanes, n iterations; out holds blocks * 256 words.
int afqp_issue(int op, uint32_t *out, int64_t blocks, int32_t n, void *stream)
{
    if (op < 0 || op > 8 || blocks <= 0 || blocks > (1 << 20) || n < 0 || n > (1 << 20) || !out) return -1;
    const dim3 g((unsigned)blocks), b(kBlock);
    hipStream_t st = (hipStream_t)stream;
    switch (op) {
    case 0: hipLaunchKernelGGL(k_issue<0>, g, b, 0, st, out, n, 1e-3f); break;
    case 1: hipLaunchKernelGGL(k_issue<1>, g, b, 0, st, out, n, 1e-3f); break;
    case 2: hipLaunchKernelGGL(k_issue<2>, g, b, 0, st, out, n, 1e-3f); break;
    case 3: hipLaunchKernelGGL(k_issue<3>, g, b, 0, st, out, n, 1e-3f); break;
    case 4: hipLaunchKernelGGL(k_issue<4>, g, b, 0, st, out, n, 1e-3f); break;
    case 5: hipLaunchKernelGGL(k_issue<5>, g, b, 0, st, out, n, 1e-3f); break;
    case 6: hipLaunchKernelGGL(k_issue<6>, g, b, 0, st, out, n, 1e-3f); break;
    case 7: hipLaunchKernelGGL(k_issue<7>, g, b, 0, st, out, n, 1e-3f); break;
    default: hipLaunchKernelGGL(k_issue<8>, g, b, 0, st, out, n, 1e-3f); break;
    }
    return (int)hipGetLastError();
}

} // extern "C"
