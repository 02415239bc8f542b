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
//   afqp_rows_pattern  the two-segment per-token norm's memory traffic
//                  without its arithmetic: one wavefront a row, four 16-B
//                  chunk loads a lane from a pitched row, a wavefront-wide
//                  sum that every store waits for, 8-B stores to two dense
//                  code arrays split at chunk C0 and a 4-B value a row and
//                  segment
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

// The two-segment per-token norm's access pattern (rows of C <= 256 chunks,
// one wavefront each, four rows a 256-lane block): the same loads and
// stores, with a wavefront-wide integer sum in place of the arithmetic.
__global__ void __launch_bounds__(kBlock) k_rows_pattern(const uint8_t *x, int64_t pitch, uint8_t *q0, uint8_t *q1,
                                                         float *s0, float *s1, int64_t M, int32_t C0, int32_t C)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return; // wavefront-uniform
    uint4 v[4];
    uint32_t acc = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int c = lane + 64 * k;
        v[k] = c < C ? ldg_stream(x + row * pitch + (int64_t)c * 16) : make_uint4(0, 0, 0, 0);
        acc += v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
    for (int off = 32; off > 0; off >>= 1) acc += (uint32_t)__shfl_xor((int)acc, off);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int c = lane + 64 * k;
        if (c >= C) continue;
        const uint2 o = make_uint2(v[k].x ^ acc, v[k].z ^ acc);
        if (c < C0) stg_stream(q0 + (row * C0 + c) * 8, o);
        else stg_stream(q1 + (row * (C - C0) + (c - C0)) * 8, o);
    }
    if (lane == 0) {
        s0[row] = __uint_as_float(acc & 0x3FFFFFFFu);
        s1[row] = __uint_as_float(acc & 0x3FFFFFFFu);
    }
}

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

// The two-segment per-token norm's memory pattern on M rows of C chunks
// (0 < C0 <= C <= 256) read from x with a pitch of `pitch` bytes (a multiple
// of 16); q0 holds M * C0 * 8 bytes, q1 M * (C - C0) * 8, s0 and s1 M floats.
int afqp_rows_pattern(const uint8_t *x, int64_t pitch, uint8_t *q0, uint8_t *q1, float *s0, float *s1, int64_t M,
                      int32_t C0, int32_t C, void *stream)
{
    if (M < 0 || C < 1 || C > 256 || C0 < 1 || C0 > C || pitch < (int64_t)C * 16 || pitch % 16 || !aligned16(x) ||
        !q0 || (C0 < C && !q1) || !s0 || !s1)
        return -1;
    const int64_t g = (M + 3) / 4;
    if (g > ((int64_t)1 << 31) - 1) return -1;
    if (g == 0) return 0;
    hipLaunchKernelGGL(k_rows_pattern, dim3((unsigned)g), dim3(kBlock), 0, (hipStream_t)stream, x, pitch, q0, q1, s0,
                       s1, M, C0, C);
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
