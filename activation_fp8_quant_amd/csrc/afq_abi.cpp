// afq_abi.cpp -- the exported C ABI: argument validation and dispatch.
//
// Everything here runs on the host before any enqueue, touches no device
// memory and makes no HIP call, so a rejected call has written nothing.
// The launchers (afq_norm.hip, afq_act.hip, afq_quant.hip) are the only
// code that talks to HIP.

#include "afq.h"
#include "afq_internal.h"

#include <cmath>
#include <cstdint>

namespace {

thread_local int g_last_hip_error = 0;

struct Span {
    uintptr_t lo = 0, hi = 0; // [lo, hi), empty when lo == hi
    bool wraps = false;       // the buffer would run past the end of the address space
};

// Byte span of a [rows, cols] array of `elt`-byte elements, row pitch in
// bytes (rows, cols, elt, pitch >= 0).  Computed in unsigned 64-bit with
// overflow checks: an extent that does not fit marks the span as wrapping.
Span span_of(const void *p, int64_t rows, int64_t cols, int64_t elt, int64_t pitch)
{
    Span s;
    if (!p || rows <= 0 || cols <= 0) return s;
    uint64_t body, last, len, end;
    if (__builtin_mul_overflow((uint64_t)(rows - 1), (uint64_t)pitch, &body) ||
        __builtin_mul_overflow((uint64_t)cols, (uint64_t)elt, &last) ||
        __builtin_add_overflow(body, last, &len) ||
        __builtin_add_overflow((uint64_t)(uintptr_t)p, len, &end)) {
        s.wraps = true;
        return s;
    }
    s.lo = (uintptr_t)p;
    s.hi = (uintptr_t)end;
    return s;
}

bool any_wraps(const Span *a, int n)
{
    for (int i = 0; i < n; ++i)
        if (a[i].wraps) return true;
    return false;
}

// Row count and row stride bounds shared by every entry point.
bool rows_ok(int64_t M) { return M >= 0 && M <= AFQ_MAX_ROWS; }
bool stride_ok(int64_t stride, int64_t min) { return stride >= min && stride <= AFQ_MAX_ROW_STRIDE; }

bool overlap(const Span &a, const Span &b)
{
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool valid_qin(int q) { return q == AFQ_QIN_DEFAULT || q == AFQ_QIN_FP32 || q == AFQ_QIN_BF16; }
int group_of(int mode) { return mode == AFQ_MXFP8 ? 32 : mode == AFQ_BLOCK128 ? 128 : 8; }

int64_t scale_cols(int mode, int64_t cols)
{
    return mode == AFQ_MXFP8 ? cols / 32 : mode == AFQ_BLOCK128 ? cols / 128 : 1;
}
int64_t scale_elt(int mode) { return mode == AFQ_MXFP8 ? 1 : 4; }

bool valid_mode(int m) { return m == AFQ_MXFP8 || m == AFQ_BLOCK128 || m == AFQ_PER_TOKEN; }

// Row width rules shared by every entry point (a copy-only launch has no
// quantisation groups: its widths need only be whole 16-byte chunks).
bool width_ok(int64_t cols, int mode, bool quant = true)
{
    return cols > 0 && cols <= AFQ_MAX_COLS && cols % 8 == 0 && (!quant || cols % group_of(mode) == 0);
}

// Outputs must not overlap each other or any input.
bool any_overlap(const Span *outs, int nout, const Span *ins, int nin)
{
    for (int i = 0; i < nout; ++i) {
        for (int j = i + 1; j < nout; ++j)
            if (overlap(outs[i], outs[j])) return true;
        for (int j = 0; j < nin; ++j)
            if (overlap(outs[i], ins[j])) return true;
    }
    return false;
}

int launched(int hip_err)
{
    if (hip_err != 0) {
        g_last_hip_error = hip_err;
        return AFQ_ERR_LAUNCH;
    }
    return AFQ_OK;
}

// Checks and dispatch shared by the SiLU-and-mul and clamped-SwiGLU entry
// points (act: 0 SiLU-and-mul, 1 clamped SwiGLU with its parameters in sw).
int act_common(const afq_act_desc *d, int act, const afq_swiglu_desc *sw, void *stream)
{
    if (!valid_qin(d->quant_input)) return AFQ_ERR_ARG;
    if (!valid_mode(d->mode)) return AFQ_ERR_ARG;
    if (d->mode == AFQ_PER_TOKEN) return AFQ_ERR_UNSUPPORTED;
    if (d->quant_input == AFQ_QIN_FP32) return AFQ_ERR_UNSUPPORTED;
    if (d->quant_input == AFQ_QIN_BF16 && d->mode != AFQ_MXFP8) return AFQ_ERR_UNSUPPORTED;
    // copy only (the SiLU-and-mul of the unfused chain): no codes or scales
    const bool quant = d->out.values || d->out.scales;
    if (!quant && d->quant_input != AFQ_QIN_DEFAULT) return AFQ_ERR_UNSUPPORTED;
    if (!rows_ok(d->M)) return AFQ_ERR_SHAPE;
    if (!width_ok(d->I, d->mode, quant)) return AFQ_ERR_SHAPE;
    if (!stride_ok(d->gate_up_row_stride, 2 * d->I)) return AFQ_ERR_SHAPE;
    if (d->M == 0) return AFQ_OK;
    if (!d->gate_up) return AFQ_ERR_NULL;
    if (quant ? (!d->out.values || !d->out.scales) : !d->out.normed) return AFQ_ERR_NULL;
    if (!aligned(d->gate_up, 16) || (d->gate_up_row_stride * 2) % 16 != 0) return AFQ_ERR_ALIGN;
    if (quant && (!aligned(d->out.values, 16) || !aligned(d->out.scales, 4))) return AFQ_ERR_ALIGN;
    if (d->out.normed && !aligned(d->out.normed, 16)) return AFQ_ERR_ALIGN;

    const int64_t M = d->M, I = d->I;
    Span outs[3] = {
        span_of(d->out.values, M, I, 1, I),
        span_of(d->out.scales, M, scale_cols(d->mode, I), scale_elt(d->mode),
                scale_cols(d->mode, I) * scale_elt(d->mode)),
        span_of(d->out.normed, M, I, 2, I * 2),
    };
    Span ins[1] = {span_of(d->gate_up, M, 2 * I, 2, d->gate_up_row_stride * 2)};
    if (any_wraps(outs, 3) || any_wraps(ins, 1)) return AFQ_ERR_SHAPE;
    if (any_overlap(outs, 3, ins, 1)) return AFQ_ERR_ALIAS;

    afq::ActPlan p{};
    p.gu = (const uint8_t *)d->gate_up;
    p.gu_pitch = d->gate_up_row_stride * 2;
    p.values = (uint8_t *)d->out.values;
    p.scales = (uint8_t *)d->out.scales;
    p.act = (uint8_t *)d->out.normed;
    p.M = M;
    p.I = (int32_t)I;
    p.mode = d->mode;
    p.qin = d->quant_input;
    p.quant = quant ? 1 : 0;
    p.act_kind = act;
    p.alpha = sw ? sw->alpha : 1.0f;
    p.beta = sw ? sw->beta : 0.0f;
    p.limit = sw ? sw->limit : INFINITY;
    return launched(afq::launch_act(p, stream));
}

} // namespace

extern "C" {

int afq_abi_version(void) { return AFQ_ABI_VERSION; }

int afq_last_hip_error(void) { return g_last_hip_error; }

const char *afq_status_string(int status)
{
    switch (status) {
    case AFQ_OK: return "ok";
    case AFQ_ERR_NULL: return "a required pointer is NULL";
    case AFQ_ERR_SHAPE: return "invalid shape (M, width, group multiple, row stride, buffer extent or segment count)";
    case AFQ_ERR_ALIGN: return "pointer or row pitch not aligned (16 bytes; scales 4 bytes)";
    case AFQ_ERR_DTYPE: return "dtype not supported by this entry point";
    case AFQ_ERR_ALIAS: return "an output overlaps another output or an input";
    case AFQ_ERR_UNSUPPORTED: return "quantisation mode, norm kind or quant_input not supported by this entry point";
    case AFQ_ERR_ARG: return "invalid argument (eps or an enum value)";
    case AFQ_ERR_LAUNCH: return "HIP kernel launch failed (see afq_last_hip_error)";
    default: return "unknown status";
    }
}

int fused_add_rmsnorm_quant(const afq_norm_desc *d, void *stream)
{
    if (!d) return AFQ_ERR_NULL;
    if (!valid_qin(d->quant_input)) return AFQ_ERR_ARG;
    if (!valid_mode(d->mode)) return AFQ_ERR_ARG;
    if (d->kind != AFQ_RMSNORM_STANDARD && d->kind != AFQ_RMSNORM_GEMMA) return AFQ_ERR_ARG;
    if (d->dtype != AFQ_BF16 && d->dtype != AFQ_FP16) {
        return (d->dtype == AFQ_FP32) ? AFQ_ERR_DTYPE : AFQ_ERR_ARG;
    }
    if (!(std::isfinite(d->eps) && d->eps >= 0.0f)) return AFQ_ERR_ARG;
    if (d->quant_input == AFQ_QIN_BF16) return AFQ_ERR_UNSUPPORTED;
    if (d->quant_input == AFQ_QIN_FP32 && d->mode == AFQ_MXFP8) return AFQ_ERR_UNSUPPORTED;
    if (d->nseg != 1 && d->nseg != 2) return AFQ_ERR_SHAPE;
    // copy only (the norm of the unfused chain): no codes or scales anywhere
    bool quant = false;
    for (int s = 0; s < d->nseg; ++s)
        quant = quant || d->seg[s].out.values || d->seg[s].out.scales;
    if (!quant && d->quant_input != AFQ_QIN_DEFAULT) return AFQ_ERR_UNSUPPORTED;
    if (!rows_ok(d->M)) return AFQ_ERR_SHAPE;
    const bool has_res = d->residual_in != nullptr || d->residual_out != nullptr;
    if (has_res && d->nseg != 1) return AFQ_ERR_SHAPE;
    for (int s = 0; s < d->nseg; ++s) {
        const afq_norm_seg &g = d->seg[s];
        if (!width_ok(g.cols, d->mode, quant)) return AFQ_ERR_SHAPE;
        if (!stride_ok(g.x_row_stride, g.cols)) return AFQ_ERR_SHAPE;
    }
    if (d->nseg == 2 && (d->seg[0].cols + d->seg[1].cols) > AFQ_MAX_COLS) return AFQ_ERR_SHAPE;
    if (d->M == 0) return AFQ_OK;

    if (has_res && (!d->residual_in || !d->residual_out)) return AFQ_ERR_NULL;
    for (int s = 0; s < d->nseg; ++s) {
        const afq_norm_seg &g = d->seg[s];
        if (!g.x || !g.weight) return AFQ_ERR_NULL;
        if (quant ? (!g.out.values || !g.out.scales) : !g.out.normed) return AFQ_ERR_NULL;
    }

    const int64_t elt = 2;
    for (int s = 0; s < d->nseg; ++s) {
        const afq_norm_seg &g = d->seg[s];
        if (!aligned(g.x, 16) || (g.x_row_stride * elt) % 16 != 0) return AFQ_ERR_ALIGN;
        if (!aligned(g.weight, 16)) return AFQ_ERR_ALIGN;
        if (quant && (!aligned(g.out.values, 16) || !aligned(g.out.scales, 4))) return AFQ_ERR_ALIGN;
        if (g.out.normed && !aligned(g.out.normed, 16)) return AFQ_ERR_ALIGN;
    }
    if (has_res && (!aligned(d->residual_in, 16) || !aligned(d->residual_out, 16)))
        return AFQ_ERR_ALIGN;

    // aliasing: outputs vs outputs and vs inputs; residual_out may be residual_in
    Span outs[7], ins[5];
    int no = 0, ni = 0;
    const int64_t M = d->M;
    for (int s = 0; s < d->nseg; ++s) {
        const afq_norm_seg &g = d->seg[s];
        outs[no++] = span_of(g.out.values, M, g.cols, 1, g.cols);
        outs[no++] = span_of(g.out.scales, M, scale_cols(d->mode, g.cols), scale_elt(d->mode),
                             scale_cols(d->mode, g.cols) * scale_elt(d->mode));
        outs[no++] = span_of(g.out.normed, M, g.cols, elt, g.cols * elt);
        ins[ni++] = span_of(g.x, M, g.cols, elt, g.x_row_stride * elt);
        ins[ni++] = span_of(g.weight, 1, g.cols, elt, g.cols * elt);
    }
    if (any_wraps(outs, no) || any_wraps(ins, ni)) return AFQ_ERR_SHAPE;
    if (has_res) {
        const int64_t c = d->seg[0].cols;
        const Span rout = span_of(d->residual_out, M, c, elt, c * elt);
        const Span rin = span_of(d->residual_in, M, c, elt, c * elt);
        if (rout.wraps || rin.wraps) return AFQ_ERR_SHAPE;
        // residual_out may only coincide exactly with residual_in
        if (d->residual_out != d->residual_in && overlap(rout, rin)) return AFQ_ERR_ALIAS;
        if (any_overlap(outs, no, ins, ni)) return AFQ_ERR_ALIAS;
        for (int i = 0; i < no; ++i)
            if (overlap(outs[i], rout) || overlap(outs[i], rin)) return AFQ_ERR_ALIAS;
        for (int i = 0; i < ni; ++i)
            if (overlap(ins[i], rout)) return AFQ_ERR_ALIAS;
    } else if (any_overlap(outs, no, ins, ni)) {
        return AFQ_ERR_ALIAS;
    }

    afq::NormPlan p{};
    for (int s = 0; s < d->nseg; ++s) {
        const afq_norm_seg &g = d->seg[s];
        p.seg[s].x = (const uint8_t *)g.x;
        p.seg[s].x_pitch = g.x_row_stride * elt;
        p.seg[s].w = (const uint8_t *)g.weight;
        p.seg[s].values = (uint8_t *)g.out.values;
        p.seg[s].scales = (uint8_t *)g.out.scales;
        p.seg[s].normed = (uint8_t *)g.out.normed;
        p.seg[s].cols = (int32_t)g.cols;
        p.seg[s].chunks = (int32_t)(g.cols / 8);
    }
    p.res_in = (const uint8_t *)d->residual_in;
    p.res_out = (uint8_t *)d->residual_out;
    p.M = d->M;
    p.eps = d->eps;
    p.nseg = d->nseg;
    p.kind = d->kind;
    p.dtype = d->dtype;
    p.mode = d->mode;
    p.qin = d->quant_input;
    p.quant = quant ? 1 : 0;
    return launched(afq::launch_norm(p, stream));
}

int silu_mul_quant(const afq_act_desc *d, void *stream)
{
    if (!d) return AFQ_ERR_NULL;
    return act_common(d, 0, nullptr, stream);
}

int swiglu_oai_quant(const afq_swiglu_desc *d, void *stream)
{
    if (!d) return AFQ_ERR_NULL;
    if (!std::isfinite(d->alpha) || !std::isfinite(d->beta) || std::isnan(d->limit) ||
        !(d->limit > 0.0f))
        return AFQ_ERR_ARG;
    if (!valid_mode(d->act.mode)) return AFQ_ERR_ARG;
    if (d->act.mode != AFQ_MXFP8) return AFQ_ERR_UNSUPPORTED;
    return act_common(&d->act, 1, d, stream);
}

int fp8_quant(const afq_quant_desc *d, void *stream)
{
    if (!d) return AFQ_ERR_NULL;
    if (!valid_mode(d->mode)) return AFQ_ERR_ARG;
    if (d->dtype != AFQ_BF16 && d->dtype != AFQ_FP16 && d->dtype != AFQ_FP32) return AFQ_ERR_ARG;
    if (!rows_ok(d->M)) return AFQ_ERR_SHAPE;
    if (!width_ok(d->cols, d->mode)) return AFQ_ERR_SHAPE;
    if (!stride_ok(d->x_row_stride, d->cols)) return AFQ_ERR_SHAPE;
    if (d->M == 0) return AFQ_OK;
    if (!d->x || !d->out.values || !d->out.scales) return AFQ_ERR_NULL;
    if (d->out.normed) return AFQ_ERR_ARG;
    const int64_t elt = d->dtype == AFQ_FP32 ? 4 : 2;
    if (!aligned(d->x, 16) || (d->x_row_stride * elt) % 16 != 0) return AFQ_ERR_ALIGN;
    if (!aligned(d->out.values, 16) || !aligned(d->out.scales, 4)) return AFQ_ERR_ALIGN;

    const int64_t M = d->M, n = d->cols;
    Span outs[2] = {
        span_of(d->out.values, M, n, 1, n),
        span_of(d->out.scales, M, scale_cols(d->mode, n), scale_elt(d->mode),
                scale_cols(d->mode, n) * scale_elt(d->mode)),
    };
    Span ins[1] = {span_of(d->x, M, n, elt, d->x_row_stride * elt)};
    if (any_wraps(outs, 2) || any_wraps(ins, 1)) return AFQ_ERR_SHAPE;
    if (any_overlap(outs, 2, ins, 1)) return AFQ_ERR_ALIAS;

    afq::QuantPlan p{};
    p.x = (const uint8_t *)d->x;
    p.x_pitch = d->x_row_stride * elt;
    p.values = (uint8_t *)d->out.values;
    p.scales = (uint8_t *)d->out.scales;
    p.M = M;
    p.cols = (int32_t)n;
    p.dtype = d->dtype;
    p.mode = d->mode;
    return launched(afq::launch_quant(p, stream));
}

} // extern "C"
