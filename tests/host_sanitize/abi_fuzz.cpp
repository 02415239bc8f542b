// abi_fuzz.cpp -- fuzzes the host-side validation of the C ABI.
//
// Built with g++ -fsanitize=address,undefined together with afq_abi.cpp (the
// plain C++ translation unit that validates every call) and no HIP code: the
// kernel launchers are replaced by the stubs below, which check the
// invariants the kernels and their launchers rely on.  Whatever descriptor
// validation accepts must satisfy them; a violation aborts.  Every status
// must be one of the documented codes, and a repeated call must return the
// same status.
#include "afq.h"
#include "afq_internal.h"

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <random>

namespace {
void require(bool ok, const char *what)
{
    if (!ok) {
        std::fprintf(stderr, "invariant violated: %s\n", what);
        std::abort();
    }
}
bool al(const void *p, uintptr_t a) { return p && (uintptr_t)p % a == 0; }
int64_t group(int mode) { return mode == AFQ_MXFP8 ? 32 : mode == AFQ_BLOCK128 ? 128 : 8; }
} // namespace

namespace afq {
int launch_norm(const NormPlan &p, void *)
{
    require(p.M > 0 && p.M <= AFQ_MAX_ROWS, "norm: 0 < M <= AFQ_MAX_ROWS");
    require(p.nseg == 1 || p.nseg == 2, "norm: nseg");
    require(p.mode >= 0 && p.mode <= 2 && (p.kind == 0 || p.kind == 1) && (p.dtype == 0 || p.dtype == 1),
            "norm: enums");
    require(p.qin == 0 || (p.qin == 1 && p.mode != AFQ_MXFP8), "norm: quant_input");
    require(p.quant == 1 || (p.quant == 0 && p.qin == 0), "norm: copy only reads the default input");
    require((p.res_in == nullptr) == (p.res_out == nullptr), "norm: residual pair");
    require(p.res_in == nullptr || p.nseg == 1, "norm: residual with one segment");
    require(p.res_in == nullptr || (al(p.res_in, 16) && al(p.res_out, 16)), "norm: residual alignment");
    int64_t total = 0;
    for (int s = 0; s < p.nseg; ++s) {
        const NormSegPlan &g = p.seg[s];
        require(g.cols > 0 && g.cols <= AFQ_MAX_COLS && g.cols % 8 == 0 &&
                    (!p.quant || g.cols % group(p.mode) == 0), "norm: width");
        require(g.chunks == g.cols / 8, "norm: chunks");
        require(al(g.x, 16) && al(g.w, 16), "norm: input pointers");
        if (p.quant)
            require(al(g.values, 16) && al(g.scales, 4), "norm: output pointers");
        else
            require(!g.values && !g.scales && al(g.normed, 16), "norm: copy-only pointers");
        require(g.normed == nullptr || al(g.normed, 16), "norm: copy pointer");
        require(g.x_pitch >= (int64_t)g.cols * 2 && g.x_pitch % 16 == 0 &&
                    g.x_pitch <= AFQ_MAX_ROW_STRIDE * 2, "norm: pitch");
        total += g.cols;
    }
    require(total <= AFQ_MAX_COLS, "norm: total width");
    require(std::isfinite(p.eps) && p.eps >= 0.0f, "norm: eps");
    return 0;
}
int launch_act(const ActPlan &p, void *)
{
    require(p.M > 0 && p.M <= AFQ_MAX_ROWS, "act: M");
    require(p.mode == AFQ_MXFP8 || p.mode == AFQ_BLOCK128, "act: mode");
    require(p.qin == 0 || (p.qin == 2 && p.mode == AFQ_MXFP8), "act: quant_input");
    require(p.quant == 1 || (p.quant == 0 && p.qin == 0), "act: copy only reads the default input");
    require(p.I > 0 && p.I <= AFQ_MAX_COLS && p.I % 8 == 0 && (!p.quant || p.I % group(p.mode) == 0),
            "act: width");
    require(al(p.gu, 16), "act: input pointer");
    if (p.quant)
        require(al(p.values, 16) && al(p.scales, 4), "act: output pointers");
    else
        require(!p.values && !p.scales && al(p.act, 16), "act: copy-only pointers");
    require(p.act == nullptr || al(p.act, 16), "act: copy pointer");
    require(p.gu_pitch >= (int64_t)p.I * 4 && p.gu_pitch % 16 == 0, "act: pitch");
    require(p.act_kind == 0 || p.act_kind == 1, "act: activation kind");
    if (p.act_kind == 1)
        require(p.mode == AFQ_MXFP8 && std::isfinite(p.alpha) && std::isfinite(p.beta) &&
                    p.limit > 0.0f && !std::isnan(p.limit), "act: clamped SwiGLU: MXFP8 and parameters");
    else
        require(p.alpha == 1.0f && p.beta == 0.0f && std::isinf(p.limit), "act: SiLU parameters");
    return 0;
}
int launch_quant(const QuantPlan &p, void *)
{
    require(p.M > 0 && p.M <= AFQ_MAX_ROWS, "quant: M");
    require(p.mode >= 0 && p.mode <= 2 && p.dtype >= 0 && p.dtype <= 2, "quant: enums");
    require(p.cols > 0 && p.cols <= AFQ_MAX_COLS && p.cols % 8 == 0 && p.cols % group(p.mode) == 0,
            "quant: width");
    require(al(p.x, 16) && al(p.values, 16) && al(p.scales, 4), "quant: pointers");
    const int64_t eb = p.dtype == 2 ? 4 : 2;
    require(p.x_pitch >= (int64_t)p.cols * eb && p.x_pitch % 16 == 0, "quant: pitch");
    return 0;
}
} // namespace afq

namespace {
std::mt19937_64 rng(20260211);
template <typename T, size_t N> T pick(const T (&a)[N]) { return a[rng() % N]; }

const int64_t kBig = std::numeric_limits<int64_t>::max();
const int64_t kRows[] = {-5, -1, 0, 1, 2, 7, 64, 1025, 16384, AFQ_MAX_ROWS, (int64_t)AFQ_MAX_ROWS + 1,
                         kBig, std::numeric_limits<int64_t>::min()};
const int64_t kCols[] = {-8, 0, 7, 8, 16, 24, 32, 48, 128, 256, 512, 1536, 2176, 6144, 32768, 32776, kBig};
const int32_t kEnum[] = {-1, 0, 1, 2, 3, 7};
const float kPar[] = {1.702f, 1.0f, 7.0f, 0.0f, -0.5f, 1e-30f, 3e38f, std::numeric_limits<float>::infinity(),
                      -std::numeric_limits<float>::infinity(), std::numeric_limits<float>::quiet_NaN()};
const float kEps[] = {1e-6f, 0.0f, -1e-6f, 1e30f, std::numeric_limits<float>::infinity(),
                      std::numeric_limits<float>::quiet_NaN()};

// A fake device address: NULL, aligned, misaligned, or near the top of the
// address space (never dereferenced: the launchers are stubs).
void *addr(int slot)
{
    switch (rng() % 8) {
    case 0: return nullptr;
    case 1: return (void *)(uintptr_t)(0x100000ull * (slot + 1) + 8);              // misaligned
    case 2: return (void *)(uintptr_t)((std::numeric_limits<uintptr_t>::max() - 4096) & ~(uintptr_t)15);
    case 3: return (void *)(uintptr_t)0x1000000ull;                                // shared by slots
    default: return (void *)(uintptr_t)(0x40000000000ull * (slot + 1));           // disjoint, aligned
    }
}
int64_t stride_for(int64_t cols)
{
    switch (rng() % 6) {
    case 0: return cols;
    case 1: return cols < kBig - 8 ? cols + 8 : kBig;
    case 2: return cols > std::numeric_limits<int64_t>::min() + 8 ? cols - 8 : cols;
    case 3: return AFQ_MAX_ROW_STRIDE;
    case 4: return AFQ_MAX_ROW_STRIDE + 8;
    default: return rng() % 2 ? kBig : -1;
    }
}

// an enum value: mostly one of the valid ones [0, n), sometimes anything
int32_t venum(int n) { return rng() % 10 ? (int32_t)(rng() % n) : pick(kEnum); }

bool documented(int st) { return st <= 0 && st >= -8; }
} // namespace

int main()
{
    long counts[4][9] = {};
    const int iters = 200000;
    for (int it = 0; it < iters; ++it) {
        int st, st2;
        switch (it % 4) {
        case 0: {
            afq_norm_desc d{};
            d.M = pick(kRows);
            d.nseg = rng() % 8 ? 1 + (int32_t)(rng() % 2) : (int32_t)(rng() % 4);
            d.kind = venum(2);
            d.dtype = venum(2);
            d.mode = venum(3);
            d.eps = rng() % 4 ? 1e-6f : pick(kEps);
            d.quant_input = venum(2);
            for (int s = 0; s < 2; ++s) {
                d.seg[s].cols = pick(kCols);
                d.seg[s].x_row_stride = stride_for(d.seg[s].cols);
                d.seg[s].x = addr(4 * s);
                d.seg[s].weight = addr(4 * s + 1);
                d.seg[s].out.values = addr(4 * s + 2);
                d.seg[s].out.scales = addr(4 * s + 3);
                d.seg[s].out.normed = rng() % 2 ? addr(8 + s) : nullptr;
            }
            if (rng() % 2) {
                void *rin = addr(10);
                d.residual_in = rin;
                d.residual_out = rng() % 3 ? addr(11) : rin;
            }
            st = fused_add_rmsnorm_quant(&d, nullptr);
            st2 = fused_add_rmsnorm_quant(&d, nullptr);
            break;
        }
        case 1: {
            afq_act_desc d{};
            d.M = pick(kRows);
            d.I = pick(kCols);
            d.gate_up_row_stride = stride_for(2 * (d.I > 0 && d.I < kBig / 4 ? d.I : 8));
            d.gate_up = addr(0);
            d.mode = venum(2);
            d.quant_input = rng() % 2 ? 0 : venum(3);
            d.out.values = addr(1);
            d.out.scales = addr(2);
            d.out.normed = rng() % 2 ? addr(3) : nullptr;
            st = silu_mul_quant(&d, nullptr);
            st2 = silu_mul_quant(&d, nullptr);
            break;
        }
        case 3: {
            afq_swiglu_desc sd{};
            afq_act_desc &d = sd.act;
            d.M = pick(kRows);
            d.I = pick(kCols);
            d.gate_up_row_stride = stride_for(2 * (d.I > 0 && d.I < kBig / 4 ? d.I : 8));
            d.gate_up = addr(0);
            d.mode = rng() % 4 ? AFQ_MXFP8 : venum(3);
            d.quant_input = rng() % 2 ? 0 : venum(3);
            d.out.values = rng() % 8 ? addr(1) : nullptr;
            d.out.scales = d.out.values ? addr(2) : nullptr;
            d.out.normed = rng() % 2 ? addr(3) : nullptr;
            sd.alpha = rng() % 3 ? 1.702f : pick(kPar);
            sd.beta = rng() % 3 ? 1.0f : pick(kPar);
            sd.limit = rng() % 3 ? 7.0f : pick(kPar);
            st = swiglu_oai_quant(&sd, nullptr);
            st2 = swiglu_oai_quant(&sd, nullptr);
            break;
        }
        default: {
            afq_quant_desc d{};
            d.M = pick(kRows);
            d.cols = pick(kCols);
            d.x_row_stride = stride_for(d.cols);
            d.x = addr(0);
            d.dtype = venum(3);
            d.mode = venum(3);
            d.out.values = addr(1);
            d.out.scales = addr(2);
            d.out.normed = rng() % 4 ? nullptr : addr(3);
            st = fp8_quant(&d, nullptr);
            st2 = fp8_quant(&d, nullptr);
            break;
        }
        }
        require(documented(st), "status is a documented code");
        require(st != AFQ_ERR_LAUNCH, "no launch error from the stubs");
        require(st == st2, "same descriptor, same status");
        require(afq_status_string(st) != nullptr, "status string");
        counts[it % 4][-st]++;
    }
    const char *names[4] = {"fused_add_rmsnorm_quant", "silu_mul_quant", "fp8_quant", "swiglu_oai_quant"};
    for (int e = 0; e < 4; ++e) {
        std::printf("%s:", names[e]);
        for (int c = 0; c < 9; ++c) std::printf(" %d:%ld", -c, counts[e][c]);
        std::printf("\n");
    }
    for (int e = 0; e < 4; ++e)
        require(counts[e][0] > 0, "some calls are accepted");
    return 0;
}
