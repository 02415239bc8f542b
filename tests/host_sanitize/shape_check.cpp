// Host check of the launch-shape rules (afq_shape.hpp), built with g++ and
// the sanitizers.  Over every chunk count a row can have (1 to 4096: rows of
// 8 to 32768 elements, one chunk of 8 per lane-slot) and a spread of row
// counts and compute-unit counts, every shape the launchers can pick is
// checked against what the kernels assume of it:
//   * a row runs on NT lanes, a whole number (1 to 16) of wavefronts of 64,
//     WPR = NT / 64, with CPL = ceil(C / NT) chunks per lane, 1 to 4 (the
//     launchers instantiate exactly these four), and no lane-slot past the
//     last one a row needs;
//   * rows of fewer than 256 lanes are packed R to a 256-lane block only
//     when NT divides 256, and R > 1 only with one or two wavefronts a row
//     (the norm kernel's row-in-block shift knows only these two);
//   * rows per launch keep a row-kernel grid within 2^31 work-items and a
//     flat launch's chunk index below 2^31;
// plus the rule's measured picks at the sizes it was swept on, and the flat
// kernels' division by C (multiplier and shift from divc) against exact
// division at every boundary n = kC - 1, kC and at random n, for every C.
#include "afq_shape.hpp"

#include <cstdio>
#include <cstdlib>
#include <random>

using namespace afq;

static long failures = 0;
#define CHECK(cond, ...)                                                                            \
    do {                                                                                            \
        if (!(cond)) {                                                                              \
            if (failures < 20) {                                                                    \
                std::printf("FAIL %s:%d %s: ", __FILE__, __LINE__, #cond);                          \
                std::printf(__VA_ARGS__);                                                           \
                std::printf("\n");                                                                  \
            }                                                                                       \
            ++failures;                                                                             \
        }                                                                                           \
    } while (0)

static void check_shape(const RowShapeRt &s, int C, const char *what, long long M, long long cus)
{
    CHECK(s.NT >= 64 && s.NT <= 1024 && s.NT % 64 == 0, "%s C=%d M=%lld cus=%lld NT=%d", what, C, M, cus, s.NT);
    CHECK(s.WPR * 64 == s.NT, "%s C=%d NT=%d WPR=%d", what, C, s.NT, s.WPR);
    CHECK(s.CPL >= 1 && s.CPL <= 4, "%s C=%d M=%lld CPL=%d", what, C, M, s.CPL);
    CHECK((long long)s.CPL * s.NT >= C, "%s C=%d NT=%d CPL=%d (row not covered)", what, C, s.NT, s.CPL);
    CHECK((long long)(s.CPL - 1) * s.NT < C, "%s C=%d NT=%d CPL=%d (idle slot)", what, C, s.NT, s.CPL);
    CHECK(s.NT - 64 < (C + s.CPL - 1) / s.CPL, "%s C=%d NT=%d CPL=%d (idle wavefront)", what, C, s.NT, s.CPL);
    if (s.R > 1) {
        CHECK(s.R * s.NT == 256, "%s C=%d NT=%d R=%d", what, C, s.NT, s.R);
        CHECK(s.WPR == 1 || s.WPR == 2, "%s C=%d WPR=%d R=%d", what, C, s.WPR, s.R);
    } else {
        CHECK(s.R == 1, "%s C=%d R=%d", what, C, s.R);
        CHECK(s.NT >= 256 || 256 % s.NT != 0, "%s C=%d NT=%d R=1 (could pack)", what, C, s.NT);
    }
    const long long step = row_rows_per_launch(s.NT, s.R);
    CHECK(step > 0 && step % s.R == 0, "%s C=%d step=%lld", what, C, step);
    CHECK(step * s.NT <= (1ll << 31), "%s C=%d NT=%d step=%lld", what, C, s.NT, step);
    CHECK((step + s.R) * s.NT > (1ll << 31), "%s C=%d NT=%d step=%lld (not the largest)", what, C, s.NT, step);
}

static void expect(const RowShapeRt &s, int NT, int CPL, int R, const char *what)
{
    CHECK(s.NT == NT && s.CPL == CPL && s.R == R, "%s: got NT=%d CPL=%d R=%d, want NT=%d CPL=%d R=%d", what, s.NT,
          s.CPL, s.R, NT, CPL, R);
}

int main()
{
    const long long Ms[] = {1, 2, 8, 63, 64, 65, 192, 255, 256, 257, 300, 511, 512, 513, 1000, 1024,
                            1025, 1280, 1536, 1537, 2048, 3072, 3584, 4096, 8192, 16384, 1 << 20, 1ll << 26};
    const long long cuss[] = {1, 32, 80, 256, 304};
    long shapes = 0;
    for (int C = 1; C <= 4096; ++C) {
        for (int cpl = 1; cpl <= 4; ++cpl) {
            check_shape(shape_at(C, cpl), C, "shape_at", 0, 0);
            ++shapes;
        }
        for (long long M : Ms) {
            for (long long cus : cuss) {
                const RowShapeRt s = quant_row_shape(C, M, cus);
                check_shape(s, C, "quant_row_shape", M, cus);
                // two chunks per lane while a round at two holds every row, else three
                const RowShapeRt s2 = shape_at(C, 2), s3 = shape_at(C, 3);
                if (rows_per_round(C, 2, 32, cus) >= M)
                    CHECK(s.NT == s2.NT && s.CPL == s2.CPL, "quant C=%d M=%lld cus=%lld", C, M, cus);
                else
                    CHECK(s.NT == s3.NT && s.CPL == s3.CPL, "quant C=%d M=%lld cus=%lld", C, M, cus);
                ++shapes;
            }
            for (long long cus : cuss)
                for (int v = 0; v < 4; ++v) { // per-token, MXFP8 with the copy, anything else, per-token
                                              // without one wavefront a row at up to 256 rows
                    const bool pt = v == 0 || v == 3;
                    const RowShapeRt s = norm_row_shape(C, M, pt, v == 1, cus, v != 3);
                    check_shape(s, C, pt ? "norm pt" : v == 1 ? "norm mx copy" : "norm other", M, cus);
                    if (pt && C > 64 && C <= 256 && (M > 256 || v == 0))
                        CHECK(s.WPR == 1 && s.CPL == (C + 63) / 64, "pt one wavefront C=%d M=%lld", C, M);
                    if (v == 2) expect(s, shape_at(C, 1).NT, shape_at(C, 1).CPL, shape_at(C, 1).R, "norm other");
                    const RowShapeRt b = shape_at(C, 1);
                    if (v == 1 && s.CPL > b.CPL) { // only taken when it holds every row in one round
                                                   // with room, and the base shape does not
                        CHECK(norm_rows_per_round(C, s.CPL, cus) >= M && norm_round_has_room(s, M, cus),
                              "mx copy C=%d M=%lld CPL=%d", C, M, s.CPL);
                        CHECK(M <= 3 * norm_rows_per_round(C, 1, cus) &&
                                  (M > norm_rows_per_round(C, 1, cus) || !norm_round_has_room(b, M, cus)),
                              "mx copy C=%d M=%lld CPL=%d", C, M, s.CPL);
                    }
                    if (v == 1 && M <= norm_rows_per_round(C, 1, cus) && norm_round_has_room(b, M, cus))
                        expect(s, b.NT, b.CPL, b.R, "mx copy, room at the base shape");
                    if (pt && M > 256) // per-token: whole rows fill a CU's 32 slots where some shape can
                        CHECK(32 % s.WPR == 0 || (32 % shape_at(C, 2).WPR && 32 % shape_at(C, 3).WPR &&
                                                  32 % shape_at(C, 4).WPR),
                              "pt C=%d M=%lld WPR=%d", C, M, s.WPR);
                    ++shapes;
                }
        }
        const long long fr = flat_rows_per_launch(C);
        CHECK(fr * C <= (1ll << 31) && (fr + 1) * C > (1ll << 31), "flat C=%d rows=%lld", C, fr);
    }

    // The rule's picks at the sizes it was measured on (256 compute units).
    expect(norm_row_shape(768, 16384, false, true, 256, false), 768, 1, 1, "width 6144, 16384 rows, MXFP8 + copy");
    expect(norm_row_shape(768, 512, false, true, 256, false), 768, 1, 1, "width 6144, 512 rows (one round)");
    expect(norm_row_shape(768, 1024, false, true, 256, false), 384, 2, 1, "width 6144, 1024 rows, MXFP8 + copy");
    expect(norm_row_shape(768, 1536, false, true, 256, false), 256, 3, 1, "width 6144, 1536 rows, MXFP8 + copy");
    expect(norm_row_shape(768, 1537, false, true, 256, false), 768, 1, 1, "width 6144, 1537 rows (four rounds)");
    expect(norm_row_shape(512, 3072, false, true, 256, false), 128, 4, 2, "width 4096, 3072 rows, MXFP8 + copy");
    expect(norm_row_shape(256, 2048, false, true, 256, false), 128, 2, 2, "width 2048, 2048 rows (a full round at one)");
    expect(norm_row_shape(512, 1024, false, true, 256, false), 256, 2, 1, "width 4096, 1024 rows (a full round at one)");
    expect(norm_row_shape(1024, 512, false, true, 256, false), 512, 2, 1, "width 8192, 512 rows (a full round at one)");
    expect(norm_row_shape(512, 2048, false, true, 256, false), 128, 4, 2, "width 4096, 2048 rows (a full round at two)");
    expect(norm_row_shape(1024, 1024, false, true, 256, false), 256, 4, 1, "width 8192, 1024 rows (a full round at two)");
    expect(norm_row_shape(896, 1536, false, true, 256, false), 256, 4, 1, "width 7168, 1536 rows, MXFP8 + copy");
    expect(norm_row_shape(896, 512, false, true, 256, false), 896, 1, 1, "width 7168, 512 rows (room at one)");
    expect(norm_row_shape(256, 2047, false, true, 256, false), 128, 2, 2, "width 2048, 2047 rows (over 90 % of the slots)");
    expect(norm_row_shape(256, 1843, false, true, 256, false), 256, 1, 1, "width 2048, 1843 rows (room at one)");
    expect(norm_row_shape(768, 1024, false, false, 256, false), 768, 1, 1, "width 6144, 1024 rows, 1x128");
    expect(norm_row_shape(768, 8, true, false, 256, true), 384, 2, 1, "width 6144, 8 rows, per-token");
    expect(norm_row_shape(256, 8, true, false, 256, true), 64, 4, 4, "width 2048, 8 rows, per-token (one wavefront a row)");
    expect(norm_row_shape(256, 8192, true, false, 256, true), 64, 4, 4, "width 2048, 8192 rows, per-token (one wavefront a row)");
    expect(norm_row_shape(65, 1, true, false, 256, true), 64, 2, 4, "width 520, 1 row, per-token (one wavefront a row)");
    expect(norm_row_shape(64, 300, true, false, 256, true), 64, 1, 4, "width 512, 300 rows, per-token (one chunk per lane)");
    expect(norm_row_shape(768, 4096, true, false, 256, true), 256, 3, 1, "width 6144, 4096 rows, per-token");
    expect(norm_row_shape(1024, 300, true, false, 256, true), 512, 2, 1, "width 8192, 300 rows, per-token");
    expect(norm_row_shape(96, 8, true, false, 256, true), 64, 2, 4, "width 768, 8 rows, per-token (one wavefront a row)");
    expect(norm_row_shape(96, 8, true, false, 256, false), 128, 1, 2, "width 768, 8 rows, per-token (multi-wavefront)");
    expect(norm_row_shape(256, 192, true, false, 256, false), 256, 1, 1, "width 2048, 192 rows, per-token (multi-wavefront)");
    expect(norm_row_shape(256, 300, true, false, 256, false), 64, 4, 4, "width 2048, 300 rows, per-token (one wavefront a row)");
    expect(norm_row_shape(4096, 8, true, false, 256, true), 1024, 4, 1, "width 32768, 8 rows, per-token");
    // rows wider than 1024 chunks: rounds counted on the shapes that run
    expect(norm_row_shape(2048, 600, false, true, 256, false), 512, 4, 1, "width 16384, 600 rows, MXFP8 + copy");
    expect(norm_row_shape(2048, 1000, false, true, 256, false), 1024, 2, 1, "width 16384, 1000 rows (two rounds at four)");
    expect(norm_row_shape(1025, 300, false, true, 256, false), 576, 2, 1, "width 8200, 300 rows (one round)");
    expect(norm_row_shape(1025, 1000, false, true, 256, false), 384, 3, 1, "width 8200, 1000 rows, MXFP8 + copy");
    // the standalone per-token quantiser at the sizes it was measured on
    expect(quant_row_shape(1024, 8, 256), 512, 2, 1, "quant width 8192, 8 rows");
    expect(quant_row_shape(1024, 1024, 256), 512, 2, 1, "quant width 8192, 1024 rows (one round at two)");
    expect(quant_row_shape(1024, 1025, 256), 384, 3, 1, "quant width 8192, 1025 rows");
    expect(quant_row_shape(256, 8192, 256), 128, 2, 2, "quant width 2048, 8192 rows");
    expect(quant_row_shape(256, 8193, 256), 128, 2, 2, "quant width 2048, 8193 rows (three collapses to two)");
    expect(quant_row_shape(768, 2048, 256), 256, 3, 1, "quant width 6144, 2048 rows");
    expect(quant_row_shape(32, 5, 256), 64, 1, 4, "quant width 256, 5 rows (one chunk per lane)");
    expect(quant_row_shape(4096, 8, 256), 1024, 4, 1, "quant width 32768 (four chunks per lane)");
    expect(quant_row_shape(384, 1100, 256), 192, 2, 1, "quant width 3072, 1100 rows");
    expect(quant_row_shape(2560, 1100, 256), 896, 3, 1, "quant width 20480, 1100 rows");
    // rows per round: 256 CUs x whole rows in 32 wavefront slots (28 at four chunks per lane)
    CHECK(norm_rows_per_round(768, 1, 256) == 512, "rows per round %lld", (long long)norm_rows_per_round(768, 1, 256));
    CHECK(norm_rows_per_round(768, 2, 256) == 1280, "rows per round %lld", (long long)norm_rows_per_round(768, 2, 256));
    CHECK(norm_rows_per_round(512, 4, 256) == 3584, "rows per round %lld", (long long)norm_rows_per_round(512, 4, 256));
    std::printf("shapes: %ld checked, %ld failures\n", shapes, failures);

    // Division by C: n / C == (mulhi(n, m) + n) >> l, the sum in 64 bits.
    std::mt19937_64 rng(20260611);
    long divs = 0;
    const auto div_ok = [](uint32_t n, uint32_t C, DivC d) {
        const uint64_t hi = ((uint64_t)n * d.m) >> 32;
        return (uint32_t)((hi + n) >> d.l) == n / C;
    };
    for (uint32_t C = 1; C <= 4096; ++C) {
        const DivC d = divc(C);
        CHECK(d.l <= 12 && (1u << d.l) >= C && (d.l == 0 || (1u << (d.l - 1)) < C), "divc C=%u l=%u", C, d.l);
        for (uint64_t k : {0ull, 1ull, 2ull, 3ull, (1ull << 31) / C - 1, (1ull << 31) / C, (1ull << 31) / C + 1,
                           (1ull << 32) / C - 1, (1ull << 32) / C}) {
            for (int64_t dn = -1; dn <= 1; ++dn) {
                const int64_t n = (int64_t)(k * C) + dn;
                if (n < 0 || n > 0xffffffffll) continue;
                CHECK(div_ok((uint32_t)n, C, d), "div C=%u n=%lld", C, (long long)n);
                ++divs;
            }
        }
        const uint32_t top = 0xffffffffu;
        CHECK(div_ok(top, C, d), "div C=%u n=max", C);
        for (int t = 0; t < 2000; ++t) {
            const uint32_t n = (uint32_t)rng();
            CHECK(div_ok(n, C, d), "div C=%u n=%u", C, n);
        }
        divs += 2001;
    }
    std::printf("divisions: %ld checked, %ld failures\n", divs, failures);
    if (failures) return 1;
    std::printf("launch shapes ok\n");
    return 0;
}
