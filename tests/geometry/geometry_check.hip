// Host-only checks of the launch geometry (make_geometry is a pure function of
// the call's shape).  Prints "geometry: ok" and exits 0 when every check holds;
// otherwise prints each failure and exits 1.
#include <cstdio>

#include "sv_common.hpp"

static int failures = 0;
#define CHECK(cond, ...)                                   \
    do {                                                   \
        if (!(cond)) {                                     \
            ++failures;                                    \
            std::printf("FAIL %s: ", #cond);               \
            std::printf(__VA_ARGS__);                      \
            std::printf("\n");                             \
        }                                                  \
    } while (0)

static sv::Geometry geo(int mode, int B, int rows, int V, int eb) {
    sv::Geometry g{};
    const bool ok = sv::make_geometry(mode, B, rows, V, eb, &g);
    CHECK(ok, "mode %d B %d rows %d V %d eb %d", mode, B, rows, V, eb);
    return g;
}

static long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

int main() {
    // The benchmarked shapes: statistics tiles of 8 vectors per thread, argmax
    // tiles of 16, sampler chunks of 32 tokens per thread at C3 and 64 at C4.
    {
        const sv::Geometry c3 = geo(0, 64, 4, 128256, 2);
        CHECK(c3.U == 8 && c3.S == 8 && c3.R == 7, "c3 tiles U %d S %d R %d", c3.U, c3.S, c3.R);
        CHECK(c3.chunk2 == 256 * 32 && c3.S2 == 16, "c3 sampler chunk %d S2 %d", c3.chunk2, c3.S2);
        const sv::Geometry c4 = geo(0, 256, 6, 151936, 4);
        CHECK(c4.U == 8 && c4.S == 19, "c4 tiles U %d S %d", c4.U, c4.S);
        CHECK(c4.chunk2 == 256 * 64 && c4.S2 == 10, "c4 sampler chunk %d S2 %d", c4.chunk2, c4.S2);
        const sv::Geometry c5 = geo(2, 32, 61, 128256, 2);
        CHECK(c5.U == 16 && c5.S == 4, "c5 argmax tiles U %d S %d", c5.U, c5.S);
        const sv::Geometry c2g = geo(1, 8, 5, 32000, 2);
        CHECK(c2g.U == 4 && c2g.S == 4, "c2 greedy tiles U %d S %d", c2g.U, c2g.S);
        const sv::Geometry c2s = geo(0, 8, 5, 32000, 2);
        CHECK(c2s.U == 2 && c2s.chunk2 == 256 * 8 && c2s.S2 == 16,
              "c2 stochastic U %d chunk2 %d S2 %d", c2s.U, c2s.chunk2, c2s.S2);
    }
    const int Bs[] = {1, 2, 3, 8, 16, 32, 64, 100, 256, 1000};
    const int Vs[] = {1, 8, 9, 1000, 2048, 2049, 4096, 4097, 32000, 50001, 77777, 128256, 151936, 262144};
    const int ks[] = {0, 1, 3, 5, 8, 16};
    for (int B : Bs)
        for (int V : Vs)
            for (int k : ks)
                for (int eb : {2, 4}) {
                    const sv::Geometry g0 = geo(0, B, k + 1, V, eb);
                    const sv::Geometry g3 = geo(3, B, k + 1, V, eb);
                    const sv::Geometry g5 = geo(5, B, k + 1, V, eb);
                    const long long items8 = (long long)B * ceil_div(V, 256 * 8);
                    // The sampler's 8-token chunks exactly while its workgroups
                    // fit one per compute unit; else at least 16 tokens.
                    CHECK((g0.chunk2 == 256 * 8) == (items8 <= 256), "B %d V %d chunk2 %d", B, V,
                          g0.chunk2);
                    CHECK(g0.S2 == ceil_div(V, g0.chunk2) && g0.S2 <= 256, "B %d V %d S2 %d", B, V,
                          g0.S2);
                    // The filtered call samples alike with or without room for
                    // candidates, never in 8-token chunks, and its candidate-
                    // free layout fits a workspace sized for the plain call.
                    CHECK(g3.chunk2 == g5.chunk2 && g3.S2 == g5.S2 && g5.chunk2 >= 256 * 16,
                          "B %d V %d chunk2 %d/%d", B, V, g3.chunk2, g5.chunk2);
                    CHECK(g5.bytes <= g0.bytes, "B %d V %d k %d eb %d: %zu > %zu", B, V, k, eb,
                          g5.bytes, g0.bytes);
                    CHECK(g3.bytes >= g5.bytes, "B %d V %d", B, V);
                    // Tile floors: a larger U was not taken while it still
                    // reached the floor (512 statistics tiles, 128 argmax).
                    const int epv = 16 / eb;
                    const long long rows0 = (long long)B * (2 * (k + 1) - 1);
                    if (g0.U < 8) {
                        const long long ce = 256LL * (2 * g0.U) * epv;
                        CHECK(rows0 * ceil_div(V, ce) < 512, "stats U %d B %d V %d", g0.U, B, V);
                    }
                    const sv::Geometry g1 = geo(1, B, k + 1, V, eb);
                    if (g1.U < 16) {
                        const long long ce = 256LL * (2 * g1.U) * epv;
                        CHECK((long long)B * (k + 1) * ceil_div(V, ce) < 128, "argmax U %d B %d V %d",
                              g1.U, B, V);
                    }
                }
    if (failures == 0) std::printf("geometry: ok\n");
    return failures == 0 ? 0 : 1;
}
