// Host-side coverage check of the column-stripe geometry of the aux-loss
// kernels: walks every block, split, wave, lane, step and component the
// kernels visit, with the same index maps (router_params.h), and checks
// that every in-range element of [T,E] is visited exactly once, that every
// other access is masked (column >= E) or past its split's buffer, that
// byte offsets fit the 32-bit buffer offsets, that the LDS column index of
// the count kernel stays within its array, and that the loss workspace fits
// the queried size (the forward's geometry; the gradient's writes only);
// for the count geometry also that the lane width and row steps are the
// ones the kernel is built for, that the accumulators and tickets fit the
// queried workspace, and that the workspace bound holds for every E.
// Prints "ok" or the first failure; exit status 0/1.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "router_params.h"

using namespace rker;

static int fail(const char *what, long long T, int E, int steps)
{
    std::printf("FAIL %s T=%lld E=%d steps=%d\n", what, T, E, steps);
    return 1;
}

static int check(int64_t T, int E, int waves, int cpl_log2, int steps, int max_blocks,
                 uint32_t esize)
{
    const ColGeo g = col_geo(T, E, waves, cpl_log2, steps, max_blocks);
    const int width = geo_width(g);
    const int cpl = 1 << cpl_log2;
    if (width > (64 << cpl_log2) || g.rows_per_split != (waves * steps << g.rpw_log2))
        return fail("geometry", T, E, steps);
    if ((int64_t)g.nstripe * width < E || (int64_t)(g.nstripe - 1) * width >= E)
        return fail("stripes", T, E, steps);
    if (g.nsplit * g.rows_per_split < T || (g.nsplit > 0 && (g.nsplit - 1) * g.rows_per_split >= T))
        return fail("splits", T, E, steps);
    if (g.gsplit > g.nsplit || (T > 0 && g.gsplit < 1) ||
        (int64_t)g.gsplit * g.nstripe > (max_blocks > g.nstripe ? max_blocks : g.nstripe))
        return fail("grid", T, E, steps);
    const size_t ws = aux_ws_bytes(T, E);
    const bool loss = waves == kLossWaves && cpl_log2 == kLossCpl && steps == kLossSteps &&
                      max_blocks == kLossMaxBlocks;
    if (loss && ((size_t)g.gsplit * g.nstripe * 8 > ws || ws > kLossScratchBytes))
        return fail("loss workspace", T, E, steps);
    std::vector<uint8_t> seen((size_t)T * E, 0);
    const unsigned grid = (unsigned)g.gsplit * (unsigned)g.nstripe;
    for (unsigned b = 0; b < grid; b++) {
        const int stripe = (int)(b % (unsigned)g.nstripe);
        const int s0 = (int)(b / (unsigned)g.nstripe);
        for (int64_t sp = s0; sp < g.nsplit; sp += g.gsplit) {
            const int64_t r0 = sp * g.rows_per_split;
            const int64_t rows = T - r0 < g.rows_per_split ? T - r0 : g.rows_per_split;
            const uint64_t limit = (uint64_t)rows * E * esize;  // buffer bytes
            if (limit >= 0x80000000ull)
                return fail("buffer range", T, E, steps);
            for (int w = 0; w < waves; w++)
                for (int lane = 0; lane < 64; lane++) {
                    const int col0 = geo_col0(g, stripe, lane);
                    if (col0 < E && col0 - stripe * width + cpl - 1 >= (64 << cpl_log2))
                        return fail("column index past the stripe", T, E, steps);
                    // the count kernel's LDS slot of (row_lane, column) is 16*lane
                    if (geo_row_lane(g, lane) * width + (col0 - stripe * width) != lane * cpl)
                        return fail("lds region index", T, E, steps);
                    if (E % cpl == 0 && col0 < E && col0 + cpl - 1 >= E)
                        return fail("vector straddles row end", T, E, steps);
                    if (E % 4 == 0 && col0 < E && col0 % 4 != 0)
                        return fail("word access misaligned", T, E, steps);
                    const int rl = geo_row_lane(g, lane);
                    for (int k = 0; k < steps; k++) {
                        const int rr = geo_split_row(g, w, k, rl);
                        for (int u = 0; u < cpl; u++) {
                            const int col = col0 + u;
                            if (col >= E)
                                continue;  // masked with the out-of-range offset
                            const uint64_t off = ((uint64_t)rr * E + col) * esize;
                            if (off >= 0x80000000ull)
                                return fail("offset overflow", T, E, steps);
                            if (off >= limit) {
                                if (rr < rows)
                                    return fail("in-range row dropped", T, E, steps);
                                continue;  // past the split: dropped
                            }
                            if (rr >= rows)
                                return fail("row past split inside buffer", T, E, steps);
                            uint8_t &s = seen[(size_t)(r0 + rr) * E + col];
                            if (++s != 1)
                                return fail("visited twice", T, E, steps);
                        }
                    }
                }
        }
    }
    for (size_t i = 0; i < seen.size(); i++)
        if (seen[i] != 1)
            return fail("not visited", T, E, steps);
    return 0;
}

// The count kernel's geometry for (T, E), walked like the others, plus its
// workspace: a 64-bit accumulator for each of nstripe*width columns inside
// count_ws_bytes(E) <= 65536 bytes, and contribution counts (gsplit per
// column) that fit the accumulator's high half.
static int check_count(int64_t T, int E)
{
    const ColGeo g = count_geo(T, E);
    if (g.cpl_log2 < 2 || g.cpl_log2 > 4 || g.steps < 1 || g.steps > kCountMaxSteps ||
        (g.steps & (g.steps - 1)) != 0)
        return fail("count lane width / steps", T, E, g.steps);
    const size_t words = (size_t)g.nstripe * geo_width(g);
    if (words > count_ws_words(E) || count_ws_words(E) * 8 > count_ws_bytes(E) ||
        count_ws_bytes(E) > 65536 || count_ws_bytes(E) % 256 != 0)
        return fail("count workspace", T, E, g.steps);
    if (T > 0 && (int64_t)g.gsplit * g.nstripe > (kCountMaxBlocks > g.nstripe ? kCountMaxBlocks
                                                                                : g.nstripe))
        return fail("count grid", T, E, g.steps);
    return check(T, E, kCountWaves, g.cpl_log2, g.steps, kCountMaxBlocks, 1);
}

int main()
{
    // the loss partials fit the library's own buffer for every E (any T:
    // the grid is capped)
    for (int E = 1; E <= 4096; E++)
        for (int64_t T : {(int64_t)1, (int64_t)8192, (int64_t)1 << 20, (int64_t)1 << 31})
            if (aux_ws_bytes(T, E) > kLossScratchBytes)
                return fail("loss partials past the library's buffer", T, E, 0);
    for (int E = 1; E <= 4096; E++)
        if (check_count(1, E))
            return 1;
    const int64_t Ts[] = {0, 1, 3, 64, 127, 128, 129, 1031, 4096, 8192, 20000};
    const int Es[] = {1, 2, 3, 4, 5, 7, 8, 16, 60, 64, 100, 128, 255, 256, 257,
                      512, 999, 1000, 2304, 4095, 4096};
    int bad = 0;
    for (int64_t T : Ts)
        for (int E : Es) {
            if (T * E > 40000000)
                continue;
            bad |= check_count(T, E);
            bad |= check(T, E, kLossWaves, kLossCpl, kLossSteps, kLossMaxBlocks, 4);
            bad |= check(T, E, kLossWaves, kLossCpl, kLossSteps, kLossMaxBlocks, 2);
            bad |= check(T, E, kLossWaves, kLossCpl, kLossBwdSteps, kLossBwdMaxBlocks, 4);
            bad |= check(T, E, kLossWaves, kLossCpl, kLossBwdSteps, kLossBwdMaxBlocks, 2);
            if (bad)
                return 1;
        }
    // grid cap reached: blocks loop over several splits
    bad |= check_count(300000, 64);
    bad |= check_count(40000, 2304);
    bad |= check_count(70000, 4096);
    bad |= check(70000, 2304, kLossWaves, kLossCpl, kLossSteps, kLossMaxBlocks, 4);
    bad |= check(100000, 4, kLossWaves, kLossCpl, kLossSteps, 64, 4);
    bad |= check(40000, 2304, kLossWaves, kLossCpl, kLossBwdSteps, kLossBwdMaxBlocks, 4);
    if (bad)
        return 1;
    std::printf("ok\n");
    return 0;
}
