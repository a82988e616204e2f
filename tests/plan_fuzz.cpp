// Host-side fuzz of the work-division arithmetic that the decode kernels and
// sr_plan_parts share (split plans, ranges, item parts), built by
// tests/test_host_sanitizers.py with the undefined-behaviour and address
// sanitizers, so any signed overflow or out-of-bounds access aborts the run.
// Draws launch layouts over the supported envelope and checks that every
// active item's chunks are covered exactly once, in workgroup order.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "sr_internal.h"

using namespace sr;

static void fail(const char* what, long long a, long long b) {
    std::fprintf(stderr, "plan fuzz: %s (%lld, %lld)\n", what, a, b);
    std::exit(2);
}

int main(int argc, char** argv) {
    const int iters = argc > 1 ? std::atoi(argv[1]) : 20000;
    std::mt19937_64 rng(20261203);
    auto pick = [&](long long lo, long long hi) {  // inclusive
        return lo + static_cast<long long>(rng() % static_cast<unsigned long long>(hi - lo + 1));
    };
    for (int it = 0; it < iters; ++it) {
        const int32_t n_items = static_cast<int32_t>(pick(0, 9) < 8 ? pick(1, 256) : pick(1, 32768));
        const int64_t T = pick(0, 3) ? pick(1, 600000) : pick(1, 0x7fffffffLL);
        const int32_t chunk = 16 << pick(0, 5);
        const int32_t fixed = pick(0, 3) ? 0 : static_cast<int32_t>(pick(1, 64));
        int64_t grid64 = fixed ? static_cast<int64_t>(n_items) * fixed : pick(1, 4) * 256;
        if (!fixed && grid64 < n_items) grid64 = n_items;
        if (grid64 > 0x7fffffffLL) continue;
        const int32_t grid = static_cast<int32_t>(grid64);
        const int32_t es = pick(0, 1) ? 2 : 4, gp = 1 << pick(0, 4), d = pick(0, 1) ? 64 : 128;
        const int32_t round = merge_round_splits(d, gp, pick(0, 1) ? 4 : 8);
        const int32_t cap = fixed ? fixed
                                  : adaptive_split_cap(T, chunk, int64_t{chunk} * 2 * d * es, round, grid);
        if (!fixed && (cap < 1 || cap > (T + chunk - 1) / chunk || cap > grid))
            fail("cap out of range", cap, T);
        const int32_t n = static_cast<int32_t>(pick(0, n_items));
        const SplitPlan p = make_split_plan(fixed, grid, cap, n, T, chunk);
        if (n == 0) continue;
        if (p.P > grid) fail("more workgroups than the grid", p.P, grid);
        const int64_t N = static_cast<int64_t>(n) * p.C;
        // ranges tile [0, N) in order
        const int32_t step = p.P > 4096 ? p.P / 2048 : 1;  // sample large grids
        int64_t prev = range_begin(p, 0);
        if (prev != 0) fail("first range does not start at 0", prev, 0);
        for (int32_t w = 1; w <= p.P; w += (w + step <= p.P ? step : 1)) {
            const int64_t b = range_begin(p, w);
            if (b < prev) fail("ranges out of order", b, prev);
            prev = b;
        }
        if (range_begin(p, p.P) != N) fail("ranges do not end at N", range_begin(p, p.P), N);
        // items: parts contiguous, first part of item i+1 follows the last of i
        int32_t expect_lo = 0;
        const int32_t istep = n > 2048 ? n / 1024 : 1;
        for (int32_t i = 0; i < n; i += istep) {
            int32_t w_lo, parts;
            item_parts(p, i, w_lo, parts);
            if (parts < 1 || w_lo < 0 || w_lo + parts > p.P) fail("item parts out of range", w_lo, parts);
            if (istep == 1 && p.balanced && w_lo != expect_lo && w_lo != expect_lo - 1)
                fail("item parts not contiguous", w_lo, expect_lo);
            expect_lo = w_lo + parts;
            int32_t ib, ie;
            range_items(p, w_lo, ib, ie);
            if (ib > i || ie <= i) fail("first part does not reach its item", ib, i);
            range_items(p, w_lo + parts - 1, ib, ie);
            if (ib > i || ie <= i) fail("last part does not reach its item", ie, i);
        }
        // lane_of inverts lane_start
        for (int32_t l = 0; l < p.S; l += (p.S > 64 ? p.S / 32 : 1)) {
            const int32_t q0 = lane_start(p, l);
            if (q0 >= p.C) continue;
            int32_t ll, kk;
            lane_of(p, q0, ll, kk);
            if (ll != l || kk != 0) fail("lane_of does not invert lane_start", ll, l);
        }
    }
    std::printf("plan fuzz: %d layouts ok\n", iters);
    return 0;
}
