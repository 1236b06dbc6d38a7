// CPU check of the two-kernel prefill's window plan (kda_window_plan.h): for
// random batches and tile spaces, every tile that prep_kernel or the state pass
// can touch lies inside the tile space, whatever chunk counts the device copy
// of cu_seqlens holds (the state pass runs chunks only for ranks below
// `active`, and at most `win` of them per window), and the windows cover every
// chunk of every sequence.  Prints "ok <cases>" or the first failure.
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <random>
#include <vector>

#include "kda_window_plan.h"

static int fail(const char* what, int a, int b) {
    printf("FAIL %s (%d, %d)\n", what, a, b);
    return 1;
}

static int check(std::vector<int> len, int H, size_t tile_space, size_t tile, int max_win,
                 bool ranked) {
    std::sort(len.begin(), len.end(), [](int a, int b) { return a > b; });
    const int n = (int)len.size();
    const std::vector<kda::Window> plan = kda::plan_windows(len, ranked, H, tile_space, tile,
                                                            max_win);
    if (n == 0) return plan.empty() ? 0 : fail("plan for no sequences", 0, 0);
    int next = 0;
    for (size_t i = 0; i < plan.size(); ++i) {
        const kda::Window& w = plan[i];
        if (w.w0 != next) return fail("windows not contiguous", w.w0, next);
        if (w.win < 1 || w.win > max_win) return fail("window length", w.win, max_win);
        if (w.active < 0 || w.active > n || w.visit < w.active || w.visit > n)
            return fail("rank counts", w.active, w.visit);
        if (w.rows > w.win) return fail("prep rows beyond the window", w.rows, w.win);
        // every tile (rank < active, window chunk < win, head < H) inside the space
        if ((size_t)w.active * w.win * H * tile > tile_space)
            return fail("tiles beyond the tile space", w.active, w.win);
        // every sequence with chunks left at w0 takes part
        for (int r = 0; r < n; ++r)
            if (len[r] > w.w0 && r >= w.active) return fail("running rank left out", r, w.w0);
        if (i == 0 && w.visit != n) return fail("first window visits every rank", w.visit, n);
        next = w.w0 + w.win;
    }
    if (next < len[0]) return fail("chunks left uncovered", next, len[0]);
    return 0;
}

int main() {
    const size_t TILE = 58112;
    const int MAX_WIN = 32;
    const size_t BUDGET = (size_t)192 << 20;
    std::mt19937 rng(12345);
    int cases = 0;
    // the batch from the review: 8 empty sequences and one of 64 tokens, H = 64
    {
        std::vector<int> len(8, 0);
        len.push_back(1);
        const size_t one = len.size() * 64 * TILE;
        if (check(len, 64, one, TILE, MAX_WIN, true)) return 1;
        ++cases;
    }
    for (int it = 0; it < 5000; ++it) {
        const int n = 1 + (int)(rng() % 700);
        const int H = 1 + (int)(rng() % 64);
        std::vector<int> len(n);
        const int maxc = 1 + (int)(rng() % 3000);
        for (int &l : len) l = (rng() % 4 == 0) ? 0 : (int)(rng() % (maxc + 1));
        // tile space: the minimum the library asks for, or more
        const size_t one = (size_t)n * H * TILE;
        size_t minimum = std::min(one * MAX_WIN, BUDGET);
        minimum = std::max(minimum, one);
        const size_t space = minimum + (rng() % 3 == 0 ? (size_t)(rng() % 7) * one : 0);
        if (check(len, H, space, TILE, MAX_WIN, n <= 4096)) return 1;
        if (check(len, H, space, TILE, MAX_WIN, false)) return 1;
        cases += 2;
    }
    printf("ok %d\n", cases);
    return 0;
}
