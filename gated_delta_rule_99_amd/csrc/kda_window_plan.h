// Window plan of the two-kernel prefill (host code only, no HIP): which ranked
// sequences take part in each window of chunks and how long the window is.
//
// The sequences are ranked by chunk count, longest first.  Window w covers
// chunks [w0, w0 + win) of every sequence still running at chunk w0: the first
// `active` ranks.  Their operand tiles share the workspace's tile space, so the
// window is as long as tile_space / (active * H * tile) allows, between 1 and
// max_win chunks.  prep_kernel forms tiles for ranks [0, active) and window
// chunks [0, rows); the state pass visits ranks [0, visit) (every rank in the
// first window, so that empty sequences get their final state) and runs chunks
// only for ranks below `active`.  Tile (rank r, window chunk cl, head h) sits at
// byte ((r * win + cl) * H + h) * tile of the tile space, so every tile either
// kernel touches lies below active * win * H * tile <= tile_space.
#pragma once

#include <stddef.h>

#include <vector>

namespace kda {

struct Window {
    int w0;      // first chunk of the window
    int win;     // chunks of tile space per rank
    int active;  // ranks with tiles (and chunks) in this window
    int visit;   // ranks the state pass visits
    int rows;    // window chunks that prep_kernel forms (<= win)
};

// sorted_len: chunk counts in non-increasing order (rank order).  ranked ==
// false: the sequences keep their order and all take part in every window.
// tile_space must hold at least one tile of every sequence and head
// (n_seqs * H * tile bytes); then every window has win >= 1.
inline std::vector<Window> plan_windows(const std::vector<int>& sorted_len, bool ranked, int H,
                                        size_t tile_space, size_t tile, int max_win) {
    std::vector<Window> plan;
    const int n_seqs = (int)sorted_len.size();
    if (n_seqs == 0) return plan;
    const int max_chunks = sorted_len[0];
    int w0 = 0;
    do {
        int active = 0;
        while (active < n_seqs && sorted_len[active] > w0) ++active;
        if (!ranked) active = n_seqs;
        const int visit = w0 == 0 ? n_seqs : active;
        const size_t w = active ? tile_space / ((size_t)active * H * tile) : 1;
        const int win = w < 1 ? 1 : (w > (size_t)max_win ? max_win : (int)w);
        const int rows = max_chunks - w0 < win ? max_chunks - w0 : win;
        plan.push_back(Window{w0, win, active, visit, rows});
        w0 += win;
    } while (w0 < max_chunks);
    return plan;
}

}  // namespace kda
