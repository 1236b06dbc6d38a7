// KDA chunked prefill, two-kernel form for gfx950: bf16 q/k/v, d_k = d_v = 128,
// chunk C = 64, fp32 state.  Per chunk, with the scaled operands of
// kda_chunk_ops.h (decay referenced to R = max(B_C, -RLIM) per channel),
//   N = strict_lower(diag(beta) Kt Kb^T),  T = (I + N)^{-1},  P = lower(Qt Kb^T)
//   G = 2^R S,  U = T diag(beta)(V - Kt G),  O = Qt G + P U,  S <- Gam S + Kbar^T U
// (recurrence from page "Ling-3.1-flash: a 560B hybrid-attention MoE, counted
// from its safetensors headers", section "How KDA and MLA split the work").
// With R = diag(beta)(V - Kt G), U = T R; T is folded into Wb^T = Kbar^T T and
// PT = P T, so that  S <- Gam S + Wb^T R  and  O = Qt G + PT R.
//
// Everything that does not depend on the state is done ONCE per (sequence,
// head, chunk) by prep_kernel, chunk-parallel, and stored in a workspace as
// operand tiles (layout in kda_state_pass.h).  state_kernel then runs the
// serial chain per (sequence, head, 32-column slice), streaming those
// fragments.  The sequences are processed in windows of up to 32 chunks (prep
// for the window, then the state pass over it), which bounds the workspace;
// the fp32 state is carried between windows in the workspace.  Only the
// sequences still running in a window take part in it: they are ranked by
// length, longest first, so that those of window w are the first A_w ranks,
// and the window's length is what the tile budget allows for A_w of them.
#include <algorithm>
#include <vector>

#include "kda_prep_tile.h"
#include "kda_window_plan.h"

namespace kda {
namespace sp {

using namespace co;

constexpr int MAX_WIN = 32;                 // chunks per window, at most
constexpr size_t TILE_BUDGET = 192u << 20;  // bytes of one window's tiles, at most
constexpr int RANK_MAX = 4096;              // sequences ranked by length, at most
constexpr size_t BATCH_TILES = (size_t)4 << 30;  // tiles of the preferred batch workspace, at most

}  // namespace sp

using namespace sp;

// ---------------------------------------------------------------- prep
// grid (active sequences * H, chunks in the window): one workgroup of 4 waves
// per (sequence rank, head, window chunk) runs the operand stages and exports
// the tile (prep_tile, kda_prep_tile.h).  order[rank] is the sequence (order
// NULL: rank = sequence).  GM: the decay inputs' GateMode (per channel, per
// head, or the projection).
template <int GM>
__global__ void __launch_bounds__(256, 3)
prep_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, Gate g,
            const float* __restrict__ beta,
            const int32_t* __restrict__ cu, const int32_t* __restrict__ order, int64_t T, int H,
            int w0, int win, uint8_t* __restrict__ ws_tiles) {
    __shared__ __attribute__((aligned(16))) PrepLds sm;
    __shared__ int slow_flags[4];
    const int slot = blockIdx.x / H, h = blockIdx.x - slot * H, cl = blockIdx.y;
    const int n = order ? order[slot] : slot;
    int64_t tb, te;
    int nc;
    seq_chunks(cu, n, T, tb, te, nc);
    const int c = w0 + cl;
    if (c >= nc) return;
    const int64_t c0 = tb + (int64_t)c * C;
    const int L = (te - c0) < C ? (int)(te - c0) : C;
    const auto rt = window(ws_tiles + ((size_t)(slot * win + cl) * H + h) * TILE, TILE);
    prep_tile<GM, 4>(sm, slow_flags, threadIdx.x >> 6, q, k, g, beta, c0, L, H, h, rt);
}

// ---------------------------------------------------------------- state pass
// grid n_pairs * NS, n_pairs = (ranked sequences in the window) * H, the slices
// of one head placed on one XCD.  Ranks at or above n_prep have no tiles in
// this window (prep_kernel ran for the first n_prep ranks only): they are
// treated as having no chunks, whatever the device's cu_seqlens says, so a
// device copy that disagrees with the host copy cannot send a tile access past
// the ranks that own tiles; 8 waves: the chain waves form R, then
// S <- G + Wb^T R and the next G; the output waves form Z = Qt G, then
// O = Z + PT R; two barriers per chunk (R complete, next G complete).
// Fragments come straight from the tiles into registers, two chunks ahead
// (three register sets in rotation), spread over the step's segments.  OG: the
// outputs are gated, O * sigmoid(z) with z the gate projection zg (o's layout),
// read by the output waves with their fragments.
template <bool OG>
__global__ void __launch_bounds__(512)
state_kernel(const bf16_t* __restrict__ v, const bf16_t* __restrict__ zg,
             const int32_t* __restrict__ cu,
             const int32_t* __restrict__ order, int64_t T, int H,
             int n_pairs, int n_prep, int w0, int win, const uint8_t* __restrict__ ws_tiles,
             float* __restrict__ ws_state, const float* __restrict__ s0,
             float* __restrict__ s_final, bf16_t* __restrict__ o, Snapshots snap) {
    __shared__ __attribute__((aligned(16))) StateLds sm;
    int rp, slice;  // (rank, head) pair and slice
    {
        const int b = blockIdx.x;
        if ((n_pairs & 7) == 0) {
            const int xcd = b & 7, kx = b >> 3;
            rp = (kx / NS) * 8 + xcd;
            slice = kx % NS;
        } else {
            rp = b / NS;
            slice = b % NS;
        }
    }
    const int slot = rp / H, h = rp - slot * H;
    const int n = order ? order[slot] : slot, pair = n * H + h;
    const int j0 = slice * DVS;
    int64_t tb, te;
    int nc;
    seq_chunks(cu, n, T, tb, te, nc);
    if (slot >= n_prep) nc = 0;
    const int c_beg = w0, c_end = min(nc, w0 + win);
    const bool first_window = w0 == 0, last_here = c_end == nc;
    const int tid = threadIdx.x, wave = tid >> 6, cw = wave & 3, lane = tid & 63;
    const int r = lane & 15, q4 = lane >> 4;
    const size_t sidx = (size_t)pair * D * D;
    const float* s_in = first_window ? s0 : ws_state;
    float* s_out = last_here ? s_final : ws_state;

    if (c_beg >= c_end) {  // nothing in this window (ended earlier, or empty sequence)
        if (first_window && nc == 0 && s_final) {
            for (int e = tid; e < D * DVS; e += 512) {
                const size_t at = sidx + (size_t)(e / DVS) * D + j0 + e % DVS;
                s_final[at] = s0 ? s0[at] : 0.f;
            }
        }
        return;
    }

    const size_t row = (size_t)H * D;
    const size_t hoff = (size_t)h * D;
    const int rowb = (int)(row * 2);
    // Rows of chunk c inside this window, 0 outside it.  Every load and store
    // below is issued unconditionally through a buffer window of that many rows
    // (a zero-size window turns it into a no-op), so the number of memory
    // operations in flight is the same on every path and the waits before the
    // first use of each prefetched set stay partial.
    auto chunk_len = [&](int c) -> int {
        if (c < c_beg || c >= c_end) return 0;
        const int64_t rem = te - (tb + (int64_t)c * C);
        return rem < C ? (int)rem : C;
    };
    auto tile_rsrc = [&](int c) {
        const int cc = c < c_end ? c : c_beg;  // keep the address inside the workspace
        return window(ws_tiles + ((size_t)(slot * win + (cc - w0)) * H + h) * TILE,
                      c < c_end ? TILE : 0);
    };
    // this lane's 16-byte piece of the wave's 16 x 32 block of V or O
    const VoPieces<DVS> vp(cw, lane);
    auto vo_rsrc = [&](const bf16_t* base, int c) {
        const int cc = (c >= c_beg && c < c_end) ? c : c_beg;
        return window(base + (size_t)(tb + (int64_t)cc * C) * row + hoff + j0, chunk_len(c) * rowb);
    };
    if (wave < 4) {
        // ============================================================ chain
        StateFrag S;
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 32 * cw + 16 * a + 4 * q4 + e, j = 16 * jb + r;
                    S[a][jb][e] = s_in ? s_in[sidx + (size_t)i * D + j0 + j] : 0.f;
                }
        auto load_a = [&](int c, ChainFragsW& f) {
            chainw_load_a(f, tile_rsrc(c), vo_rsrc(v, c), vp, rowb, cw, lane);
        };
        auto load_b = [&](int c, ChainFragsW& f) { chainw_load_b(f, tile_rsrc(c), cw, lane); };
        ChainFragsW F0, F1, F2;
        load_a(c_beg, F0);
        load_b(c_beg, F0);
        load_a(c_beg + 1, F1);
        load_b(c_beg + 1, F1);
        chain_scale_store(sm, S, F0.gam, cw, lane);
        __syncthreads();
        auto step = [&](int c, const ChainFragsW& cur, const ChainFragsW& nxt,
                        ChainFragsW& later) {
            chain_stage_v(sm, cur.v, vp);
            load_a(c + 2, later);
            chain_yr(sm, cur, cw, lane);
            __syncthreads();
            load_b(c + 2, later);
            chainw_s(sm, cur, nxt.gam, c + 1 < c_end, S,
                     snapshot_at(snap, n, h, H, D, (int64_t)(c + 1) * C, te - tb), j0, cw, lane);
            __syncthreads();
        };
        int c = c_beg;
        for (; c + 3 <= c_end; c += 3) {
            step(c, F0, F1, F2);
            step(c + 1, F1, F2, F0);
            step(c + 2, F2, F0, F1);
        }
        if (c < c_end) step(c, F0, F1, F2);
        if (c + 1 < c_end) step(c + 1, F1, F2, F0);
        if (s_out) {
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 32 * cw + 16 * a + 4 * q4 + e, j = 16 * jb + r;
                        s_out[sidx + (size_t)i * D + j0 + j] = S[a][jb][e];
                    }
        }
    } else {
        // ============================================================ output
        auto load_a = [&](int c, OutFrags& f) { outw_load_a(f, tile_rsrc(c), cw, lane); };
        auto load_b = [&](int c, OutFrags& f) {
            outw_load_b(f, tile_rsrc(c), cw, lane);
            if constexpr (OG) out_load_z(f, vo_rsrc(zg, c), vp, rowb);
        };
        OutFrags F0, F1, F2;
        load_a(c_beg, F0);
        load_b(c_beg, F0);
        load_a(c_beg + 1, F1);
        load_b(c_beg + 1, F1);
        __syncthreads();
        auto step = [&](int c, const OutFrags& cur, OutFrags& later) {
            f32x4 Zc[2];
            out_z(sm, cur, Zc, lane);
            __syncthreads();
            u32x4 out[1];
            outw_o<OG>(sm, cur, Zc, cw, lane, vp, out);
            __builtin_amdgcn_raw_buffer_store_b128(out[0], vo_rsrc(o, c), vp.off(0, rowb), 0, 0);
            load_a(c + 2, later);
            load_b(c + 2, later);
            __syncthreads();
        };
        int c = c_beg;
        for (; c + 3 <= c_end; c += 3) {
            step(c, F0, F2);
            step(c + 1, F1, F0);
            step(c + 2, F2, F1);
        }
        if (c < c_end) step(c, F0, F2);
        if (c + 1 < c_end) step(c + 1, F1, F0);
    }
}

// Rank of every sequence by chunk count, longest first (ties by index):
// order[rank] = sequence.  One thread per sequence.
__global__ void __launch_bounds__(256)
seq_order_kernel(const int32_t* __restrict__ cu, int n_seqs, int64_t T,
                 int32_t* __restrict__ order) {
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= n_seqs) return;
    int64_t b, e;
    int nc;
    seq_chunks(cu, n, T, b, e, nc);
    int rank = 0;
    for (int m = 0; m < n_seqs; ++m) {
        int mc;
        seq_chunks(cu, m, T, b, e, mc);
        rank += (mc > nc) || (mc == nc && m < n);
    }
    order[rank] = n;
}

// Workspace: the fp32 state carry, the rank table, then the tiles of one
// window.  The minimum holds TILE_BUDGET bytes of tiles, or MAX_WIN chunks of
// every sequence if that is less, and at least one chunk of every sequence.
static size_t order_bytes(int n_seqs) { return ((size_t)n_seqs * 4 + 255) & ~(size_t)255; }
static size_t tile_bytes(int n_seqs, int H) {
    const size_t one = (size_t)n_seqs * H * TILE;
    const size_t most = one * MAX_WIN < TILE_BUDGET ? one * MAX_WIN : TILE_BUDGET;
    return most > one ? most : one;
}
size_t prefill_split_workspace_bytes_least(int n_seqs, int H) {
    return (size_t)n_seqs * H * D * D * 4 + order_bytes(n_seqs) + (size_t)n_seqs * H * TILE;
}
size_t prefill_split_workspace_bytes(int n_seqs, int H) {
    return (size_t)n_seqs * H * D * D * 4 + order_bytes(n_seqs) + tile_bytes(n_seqs, H);
}

// Windows of min(32, longest) chunks of every sequence, if that fits
// BATCH_TILES; never below the minimum.  Longer windows amortise the state
// pass's start per window: measured at H = 64, batches of 16-128 sequences ran
// 1.4-2x faster with 8-32 chunk windows than with the 1-2 chunk windows that
// the minimum leaves them.
size_t prefill_split_workspace_bytes_batch(const int32_t* cu_host, int n_seqs, int H) {
    const size_t need = prefill_split_workspace_bytes(n_seqs, H);
    int longest = 0;
    for (int n = 0; n < n_seqs; ++n) {
        const int nc = (int)(((int64_t)cu_host[n + 1] - cu_host[n] + C - 1) / C);
        longest = nc > longest ? nc : longest;
    }
    const size_t one = (size_t)n_seqs * H * TILE;
    size_t win = longest < MAX_WIN ? (size_t)longest : (size_t)MAX_WIN;
    if (one && win * one > BATCH_TILES) win = BATCH_TILES / one;
    const size_t want = (size_t)n_seqs * H * D * D * 4 + order_bytes(n_seqs) + win * one;
    return want > need ? want : need;
}

// Windows run one after the other on the caller's stream: operand kernel, then
// state pass.  (Running the operand kernel of the next window concurrently on a
// second stream was measured slower: a state-pass workgroup takes its CU's
// whole register file, so the two kernels cannot share a CU, and both stream
// the tiles through HBM.)
hipError_t launch_prefill_split(const void* q, const void* k, const void* v, Gate g,
                                const float* beta, const int32_t* cu, const int32_t* cu_host,
                                int n_seqs, int64_t T, int H, const float* s0, float* s_final,
                                const void* out_gate, void* o, Snapshots snap, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    if ((int64_t)n_seqs * H == 0) return hipSuccess;
    // chunk counts, longest first: the ranks' lengths
    std::vector<int> len(n_seqs);
    for (int n = 0; n < n_seqs; ++n) len[n] = (int)(((int64_t)cu_host[n + 1] - cu_host[n] + C - 1) / C);
    std::sort(len.begin(), len.end(), [](int a, int b) { return a > b; });
    float* ws_state = reinterpret_cast<float*>(workspace);
    int32_t* order = reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(workspace) +
                                                (size_t)n_seqs * H * D * D * 4);
    uint8_t* tiles = reinterpret_cast<uint8_t*>(order) + order_bytes(n_seqs);
    // tiles: whatever the caller's workspace holds beyond the state carry and
    // the rank table (at least tile_bytes(n_seqs, H), checked by the caller)
    const size_t tbytes = workspace_bytes - (size_t)(tiles - reinterpret_cast<uint8_t*>(workspace));
    const bool ranked = n_seqs <= RANK_MAX;
    // no table when the ranking is the identity (lengths already non-increasing)
    bool identity = true;
    for (int n = 0; n + 1 < n_seqs && identity; ++n)
        identity = (cu_host[n + 1] - cu_host[n] + C - 1) / C >= (cu_host[n + 2] - cu_host[n + 1] + C - 1) / C;
    hipError_t err = hipSuccess;
    if (ranked && !identity) {
        hipLaunchKernelGGL(seq_order_kernel, dim3((unsigned)((n_seqs + 255) / 256)), dim3(256), 0,
                           stream, cu, n_seqs, T, order);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    } else {
        order = nullptr;
    }
    auto prep = g.mode == GATE_HEAD   ? prep_kernel<GATE_HEAD>
                : g.mode == GATE_PROJ ? prep_kernel<GATE_PROJ>
                                      : prep_kernel<GATE_CH>;
    for (const Window& wd : plan_windows(len, ranked, H, tbytes, TILE, MAX_WIN)) {
        if (wd.rows > 0 && wd.active > 0) {
            hipLaunchKernelGGL(prep, dim3((unsigned)(wd.active * H), (unsigned)wd.rows),
                               dim3(256), 0, stream, (const bf16_t*)q, (const bf16_t*)k, g, beta,
                               cu, order, T, H, wd.w0, wd.win, tiles);
            err = hipGetLastError();
            if (err != hipSuccess) return err;
        }
        hipLaunchKernelGGL(out_gate ? state_kernel<true> : state_kernel<false>,
                           dim3((unsigned)((int64_t)wd.visit * H * NS)), dim3(512), 0, stream,
                           (const bf16_t*)v, (const bf16_t*)out_gate, cu, order, T, H,
                           wd.visit * H, wd.active,
                           wd.w0, wd.win, tiles, ws_state, s0, s_final, (bf16_t*)o, snap);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace kda
