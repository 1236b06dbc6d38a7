// KDA chunked prefill, two-kernel form for gfx950: bf16 q/k/v, d_k = d_v = 128,
// chunk C = 64, fp32 state.  Per chunk, with the decay referenced to the chunk end,
//   Kt = K * D, Qt = Q * D, Kb = K * F   (D = e^{b - b_C}, F = e^{b_C - b})
//   N = strict_lower(diag(beta) Kt Kb^T),  T = (I + N)^{-1},  P = lower(Qt Kb^T)
//   G = Gam * S,  U = T diag(beta)(V - Kt G),  O = Qt G + P U,  S <- G + Kb^T U
// (recurrence from page "Ling-3.1-flash: a 560B hybrid-attention MoE, counted
// from its safetensors headers", section "How KDA and MLA split the work").
//
// Everything that does not depend on the state is done ONCE per (sequence,
// head, chunk) by prep_kernel, chunk-parallel, and stored in a workspace in
// the exact lane order of the state pass's MFMA operands (each lane later
// reads one contiguous 16-byte fragment).  state_kernel then runs the serial
// chain per (sequence, head, 32-column slice), streaming those fragments.
// The sequence is processed in windows of up to 32 chunks (prep for the
// window, then the state pass over it), which bounds the workspace; the fp32
// state is carried between windows in the workspace.
//
// Workspace tile of one (sequence, window chunk, head), byte offsets:
//   0      Kt fragments   [row block c 0..3][kk 0..3][lane 64][16 B]
//   16384  Qt fragments   same
//   32768  Kb^T fragments [c 0..3][a 0..1][kk 0..1][lane][16 B]   (rows 32c+16a)
//   49152  T fragments    [c 0..3][kk 0..1][lane][16 B]
//   57344  P fragments    same
//   65536  beta[64] fp32, 65792 Gam[128] fp32
// MFMA operand layouts (gfx950, lane l, r = l % 16, q4 = l / 16):
//   16x16x32 bf16: A[r][8 q4 + e], B[8 q4 + e][r], D[4 q4 + e][r]
//   16x16x16 bf16: A[r][4 q4 + e], B[4 q4 + e][r], D[4 q4 + e][r]
#include "kda_chunk_ops.h"

namespace kda {
namespace sp {

using namespace co;

constexpr int DVS = 32, NS = D / DVS;
constexpr int MAX_WIN = 32;                 // chunks per window, at most
constexpr size_t TILE_BUDGET = 192u << 20;  // bytes of one window's tiles, at most
constexpr int TILE = 66304;
constexpr int OFF_KT = 0, OFF_QT = 16384, OFF_KBT = 32768, OFF_T = 49152, OFF_P = 57344,
              OFF_BETA = 65536, OFF_GAM = 65792;

}  // namespace sp

using namespace sp;

// ---------------------------------------------------------------- prep
// grid (n_seqs * H, chunks in the window): one workgroup of 4 waves per
// (sequence, head, window chunk) runs the operand stages and exports the tile.
// GH: g holds one log decay per (token, head) instead of one per key channel.
template <bool GH>
__global__ void __launch_bounds__(256, 2)
prep_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
            const float* __restrict__ g, const float* __restrict__ beta,
            const int32_t* __restrict__ cu, int64_t T, int H, int w0, int win,
            uint8_t* __restrict__ ws_tiles) {
    __shared__ __attribute__((aligned(16))) ChunkLds sm;
    const int pair = blockIdx.x, cl = blockIdx.y, n = pair / H, h = pair - n * H;
    int64_t tb, te;
    int nc;
    seq_chunks(cu, n, T, tb, te, nc);
    const int c = w0 + cl;
    if (c >= nc) return;
    const int tid = threadIdx.x, p = tid >> 6, lane = tid & 63;
    const int r = lane & 15, q4 = lane >> 4;
    const int64_t c0 = tb + (int64_t)c * C;
    const int L = (te - c0) < C ? (int)(te - c0) : C;
    const auto rt = window(ws_tiles + ((size_t)(n * win + cl) * H + h) * TILE, TILE);

    zero_tp(sm, tid, 256);
    ChunkIn in;
    load_chunk<GH>(in, q, k, g, beta, c0, L, H, h, p, lane);
    if (p == 0)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(in.beta), rt, OFF_BETA + 4 * lane, 0,
                                              0);
    decay_stage(
        sm, in, p, lane,
        [&](int ch0, const float(&gam)[4]) {
            __builtin_amdgcn_raw_buffer_store_b128(
                u32x4{__float_as_uint(gam[0]), __float_as_uint(gam[1]), __float_as_uint(gam[2]),
                      __float_as_uint(gam[3])},
                rt, OFF_GAM + 4 * ch0, 0, 0);
        },
        [&](int i, int tg, u32x4 piece) {
            // Kb^T fragment (row block i / 16, k block tg / 4), lane (i % 16, tg % 4)
            const int blk = (i >> 5) * 4 + ((i >> 4) & 1) * 2 + (tg >> 2);
            const int ln = (i & 15) + 16 * (tg & 3);
            __builtin_amdgcn_raw_buffer_store_b128(piece, rt, OFF_KBT + (blk * 64 + ln) * 16, 0, 0);
        });
    __syncthreads();
    // Kt and Qt fragments out (wave p exports row block p)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 a = ld8(sm.Kt + (16 * p + r) * LDK + 32 * kk + 8 * q4);
        const bf16x8 b = ld8(sm.Qt + (16 * p + r) * LDK + 32 * kk + 8 * q4);
        __builtin_amdgcn_raw_buffer_store_b128(as_u4(a), rt, OFF_KT + ((p * 4 + kk) * 64 + lane) * 16,
                                               0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(as_u4(b), rt, OFF_QT + ((p * 4 + kk) * 64 + lane) * 16,
                                               0, 0);
    }
    n_stage(sm, p, lane);
    __syncthreads();
    merge_stage(sm, p, lane);
    __syncthreads();
    // T and P fragments out (wave p exports row block p)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 a = ld8(sm.T + (16 * p + r) * LDT + 32 * kk + 8 * q4);
        const bf16x8 b = ld8(sm.P + (16 * p + r) * LDT + 32 * kk + 8 * q4);
        __builtin_amdgcn_raw_buffer_store_b128(as_u4(a), rt, OFF_T + ((p * 2 + kk) * 64 + lane) * 16,
                                               0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(as_u4(b), rt, OFF_P + ((p * 2 + kk) * 64 + lane) * 16,
                                               0, 0);
    }
}

// ---------------------------------------------------------------- state pass
// grid n_seqs * H * NS (the slices of one head placed on one XCD); 8 waves.
// Waves 0-3 carry the chain that the next chunk depends on,
//   Y = Kt G,  R = diag(beta)(V - Y),  U = T R,  S <- G + Kb^T U,  G' = Gam' S;
// waves 4-7 produce the output off that chain, Z = Qt G and O = Z + P U.
// Wave c of either group owns rows [16c, 16c+16) of the chunk (Y, R, U, Z, O)
// and chain wave c owns state rows [32c, 32c+32) of the slice.  Per chunk the
// two groups meet at three barriers: R complete, U complete, next G complete.
// V and O move with one 16-byte access per lane (16 rows x 32 columns per wave)
// and are turned into the accumulator layout (lane (r, q4) holds rows 4q4 + e
// of column r) through a staging tile that only the wave itself touches.
constexpr int LDX = 40;  // row stride (bf16) of the V and O staging tiles
struct StateSmem {
    uint16_t Gt[DVS * LDK];  // bf16 (Gam * S)^T [j][i]
    uint16_t Rt[DVS * LDT];  // R^T [j][t]
    uint16_t Ut[DVS * LDT];  // U^T [j][t]
    uint16_t V[C * LDX];     // V slice [t][j]: each chain wave stages its own 16 rows
    uint16_t O[C * LDX];     // O slice [t][j]: each output wave stages its own 16 rows
};

struct ChainFrags {
    bf16x8 K[4], Kb[2][2], T[2];
    float4 bet, gam[2];
    uint4 v;  // V[16c + (lane >> 2)][8 (lane & 3) + 0..7]
};
struct OutFrags {
    bf16x8 Q[4], P[2];
};

__global__ void __launch_bounds__(512)
state_kernel(const bf16_t* __restrict__ v, const int32_t* __restrict__ cu, int64_t T, int H,
             int n_pairs, int w0, int win, const uint8_t* __restrict__ ws_tiles,
             float* __restrict__ ws_state, const float* __restrict__ s0,
             float* __restrict__ s_final, bf16_t* __restrict__ o, Snapshots snap) {
    __shared__ __attribute__((aligned(16))) StateSmem sm;
    int pair, slice;
    {
        const int b = blockIdx.x;
        if ((n_pairs & 7) == 0) {
            const int xcd = b & 7, kx = b >> 3;
            pair = (kx / NS) * 8 + xcd;
            slice = kx % NS;
        } else {
            pair = b / NS;
            slice = b % NS;
        }
    }
    const int n = pair / H, h = pair - n * H;
    const int j0 = slice * DVS;
    int64_t tb, te;
    int nc;
    seq_chunks(cu, n, T, tb, te, nc);
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
        return window(ws_tiles + ((size_t)(n * win + (cc - w0)) * H + h) * TILE,
                      c < c_end ? TILE : 0);
    };
    // this lane's (row, column) of the chunk in the accumulator layout, as a
    // byte offset from the slice's first element of the chunk's first row
    // this lane's 16-byte piece of the wave's 16 x 32 block of V or O:
    // row 16c + (lane >> 2), columns 8 (lane & 3) .. + 8
    const int xrow = 16 * cw + (lane >> 2), xcol = 8 * (lane & 3);
    const int xoff = xrow * rowb + xcol * 2;
    auto vo_rsrc = [&](const bf16_t* base, int c) {
        const int cc = (c >= c_beg && c < c_end) ? c : c_beg;
        return window(base + (size_t)(tb + (int64_t)cc * C) * row + hoff + j0, chunk_len(c) * rowb);
    };
    auto ld_frag = [&](__amdgpu_buffer_rsrc_t rt, int off) {
        return as_bf8(__builtin_amdgcn_raw_buffer_load_b128(rt, off, 0, 0));
    };

    if (wave < 4) {
        // ============================================================ chain
        f32x4 S[2][2];  // S[32c + 16a + 4q4 + e][16jb + r]
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 32 * cw + 16 * a + 4 * q4 + e, j = 16 * jb + r;
                    S[a][jb][e] = s_in ? s_in[sidx + (size_t)i * D + j0 + j] : 0.f;
                }
        auto load_a = [&](int c, ChainFrags& f) {  // K, beta, Gam, V
            const auto rt = tile_rsrc(c);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) f.K[kk] = ld_frag(rt, OFF_KT + ((cw * 4 + kk) * 64 + lane) * 16);
            const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rt, OFF_BETA + (16 * cw + 4 * q4) * 4, 0, 0);
            f.bet = make_float4(__uint_as_float(b[0]), __uint_as_float(b[1]), __uint_as_float(b[2]),
                                __uint_as_float(b[3]));
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                const u32x4 gg = __builtin_amdgcn_raw_buffer_load_b128(
                    rt, OFF_GAM + (32 * cw + 16 * a + 4 * q4) * 4, 0, 0);
                f.gam[a] = make_float4(__uint_as_float(gg[0]), __uint_as_float(gg[1]),
                                       __uint_as_float(gg[2]), __uint_as_float(gg[3]));
            }
            const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(vo_rsrc(v, c), xoff, 0, 0);
            f.v = make_uint4(x[0], x[1], x[2], x[3]);
        };
        auto load_b = [&](int c, ChainFrags& f) {  // Kb^T, T
            const auto rt = tile_rsrc(c);
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    f.Kb[a][kk] = ld_frag(rt, OFF_KBT + ((cw * 4 + a * 2 + kk) * 64 + lane) * 16);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) f.T[kk] = ld_frag(rt, OFF_T + ((cw * 2 + kk) * 64 + lane) * 16);
        };
        ChainFrags F0, F1, F2;
        load_a(c_beg, F0);
        load_b(c_beg, F0);
        load_a(c_beg + 1, F1);
        load_b(c_beg + 1, F1);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                S[a][jb][0] *= F0.gam[a].x; S[a][jb][1] *= F0.gam[a].y;
                S[a][jb][2] *= F0.gam[a].z; S[a][jb][3] *= F0.gam[a].w;
                st4(sm.Gt + (16 * jb + r) * LDK + 32 * cw + 16 * a + 4 * q4, S[a][jb]);
            }
        __syncthreads();
        auto step = [&](int c, const ChainFrags& cur, const ChainFrags& nxt, ChainFrags& later) {
            const bool more = c + 1 < c_end;
            // ---- Y = Kt G; R = diag(beta)(V - Y)
            // stage this wave's V rows (read back below by the same wave only)
            *reinterpret_cast<uint4*>(sm.V + xrow * LDX + xcol) = cur.v;
            __builtin_amdgcn_wave_barrier();
            load_a(c + 2, later);
            f32x4 Y[2] = {Z4, Z4};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                Y[0] = mma32(cur.K[kk], ld8(sm.Gt + r * LDK + 32 * kk + 8 * q4), Y[0]);
                Y[1] = mma32(cur.K[kk], ld8(sm.Gt + (16 + r) * LDK + 32 * kk + 8 * q4), Y[1]);
            }
            const float bb[4] = {cur.bet.x, cur.bet.y, cur.bet.z, cur.bet.w};
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                f32x4 rv;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    rv[e] = bb[e] * (bf16_bits_to_f32(sm.V[(16 * cw + 4 * q4 + e) * LDX + 16 * jb + r]) -
                                     Y[jb][e]);
                st4(sm.Rt + (16 * jb + r) * LDT + 16 * cw + 4 * q4, rv);
            }
            __syncthreads();
            // ---- U = T R
            load_b(c + 2, later);
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                f32x4 u = mma32(cur.T[0], ld8(sm.Rt + (16 * jb + r) * LDT + 8 * q4), Z4);
                if (cw >= 2) u = mma32(cur.T[1], ld8(sm.Rt + (16 * jb + r) * LDT + 32 + 8 * q4), u);
                st4(sm.Ut + (16 * jb + r) * LDT + 16 * cw + 4 * q4, u);
            }
            __syncthreads();
            // ---- S <- G + Kb^T U (a snapshot when one falls here); next G
            float* snp = snapshot_at(snap, n, h, H, D, (int64_t)(c + 1) * C, te - tb);
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                const bf16x8 u0 = ld8(sm.Ut + (16 * jb + r) * LDT + 8 * q4);
                const bf16x8 u1 = ld8(sm.Ut + (16 * jb + r) * LDT + 32 + 8 * q4);
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    f32x4 s = mma32(cur.Kb[a][1], u1, mma32(cur.Kb[a][0], u0, S[a][jb]));
                    if (snp) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            snp[(size_t)(32 * cw + 16 * a + 4 * q4 + e) * D + j0 + 16 * jb + r] = s[e];
                    }
                    if (more) {
                        s[0] *= nxt.gam[a].x; s[1] *= nxt.gam[a].y;
                        s[2] *= nxt.gam[a].z; s[3] *= nxt.gam[a].w;
                        st4(sm.Gt + (16 * jb + r) * LDK + 32 * cw + 16 * a + 4 * q4, s);
                    }
                    S[a][jb] = s;
                }
            }
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
        auto load_a = [&](int c, OutFrags& f) {  // Qt
            const auto rt = tile_rsrc(c);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) f.Q[kk] = ld_frag(rt, OFF_QT + ((cw * 4 + kk) * 64 + lane) * 16);
        };
        auto load_b = [&](int c, OutFrags& f) {  // P
            const auto rt = tile_rsrc(c);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) f.P[kk] = ld_frag(rt, OFF_P + ((cw * 2 + kk) * 64 + lane) * 16);
        };
        OutFrags F0, F1, F2;
        load_a(c_beg, F0);
        load_b(c_beg, F0);
        load_a(c_beg + 1, F1);
        load_b(c_beg + 1, F1);
        __syncthreads();
        auto step = [&](int c, const OutFrags& cur, OutFrags& later) {
            // ---- Z = Qt G
            f32x4 Zc[2] = {Z4, Z4};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                Zc[0] = mma32(cur.Q[kk], ld8(sm.Gt + r * LDK + 32 * kk + 8 * q4), Zc[0]);
                Zc[1] = mma32(cur.Q[kk], ld8(sm.Gt + (16 + r) * LDK + 32 * kk + 8 * q4), Zc[1]);
            }
            __syncthreads();
            __syncthreads();
            // ---- O = Z + P U, staged through this wave's rows, one 16-byte store
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                f32x4 acc = mma32(cur.P[0], ld8(sm.Ut + (16 * jb + r) * LDT + 8 * q4), Zc[jb]);
                if (cw >= 2) acc = mma32(cur.P[1], ld8(sm.Ut + (16 * jb + r) * LDT + 32 + 8 * q4), acc);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sm.O[(16 * cw + 4 * q4 + e) * LDX + 16 * jb + r] = f32_to_bf16_bits(acc[e]);
            }
            __builtin_amdgcn_wave_barrier();
            const uint4 x = *reinterpret_cast<const uint4*>(sm.O + xrow * LDX + xcol);
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{x.x, x.y, x.z, x.w}, vo_rsrc(o, c), xoff, 0, 0);
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

int prefill_split_window(int n_seqs, int H) {
    const size_t per_chunk = (size_t)n_seqs * H * TILE;
    const size_t w = TILE_BUDGET / per_chunk;
    return w < 1 ? 1 : (w > (size_t)MAX_WIN ? MAX_WIN : (int)w);
}

// State carry, then the tiles of one window.
size_t prefill_split_workspace_bytes(int n_seqs, int H) {
    return (size_t)n_seqs * H * D * D * 4 +
           (size_t)n_seqs * prefill_split_window(n_seqs, H) * H * TILE;
}

// Windows run one after the other on the caller's stream: operand kernel, then
// state pass.  (Running the operand kernel of the next window concurrently on a
// second stream was measured slower: both kernels then share the HBM bandwidth
// that the tile round trip already saturates.)
hipError_t launch_prefill_split(const void* q, const void* k, const void* v, const float* g,
                                const float* beta, bool g_head, const int32_t* cu, int n_seqs,
                                int64_t T, int H, int max_chunks, const float* s0,
                                float* s_final, void* o, Snapshots snap, void* workspace,
                                hipStream_t stream) {
    const int64_t n_pairs = (int64_t)n_seqs * H;
    if (n_pairs == 0) return hipSuccess;
    const int win = prefill_split_window(n_seqs, H);
    float* ws_state = reinterpret_cast<float*>(workspace);
    uint8_t* tiles = reinterpret_cast<uint8_t*>(workspace) + (size_t)n_pairs * D * D * 4;
    const int n_win = max_chunks > 0 ? (max_chunks + win - 1) / win : 1;
    for (int w = 0; w < n_win; ++w) {
        const int w0 = w * win;
        const int rows = max_chunks - w0 < win ? max_chunks - w0 : win;
        if (rows > 0) {
            hipLaunchKernelGGL(g_head ? prep_kernel<true> : prep_kernel<false>,
                               dim3((unsigned)n_pairs, (unsigned)rows), dim3(256), 0, stream,
                               (const bf16_t*)q, (const bf16_t*)k, g, beta, cu, T, H, w0, win,
                               tiles);
            hipError_t err = hipGetLastError();
            if (err != hipSuccess) return err;
        }
        hipLaunchKernelGGL(state_kernel, dim3((unsigned)(n_pairs * NS)), dim3(512), 0, stream,
                           (const bf16_t*)v, cu, T, H, (int)n_pairs, w0, win, tiles, ws_state, s0,
                           s_final, (bf16_t*)o, snap);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace kda
