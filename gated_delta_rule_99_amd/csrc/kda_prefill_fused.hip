// KDA chunked prefill, fused form for gfx950: bf16 q/k/v, d_k = d_v = 128,
// chunk C = 64, fp32 state, no workspace.  Same algebra as the two-kernel path
// (kda_prefill_split.hip; recurrence from page "Ling-3.1-flash: a 560B
// hybrid-attention MoE, counted from its safetensors headers", section "How
// KDA and MLA split the work"):
//   G = 2^R S,  U = T diag(beta)(V - Kt G),  O = Qt G + P U,  S <- Gam S + Kbar^T U.
//
// One workgroup per (sequence, head, 32-column slice of the state), the four
// slices of a head on one XCD so that q, k, g come from HBM once and from L2
// three times: HBM traffic stays at the algorithmic bytes.  Twelve waves in
// three roles meet at four barriers per chunk:
//   waves 0-3  producer: the operand stages of chunk c + 1 (decay scaling, N and
//              T's diagonal blocks, T's merges and P) into LDS, while
//   waves 4-7  chain: Y = Kt G, R, U = T R, S <- G + Kb^T U, next G, and
//   waves 8-11 output: Z = Qt G, O = Z + P U
// run chunk c from register copies of its fragments, taken from LDS at the end
// of the previous step.  The chain and output steps are the state pass's own
// (kda_state_pass.h); only where their fragments come from differs.
//
//   step s:  [A] producer decay(s+1) | chain Y, R      | output Z
//            B1
//            [B] producer N(s+1)     | chain U          |
//                (a chunk on the pairwise path: PAIR_SYNCS more barriers here,
//                 which every wave takes; it also forms P here)
//            B2
//            [C] producer merge(s+1) | chain S, G(s+1)  | output O, store
//            B3
//            [D]                     | chain copy-in(s+1) | output copy-in(s+1)
//            B0
#include "kda_state_pass.h"

namespace kda {
namespace fu {

using namespace co;

struct FusedLds {
    ChunkLds ck;              // operand stages of the next chunk
    uint16_t KbT[D * LDT];    // Kbar^T [i][t] of the next chunk
    float gam[D];             // Gam of the next chunk
    int slow[4];              // per producer wave: the next chunk takes the pairwise path
    StateLds st;              // state pass (kda_state_pass.h)
};
// The pairwise path's rows sit over Kb, T, Tt and P: Kt and Qt stay for the
// copy-in of the chunk's fragments.
static_assert(sizeof(PairLds) <= sizeof(ChunkLds) - offsetof(ChunkLds, Kb) - sizeof(float) * C,
              "the pairwise path's rows fit over Kb, T, Tt and P");
// Barriers that a chunk on the pairwise path adds to the producer's N phase (four
// in slow_products and one before its results are stored); the other waves
// match them.
constexpr int PAIR_SYNCS = 5;

// The N phase of a chunk on the pairwise path (a chunk that decays below
// 2^-SLOW on some channel): N, T's diagonal blocks and P from the reloaded
// inputs of rows [c0, c0 + L), written to sm (PAIR_SYNCS barriers).  Kept out
// of line, with plain arguments and its results in LDS, so that its registers
// are saved around this rare call instead of squeezing the producer's loop.
template <int GM>
__device__ __attribute__((noinline)) void slow_n_phase(ChunkLds* sm, const bf16_t* q,
                                                       const bf16_t* k, Gate g,
                                                       const float* beta, int64_t c0, int L,
                                                       int H, int h, int p, int lane) {
    const int r = lane & 15, q4 = lane >> 4;
    ChunkIn in;
    load_chunk<GM>(in, q, k, g, beta, c0, L, H, h, p, lane);
    NRaw nw;
    f32x4 pb[3];
    slow_products<GM>(*reinterpret_cast<PairLds*>(sm->Kb), in, p, lane, nw, pb,
                      [] { __syncthreads(); });
    NRegs nr;
    n_finish(sm->beta, p, lane, nw, nr);
    __syncthreads();  // the pairwise rows are read in full
    n_store(*sm, p, lane, nr);
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        if (j >= p_count(p)) break;
        int rb, cb;
        lower_block(p_first(p) + j, rb, cb);
        p_store(*sm, rb, cb, lane, pb[j]);
    }
    if (p == 0 || p == 2) {  // T's and P's upper blocks the copy-in reads: (0,1), (2,3)
        st4(sm->T + (16 * p + r) * LDT + 16 * (p + 1) + 4 * q4, Z4);
        st4(sm->P + (16 * p + r) * LDT + 16 * (p + 1) + 4 * q4, Z4);
    }
}

}  // namespace fu

using namespace fu;

// GM: the decay inputs' GateMode (per channel, per head, or the projection).
// OG: the outputs are gated, O * sigmoid(z), z the gate projection zg (o's
// layout), read one chunk ahead by the output waves.
template <int GM, bool OG>
__global__ void __launch_bounds__(768)
prefill_fused_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                     const bf16_t* __restrict__ v, const bf16_t* __restrict__ zg, Gate g,
                     const float* __restrict__ beta, const int32_t* __restrict__ cu,
                     int64_t T, int H, int n_pairs, const float* __restrict__ s0,
                     float* __restrict__ s_final, bf16_t* __restrict__ o, Snapshots snap) {
    __shared__ __attribute__((aligned(16))) FusedLds sm;
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
    const int tid = threadIdx.x, wave = tid >> 6, w4 = wave & 3, lane = tid & 63;
    const int r = lane & 15, q4 = lane >> 4;
    const size_t sidx = (size_t)pair * D * D;

    if (nc == 0) {  // empty sequence: the final state is the initial one
        if (s_final)
            for (int e = tid; e < D * DVS; e += 768) {
                const size_t at = sidx + (size_t)(e / DVS) * D + j0 + e % DVS;
                s_final[at] = s0 ? s0[at] : 0.f;
            }
        return;
    }

    const size_t row = (size_t)H * D;
    const size_t hoff = (size_t)h * D;
    const int rowb = (int)(row * 2);
    auto chunk_len = [&](int c) -> int {  // 0 outside [0, nc)
        if (c < 0 || c >= nc) return 0;
        const int64_t rem = te - (tb + (int64_t)c * C);
        return rem < C ? (int)rem : C;
    };
    // this lane's 16-byte piece of a wave's 16 x 32 block of V or O
    const VoPieces<DVS> vp(w4, lane);
    const int xoff = vp.off(0, rowb);
    auto vo_rsrc = [&](const bf16_t* base, int c) {
        const int cc = (c >= 0 && c < nc) ? c : 0;
        return window(base + (size_t)(tb + (int64_t)cc * C) * row + hoff + j0, chunk_len(c) * rowb);
    };

    if (wave < 4) {
        // ============================================================ producer
        const int p = w4;
        zero_tp(sm.ck, tid, 256);
        auto gam_sink = [&](int ch0, const float(&gm)[4]) {
            *reinterpret_cast<float4*>(sm.gam + ch0) = make_float4(gm[0], gm[1], gm[2], gm[3]);
        };
        auto kbt_sink = [&](int i, int tg, u32x4 piece) {
            *reinterpret_cast<u32x4*>(sm.KbT + i * LDT + 8 * tg) = piece;
        };
        // [B] of chunk c: N (and T's diagonal blocks) on the matrix cores, or on
        // the pairwise path (then P too, and PAIR_SYNCS barriers)
        auto n_phase = [&](int c, bool slow) {
            if (!slow)
                n_stage(sm.ck, p, lane);
            else
                slow_n_phase<GM>(&sm.ck, q, k, g, beta, tb + (int64_t)c * C, chunk_len(c), H, h, p,
                                 lane);
        };
        auto slow_flag = [&]() { return sm.slow[0] | sm.slow[1] | sm.slow[2] | sm.slow[3]; };
        ChunkIn in;
        // the inputs of chunk c2, loaded while chunk c's N phase runs: before it
        // on the matrix-core path, after it on the pairwise path, which reloads
        // chunk c's own inputs (so that the two sets are never live together)
        auto n_phase_load = [&](int c, bool slow, int c2) {
            if (!slow) {
                load_chunk<GM>(in, q, k, g, beta, tb + (int64_t)c2 * C, chunk_len(c2), H, h, p,
                               lane);
                if (c < nc) n_phase(c, false);
            } else {
                n_phase(c, true);
                load_chunk<GM>(in, q, k, g, beta, tb + (int64_t)c2 * C, chunk_len(c2), H, h, p,
                               lane);
            }
        };
        load_chunk<GM>(in, q, k, g, beta, tb, chunk_len(0), H, h, p, lane);
        {
            const bool ws = decay_stage<GM>(sm.ck, in, p, lane, gam_sink, kbt_sink);
            if (lane == 0) sm.slow[p] = ws;
        }
        __syncthreads();  // P1
        bool slow = slow_flag();
        n_phase_load(0, slow, 1);
        __syncthreads();  // P2
        merge_stage(sm.ck, p, lane, !slow);
        __syncthreads();  // P3
        __syncthreads();  // P4: copy-in of chunk 0 done
        for (int s = 0; s < nc; ++s) {
            const bool next = s + 1 < nc;
            if (next) {
                const bool ws = decay_stage<GM>(sm.ck, in, p, lane, gam_sink, kbt_sink);
                if (lane == 0) sm.slow[p] = ws;
            }
            __syncthreads();  // B1
            slow = next && slow_flag();
            n_phase_load(next ? s + 1 : nc, slow, s + 2);
            __syncthreads();  // B2
            if (next) merge_stage(sm.ck, p, lane, !slow);
            __syncthreads();  // B3
            __syncthreads();  // B0
        }
    } else if (wave < 8) {
        // ============================================================ chain
        const int cw = w4;
        StateFrag S;
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 32 * cw + 16 * a + 4 * q4 + e, j = 16 * jb + r;
                    S[a][jb][e] = s0 ? s0[sidx + (size_t)i * D + j0 + j] : 0.f;
                }
        auto load_v = [&](int c) {
            const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(vo_rsrc(v, c), xoff, 0, 0);
            return make_uint4(x[0], x[1], x[2], x[3]);
        };
        uint4 vnext = load_v(1);
        ChainFrags cur;  // chunk s's fragments, copied from the producer's LDS
        cur.v[0] = load_v(0);
        auto gam_lds = [&](float4 (&gm)[2]) {
#pragma unroll
            for (int a = 0; a < 2; ++a)
                gm[a] = *reinterpret_cast<const float4*>(sm.gam + 32 * cw + 16 * a + 4 * q4);
        };
        auto copy_in = [&]() {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) cur.K[kk] = ld8(sm.ck.Kt + (16 * cw + r) * LDK + 32 * kk + 8 * q4);
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    cur.Kb[a][kk] = ld8(sm.KbT + (32 * cw + 16 * a + r) * LDT + 32 * kk + 8 * q4);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) cur.T[kk] = ld8(sm.ck.T + (16 * cw + r) * LDT + 32 * kk + 8 * q4);
            cur.bet = *reinterpret_cast<const float4*>(sm.ck.beta + 16 * cw + 4 * q4);
        };
        auto pair_syncs = [&](bool slow) {  // the producer's pairwise path, if taken
            if (slow)
                for (int i = 0; i < PAIR_SYNCS; ++i) __syncthreads();
        };
        auto slow_flag = [&]() { return sm.slow[0] | sm.slow[1] | sm.slow[2] | sm.slow[3]; };
        __syncthreads();  // P1: Gam of chunk 0 is in LDS
        {
            float4 gm[2];
            gam_lds(gm);
            chain_scale_store(sm.st, S, gm, cw, lane);
        }
        pair_syncs(slow_flag());
        __syncthreads();  // P2
        __syncthreads();  // P3
        copy_in();
        __syncthreads();  // P4
        for (int s = 0; s < nc; ++s) {
            const bool next = s + 1 < nc;
            // ---- [A] Y = Kt G; R = diag(beta)(V - Y)
            chain_stage_v(sm.st, cur.v, vp);
            chain_yr(sm.st, cur, cw, lane);
            cur.v[0] = vnext;
            vnext = load_v(s + 2);
            __syncthreads();  // B1
            const bool slow = next && slow_flag();
            // ---- [B] U = T R
            chain_u(sm.st, cur, cw, lane);
            pair_syncs(slow);
            __syncthreads();  // B2
            // ---- [C] S <- Gam S + Kbar^T U (a snapshot when one falls here); next operand
            {
                float4 gm[2];
                gam_lds(gm);
                chain_s(sm.st, cur, gm, next, S,
                        snapshot_at(snap, n, h, H, D, (int64_t)(s + 1) * C, te - tb), j0, cw, lane);
            }
            __syncthreads();  // B3
            // ---- [D] fragments of chunk s + 1
            if (next) copy_in();
            __syncthreads();  // B0
        }
        if (s_final) {
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 32 * cw + 16 * a + 4 * q4 + e, j = 16 * jb + r;
                        s_final[sidx + (size_t)i * D + j0 + j] = S[a][jb][e];
                    }
        }
    } else {
        // ============================================================ output
        const int cw = w4;
        OutFrags cur;  // chunk s's fragments, copied from the producer's LDS
        auto copy_in = [&]() {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) cur.Q[kk] = ld8(sm.ck.Qt + (16 * cw + r) * LDK + 32 * kk + 8 * q4);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) cur.P[kk] = ld8(sm.ck.P + (16 * cw + r) * LDT + 32 * kk + 8 * q4);
        };
        auto load_z = [&](int c) {
            uint4 z = make_uint4(0u, 0u, 0u, 0u);
            if constexpr (OG) {
                const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(vo_rsrc(zg, c), xoff, 0, 0);
                z = make_uint4(x[0], x[1], x[2], x[3]);
            }
            return z;
        };
        uint4 znext = load_z(0);
        auto pair_syncs = [&](bool slow) {  // the producer's pairwise path, if taken
            if (slow)
                for (int i = 0; i < PAIR_SYNCS; ++i) __syncthreads();
        };
        auto slow_flag = [&]() { return sm.slow[0] | sm.slow[1] | sm.slow[2] | sm.slow[3]; };
        __syncthreads();  // P1
        pair_syncs(slow_flag());
        __syncthreads();  // P2
        __syncthreads();  // P3
        copy_in();
        __syncthreads();  // P4
        for (int s = 0; s < nc; ++s) {
            const bool next = s + 1 < nc;
            const uint4 zc[1] = {znext};
            znext = load_z(s + 1);
            // ---- [A] Z = Qt G
            f32x4 Zc[2];
            out_z(sm.st, cur, Zc, lane);
            __syncthreads();  // B1
            pair_syncs(next && slow_flag());
            __syncthreads();  // B2
            // ---- [C] O = Z + P U (gated), staged through this wave's rows, one 16-byte store
            u32x4 out[1];
            out_o<OG>(sm.st, cur, Zc, zc, cw, lane, vp, out);
            __builtin_amdgcn_raw_buffer_store_b128(out[0], vo_rsrc(o, s), xoff, 0, 0);
            __syncthreads();  // B3
            // ---- [D] fragments of chunk s + 1
            if (next) copy_in();
            __syncthreads();  // B0
        }
    }
}

template <bool OG>
static hipError_t launch_fused_og(const void* q, const void* k, const void* v, Gate g,
                                  const float* beta, const int32_t* cu, int64_t n_pairs,
                                  int64_t T, int H, const float* s0, float* s_final,
                                  const void* out_gate, void* o, Snapshots snap,
                                  hipStream_t stream) {
    auto kern = g.mode == GATE_HEAD   ? prefill_fused_kernel<GATE_HEAD, OG>
                : g.mode == GATE_PROJ ? prefill_fused_kernel<GATE_PROJ, OG>
                                      : prefill_fused_kernel<GATE_CH, OG>;
    hipLaunchKernelGGL(kern, dim3((unsigned)(n_pairs * NS)), dim3(768), 0, stream, (const bf16_t*)q,
                       (const bf16_t*)k, (const bf16_t*)v, (const bf16_t*)out_gate, g, beta, cu,
                       T, H, (int)n_pairs, s0, s_final, (bf16_t*)o, snap);
    return hipGetLastError();
}

hipError_t launch_prefill_fused(const void* q, const void* k, const void* v, Gate g,
                                const float* beta, const int32_t* cu, int n_seqs,
                                int64_t T, int H, const float* s0, float* s_final,
                                const void* out_gate, void* o, Snapshots snap, hipStream_t stream) {
    const int64_t n_pairs = (int64_t)n_seqs * H;
    if (n_pairs == 0) return hipSuccess;
    if (out_gate)
        return launch_fused_og<true>(q, k, v, g, beta, cu, n_pairs, T, H, s0, s_final, out_gate, o,
                                     snap, stream);
    return launch_fused_og<false>(q, k, v, g, beta, cu, n_pairs, T, H, s0, s_final, nullptr, o,
                                  snap, stream);
}

}  // namespace kda
