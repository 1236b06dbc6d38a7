// The operand tile of one (sequence, head, chunk) of the chunked prefill,
// formed by four waves: the body of the two-kernel path's operand kernel
// (kda_prefill_split.hip).  Recurrence from page "Ling-3.1-flash: a 560B
// hybrid-attention MoE, counted from its safetensors headers", section "How
// KDA and MLA split the work"; stages in kda_chunk_ops.h, tile layout in
// kda_state_pass.h.
#pragma once

#include "kda_state_pass.h"

namespace kda {
namespace co {

// LDS of one tile's four waves: the decay stage's Kt, Qt and Kb rows and beta.
// Once the N and P blocks are in registers, T, Tt and P take the place of Kt
// and Qt (TpLds), so that the four waves need 52.5 KB (three such workgroups
// fit a CU's 160 KB; with T, Tt and P beside the rows, 80 KB: two).  After the
// merge, T^T replaces Tt, the Kb^T rows (kept in registers since the decay
// stage) go after P, and Wb^T and PT are formed over the Kb^T rows and T.
struct PrepLds {
    uint16_t Kt[C * LDK];  // [t][i]
    uint16_t Qt[C * LDK];  // [t][i]
    uint16_t Kb[C * LDK];  // [t][i]
    float beta[C];
};
struct TpLds {
    uint16_t T[C * LDT];   // T [t][s], then PT [t][u]
    uint16_t Tt[C * LDT];  // T^T [s][t] on the diagonal blocks, N [t][s] below them;
                           // after the merge, all of T^T [u][s] (zero for s < u)
    uint16_t P[C * LDT];   // P [t][s]
    uint16_t Kbt[D * LDT]; // Kb^T [i][t], then Wb^T [i][u]
};
static_assert(sizeof(TpLds) <= sizeof(PrepLds), "the folded operands fit the stage rows");
static_assert(sizeof(PairLds) <= 3 * C * LDK * 2, "the pairwise path's rows fit the stage rows");

// The decay stage's sinks: Gam to the tile, the Kb^T pieces of channels
// ch0 .. ch0 + 3 (ch0 a multiple of 4) into registers.
struct PrepSinks {
    __amdgpu_buffer_rsrc_t rt;
    u32x4* kbt;
    __device__ __forceinline__ void operator()(int ch0, const float (&gam)[4]) const {
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{__float_as_uint(gam[0]), __float_as_uint(gam[1]), __float_as_uint(gam[2]),
                  __float_as_uint(gam[3])},
            rt, OFF_GAM + 4 * ch0, 0, 0);
    }
    __device__ __forceinline__ void operator()(int i, int tg, u32x4 piece) const {
        kbt[i & 3] = piece;
    }
};

// Runs the operand stages of the chunk whose first token is c0 (L tokens of
// it; rows past L read as zero) for head h, and writes its tile through rt.
// Wave p (0..3) of the four forms P's blocks 2, 2, 3, 3 of the ten in row order
// beside its N blocks, while Kt and Qt are still in LDS; after the merge, rows
// [32p, 32p + 32) of Wb^T = Kb^T T and row block p of PT = P T.
// Every barrier is a workgroup barrier: all waves of the workgroup call this
// together, NW of them in groups of four, each group on its own sm.  slow_flags
// [NW] in LDS gathers whether some wave's chunk decays too strongly for the
// factored products; then every group takes the pairwise path (exact for any
// decay), so that all groups pass the same barriers.  wave: this wave's index
// among the NW.
template <int GM, int NW>
__device__ __forceinline__ void prep_tile(PrepLds& sm, int* slow_flags, int wave,
                                          const bf16_t* __restrict__ q,
                                          const bf16_t* __restrict__ k, const Gate& g,
                                          const float* __restrict__ beta, int64_t c0, int L,
                                          int H, int h, __amdgpu_buffer_rsrc_t rt) {
    TpLds& tp = *reinterpret_cast<TpLds*>(sm.Kt);
    const int p = wave & 3, lane = threadIdx.x & 63;
    const int r = lane & 15, q4 = lane >> 4;

    ChunkIn in;
    load_chunk<GM>(in, q, k, g, beta, c0, L, H, h, p, lane);
    if (p == 0)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(chunk_beta<GM>(in, lane)), rt,
                                              OFF_BETA + 4 * lane, 0, 0);
    u32x4 kbt[4];  // Kb^T pieces: channel ch0 + e, tokens [8tg, 8tg + 8)
    const PrepSinks sinks{rt, kbt};
    const bool wave_slow = decay_stage<GM>(sm, in, p, lane, sinks, sinks);
    if (lane == 0) slow_flags[wave] = wave_slow;
    __syncthreads();
    bool slow = false;  // uniform over the workgroup
#pragma unroll
    for (int w = 0; w < NW; ++w) slow |= slow_flags[w] != 0;
    tile_export_kq(sm, rt, p, lane);
    const int pn = p_count(p), pk0 = p_first(p);
    NRegs nr;
    f32x4 pb[3];
    if (!slow) {
        n_regs(sm, p, lane, nr);
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            if (j >= pn) break;
            int rb, cb;
            lower_block(pk0 + j, rb, cb);
            pb[j] = p_tile(sm, rb, cb, lane);
        }
    } else {
        // some channel decays too strongly for the factored products: the
        // pairwise path over the reloaded inputs (the stage rows are reused)
        ChunkIn in2;
        load_chunk<GM>(in2, q, k, g, beta, c0, L, H, h, p, lane);
        NRaw nw;
        slow_products<GM>(*reinterpret_cast<PairLds*>(sm.Kt), in2, p, lane, nw, pb,
                          [] { __syncthreads(); });
        n_finish(sm.beta, p, lane, nw, nr);
    }
    __syncthreads();  // the stage rows are read in full: T, Tt, P and Kb^T take their place
    n_store(tp, p, lane, nr);
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        if (j >= pn) break;
        int rb, cb;
        lower_block(pk0 + j, rb, cb);
        p_store(tp, rb, cb, lane, pb[j]);
    }
    if (p == 0 || p == 2)  // P's upper blocks that PT's k-steps read: (0,1), (2,3)
        st4(tp.P + (16 * p + r) * LDT + 16 * (p + 1) + 4 * q4, Z4);
    {
        const int cg = lane & 7, tg = lane >> 3, ch0 = 32 * p + 4 * cg;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            *reinterpret_cast<u32x4*>(tp.Kbt + (ch0 + e) * LDT + 8 * tg) = kbt[e];
    }
    __syncthreads();
    if (p == 0) merge_t<true>(tp, lane);  // T's off-diagonal blocks; all of T^T in Tt
    __syncthreads();
    // Wb^T rows [32p, 32p + 32): Wb^T[i][u] = sum_{s >= u} Kb^T[i][s] T[s][u]
    // (computed transposed, so that a lane's 4 results lie along a row)
    f32x4 wacc[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int ub = 0; ub < 4; ++ub) {
            f32x4 acc = Z4;
#pragma unroll
            for (int kk = (ub >= 2 ? 1 : 0); kk < 2; ++kk)
                acc = mma32(ld8(tp.Tt + (16 * ub + r) * LDT + 32 * kk + 8 * q4),
                            ld8(tp.Kbt + (32 * p + 16 * a + r) * LDT + 32 * kk + 8 * q4), acc);
            wacc[a][ub] = acc;
        }
    // PT row block p: PT[t][u] = sum_{u <= s <= t} P[t][s] T[s][u]; the
    // exported blocks, (0,1) and (2,3) coming out zero
    const int nk = p >= 2 ? 2 : 1, nub = p >= 2 ? 4 : 2;
#pragma unroll
    for (int ub = 0; ub < 4; ++ub) {
        if (ub >= nub) break;
        f32x4 acc = Z4;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if (kk >= nk) break;
            acc = mma32(ld8(tp.Tt + (16 * ub + r) * LDT + 32 * kk + 8 * q4),
                        ld8(tp.P + (16 * p + r) * LDT + 32 * kk + 8 * q4), acc);
        }
        st4(tp.T + (16 * p + r) * LDT + 16 * ub + 4 * q4, acc);  // T is no longer read
    }
    // Wb^T over this wave's own Kb^T rows: every store needs an MFMA result
    // that has consumed the loads of the columns it overwrites (those of ub >= 2
    // write only columns that the loads they wait for cover), and LDS accesses
    // of one wave complete in order
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int ub = 0; ub < 4; ++ub)
            st4(tp.Kbt + (32 * p + 16 * a + r) * LDT + 16 * ub + 4 * q4, wacc[a][ub]);
    // the exports read what other lanes of this wave wrote
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // exports: Wb^T fragments [a][kk] of rows 32p + 16a, PT fragments of row block p
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
            __builtin_amdgcn_raw_buffer_store_b128(
                as_u4(ld8(tp.Kbt + (32 * p + 16 * a + r) * LDT + 32 * kk + 8 * q4)), rt,
                OFF_WBT + ((p * 4 + a * 2 + kk) * 64 + lane) * 16, 0, 0);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        if (kk >= nk) break;
        __builtin_amdgcn_raw_buffer_store_b128(
            as_u4(ld8(tp.T + (16 * p + r) * LDT + 32 * kk + 8 * q4)), rt,
            OFF_PT + ((p * 2 + kk) * 64 + lane) * 16, 0, 0);
    }
}

}  // namespace co
}  // namespace kda
