// KDA chunked prefill, fused form for gfx950: bf16 q/k/v, d_k = d_v = 128,
// chunk C = 64, fp32 state, no workspace.  Same algebra as the two-kernel path
// (kda_prefill_split.hip; recurrence from page "Ling-3.1-flash: a 560B
// hybrid-attention MoE, counted from its safetensors headers", section "How
// KDA and MLA split the work"):
//   G = Gam * S,  U = T diag(beta)(V - Kt G),  O = Qt G + P U,  S <- G + Kb^T U.
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
// of the previous step.
//
//   step s:  [A] producer decay(s+1) | chain Y, R      | output Z
//            B1
//            [B] producer N(s+1)     | chain U          |
//            B2
//            [C] producer merge(s+1) | chain S, G(s+1)  | output O, store
//            B3
//            [D]                     | chain copy-in(s+1) | output copy-in(s+1)
//            B0
#include "kda_chunk_ops.h"

namespace kda {
namespace fu {

using namespace co;

constexpr int DVS = 32, NS = D / DVS;
constexpr int LDX = 40;  // row stride (bf16) of the V and O staging tiles

struct FusedLds {
    ChunkLds ck;              // operand stages of the next chunk
    uint16_t KbT[D * LDT];    // Kb^T [i][t] of the next chunk
    float gam[D];             // Gam of the next chunk
    uint16_t Gt[DVS * LDK];   // bf16 (Gam * S)^T [j][i]
    uint16_t Rt[DVS * LDT];   // R^T [j][t]
    uint16_t Ut[DVS * LDT];   // U^T [j][t]
    uint16_t V[C * LDX];      // V slice [t][j]: each chain wave stages its own 16 rows
    uint16_t O[C * LDX];      // O slice [t][j]: each output wave stages its own 16 rows
};

}  // namespace fu

using namespace fu;

// GH: g holds one log decay per (token, head) instead of one per key channel.
template <bool GH>
__global__ void __launch_bounds__(768)
prefill_fused_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                     const bf16_t* __restrict__ v, const float* __restrict__ g,
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
    const int xrow = 16 * w4 + (lane >> 2), xcol = 8 * (lane & 3);
    const int xoff = xrow * rowb + xcol * 2;
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
        ChunkIn in;
        load_chunk<GH>(in, q, k, g, beta, tb, chunk_len(0), H, h, p, lane);
        decay_stage(sm.ck, in, p, lane, gam_sink, kbt_sink);
        load_chunk<GH>(in, q, k, g, beta, tb + C, chunk_len(1), H, h, p, lane);
        __syncthreads();  // P1
        n_stage(sm.ck, p, lane);
        __syncthreads();  // P2
        merge_stage(sm.ck, p, lane);
        __syncthreads();  // P3
        __syncthreads();  // P4: copy-in of chunk 0 done
        for (int s = 0; s < nc; ++s) {
            const bool next = s + 1 < nc;
            if (next) decay_stage(sm.ck, in, p, lane, gam_sink, kbt_sink);
            load_chunk<GH>(in, q, k, g, beta, tb + (int64_t)(s + 2) * C, chunk_len(s + 2), H, h, p,
                           lane);
            __syncthreads();  // B1
            if (next) n_stage(sm.ck, p, lane);
            __syncthreads();  // B2
            if (next) merge_stage(sm.ck, p, lane);
            __syncthreads();  // B3
            __syncthreads();  // B0
        }
    } else if (wave < 8) {
        // ============================================================ chain
        const int cw = w4;
        f32x4 S[2][2];  // S[32cw + 16a + 4q4 + e][16jb + r]
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
        uint4 vcur = load_v(0), vnext = load_v(1);
        bf16x8 K[4], Kb[2][2], Tf[2];
        float4 bet;
        auto copy_in = [&]() {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) K[kk] = ld8(sm.ck.Kt + (16 * cw + r) * LDK + 32 * kk + 8 * q4);
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    Kb[a][kk] = ld8(sm.KbT + (32 * cw + 16 * a + r) * LDT + 32 * kk + 8 * q4);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) Tf[kk] = ld8(sm.ck.T + (16 * cw + r) * LDT + 32 * kk + 8 * q4);
            bet = *reinterpret_cast<const float4*>(sm.ck.beta + 16 * cw + 4 * q4);
        };
        __syncthreads();  // P1: Gam of chunk 0 is in LDS
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const float4 gm = *reinterpret_cast<const float4*>(sm.gam + 32 * cw + 16 * a + 4 * q4);
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                S[a][jb][0] *= gm.x; S[a][jb][1] *= gm.y; S[a][jb][2] *= gm.z; S[a][jb][3] *= gm.w;
                st4(sm.Gt + (16 * jb + r) * LDK + 32 * cw + 16 * a + 4 * q4, S[a][jb]);
            }
        }
        __syncthreads();  // P2
        __syncthreads();  // P3
        copy_in();
        __syncthreads();  // P4
        for (int s = 0; s < nc; ++s) {
            const bool next = s + 1 < nc;
            // ---- [A] Y = Kt G; R = diag(beta)(V - Y)
            *reinterpret_cast<uint4*>(sm.V + xrow * LDX + xcol) = vcur;
            __builtin_amdgcn_wave_barrier();
            f32x4 Y[2] = {Z4, Z4};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                Y[0] = mma32(K[kk], ld8(sm.Gt + r * LDK + 32 * kk + 8 * q4), Y[0]);
                Y[1] = mma32(K[kk], ld8(sm.Gt + (16 + r) * LDK + 32 * kk + 8 * q4), Y[1]);
            }
            const float bb[4] = {bet.x, bet.y, bet.z, bet.w};
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                f32x4 rv;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    rv[e] = bb[e] * (bf16_bits_to_f32(sm.V[(16 * cw + 4 * q4 + e) * LDX + 16 * jb + r]) -
                                     Y[jb][e]);
                st4(sm.Rt + (16 * jb + r) * LDT + 16 * cw + 4 * q4, rv);
            }
            vcur = vnext;
            vnext = load_v(s + 2);
            __syncthreads();  // B1
            // ---- [B] U = T R
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                f32x4 u = mma32(Tf[0], ld8(sm.Rt + (16 * jb + r) * LDT + 8 * q4), Z4);
                if (cw >= 2) u = mma32(Tf[1], ld8(sm.Rt + (16 * jb + r) * LDT + 32 + 8 * q4), u);
                st4(sm.Ut + (16 * jb + r) * LDT + 16 * cw + 4 * q4, u);
            }
            __syncthreads();  // B2
            // ---- [C] S <- G + Kb^T U (a snapshot when one falls here); next G = Gam(s+1) * S
            float* snp = snapshot_at(snap, n, h, H, D, (int64_t)(s + 1) * C, te - tb);
            float4 gm[2];
#pragma unroll
            for (int a = 0; a < 2; ++a)
                gm[a] = *reinterpret_cast<const float4*>(sm.gam + 32 * cw + 16 * a + 4 * q4);
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                const bf16x8 u0 = ld8(sm.Ut + (16 * jb + r) * LDT + 8 * q4);
                const bf16x8 u1 = ld8(sm.Ut + (16 * jb + r) * LDT + 32 + 8 * q4);
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    f32x4 st = mma32(Kb[a][1], u1, mma32(Kb[a][0], u0, S[a][jb]));
                    if (snp) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            snp[(size_t)(32 * cw + 16 * a + 4 * q4 + e) * D + j0 + 16 * jb + r] = st[e];
                    }
                    if (next) {
                        st[0] *= gm[a].x; st[1] *= gm[a].y; st[2] *= gm[a].z; st[3] *= gm[a].w;
                        st4(sm.Gt + (16 * jb + r) * LDK + 32 * cw + 16 * a + 4 * q4, st);
                    }
                    S[a][jb] = st;
                }
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
        bf16x8 Qf[4], Pf[2];
        auto copy_in = [&]() {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) Qf[kk] = ld8(sm.ck.Qt + (16 * cw + r) * LDK + 32 * kk + 8 * q4);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) Pf[kk] = ld8(sm.ck.P + (16 * cw + r) * LDT + 32 * kk + 8 * q4);
        };
        __syncthreads();  // P1
        __syncthreads();  // P2
        __syncthreads();  // P3
        copy_in();
        __syncthreads();  // P4
        for (int s = 0; s < nc; ++s) {
            const bool next = s + 1 < nc;
            // ---- [A] Z = Qt G
            f32x4 Zc[2] = {Z4, Z4};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                Zc[0] = mma32(Qf[kk], ld8(sm.Gt + r * LDK + 32 * kk + 8 * q4), Zc[0]);
                Zc[1] = mma32(Qf[kk], ld8(sm.Gt + (16 + r) * LDK + 32 * kk + 8 * q4), Zc[1]);
            }
            __syncthreads();  // B1
            __syncthreads();  // B2
            // ---- [C] O = Z + P U, staged through this wave's rows, one 16-byte store
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                f32x4 acc = mma32(Pf[0], ld8(sm.Ut + (16 * jb + r) * LDT + 8 * q4), Zc[jb]);
                if (cw >= 2) acc = mma32(Pf[1], ld8(sm.Ut + (16 * jb + r) * LDT + 32 + 8 * q4), acc);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sm.O[(16 * cw + 4 * q4 + e) * LDX + 16 * jb + r] = f32_to_bf16_bits(acc[e]);
            }
            __builtin_amdgcn_wave_barrier();
            const uint4 x = *reinterpret_cast<const uint4*>(sm.O + xrow * LDX + xcol);
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{x.x, x.y, x.z, x.w}, vo_rsrc(o, s), xoff, 0, 0);
            __syncthreads();  // B3
            // ---- [D] fragments of chunk s + 1
            if (next) copy_in();
            __syncthreads();  // B0
        }
    }
}

hipError_t launch_prefill_fused(const void* q, const void* k, const void* v, const float* g,
                                const float* beta, bool g_head, const int32_t* cu, int n_seqs,
                                int64_t T, int H, const float* s0, float* s_final, void* o,
                                Snapshots snap, hipStream_t stream) {
    const int64_t n_pairs = (int64_t)n_seqs * H;
    if (n_pairs == 0) return hipSuccess;
    hipLaunchKernelGGL(g_head ? prefill_fused_kernel<true> : prefill_fused_kernel<false>,
                       dim3((unsigned)(n_pairs * NS)), dim3(768), 0, stream, (const bf16_t*)q,
                       (const bf16_t*)k, (const bf16_t*)v, g, beta, cu, T, H, (int)n_pairs, s0,
                       s_final, (bf16_t*)o, snap);
    return hipGetLastError();
}

}  // namespace kda
