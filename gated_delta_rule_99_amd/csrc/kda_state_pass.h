// Operand tiles and the pieces of the state pass of the two-kernel prefill
// (kda_prefill_split.hip), and the per-chunk steps the fused kernel
// (kda_prefill_fused.hip) shares with it.
//
// A tile holds everything the two-kernel state pass needs of one (sequence,
// head, chunk) that does not depend on the state, in the exact lane order of
// its MFMA operands, so that each lane reads one contiguous 16-byte fragment.
// T is folded into the operands that follow it: Wb^T = Kb^T T and PT = P T.
// Byte offsets:
//   0      Kt fragments    [row block c 0..3][kk 0..3][lane 64][16 B]
//   16384  Qt fragments    same
//   32768  Wb^T fragments  [c 0..3][a 0..1][kk 0..1][lane][16 B]   (rows 32c+16a)
//   49152  PT fragments    [c 0..3][kk 0..1][lane][16 B] (zero fragments skipped)
//   57344  beta[64] fp32, 57600 Gam[128] fp32
//
// State pass of one (sequence, head, 32-column slice of the state), 8 waves
// (recurrence from page "Ling-3.1-flash: a 560B hybrid-attention MoE, counted
// from its safetensors headers", section "How KDA and MLA split the work"):
// waves 0-3 carry the chain that the next chunk depends on, waves 4-7 produce
// the output off that chain.  Wave c of either group owns rows [16c, 16c+16) of
// the chunk and chain wave c owns state rows [32c, 32c+32) of the slice.
//   two-kernel path (chainw_*, outw_*; two barriers per chunk: R complete,
//   next G complete):
//     chain  Y = Kt G,  R = diag(beta)(V - Y),  S <- Gam S + Wb^T R,  G' = 2^R' S
//     output Z = Qt G,  O = Z + PT R
//   fused kernel (chain_*, out_*; three barriers: R, U, next G):
//     chain  Y = Kt G,  R = diag(beta)(V - Y),  U = T R,  S <- Gam S + Kb^T U
//     output Z = Qt G,  O = Z + P U
// with G = 2^R S the chunk's state operand in bf16 (2^R = max(Gam, 2^-RLIM),
// kda_chunk_ops.h) and Gam S kept in the fp32 accumulators.
// V and O move with one 16-byte access per lane (16 rows x 32 columns per wave)
// and are turned into the accumulator layout (lane (r, q4) holds rows 4q4 + e
// of column r) through a staging tile that only the wave itself touches.
#pragma once

#include "kda_chunk_ops.h"

namespace kda {
namespace co {

constexpr int DVS = 32, NS = D / DVS;  // state columns per workgroup, slices per head
constexpr int TILE = 58112;
constexpr int OFF_KT = 0, OFF_QT = 16384, OFF_WBT = 32768, OFF_PT = 49152, OFF_BETA = 57344,
              OFF_GAM = 57600;
static_assert(TILE % 256 == 0, "tiles stay 256-byte aligned");
constexpr int LDX = 40;  // row stride (bf16) of the V and O staging tiles

// ---------------------------------------------------------------- tile export
// Kt and Qt fragments out of LDS (wave p exports row block p); after the decay
// stage is visible.
template <typename L>
__device__ __forceinline__ void tile_export_kq(const L& sm, __amdgpu_buffer_rsrc_t rt, int p,
                                               int lane) {
    const int r = lane & 15, q4 = lane >> 4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 a = ld8(sm.Kt + (16 * p + r) * LDK + 32 * kk + 8 * q4);
        const bf16x8 b = ld8(sm.Qt + (16 * p + r) * LDK + 32 * kk + 8 * q4);
        __builtin_amdgcn_raw_buffer_store_b128(as_u4(a), rt, OFF_KT + ((p * 4 + kk) * 64 + lane) * 16,
                                               0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(as_u4(b), rt, OFF_QT + ((p * 4 + kk) * 64 + lane) * 16,
                                               0, 0);
    }
}

// ---------------------------------------------------------------- state pass
struct StateLds {
    uint16_t Gt[DVS * LDK];  // bf16 (2^R * S)^T [j][i]
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
    uint4 z;  // output gate: this lane's 16-byte piece of the gate projection
};

__device__ __forceinline__ bf16x8 ld_frag(__amdgpu_buffer_rsrc_t rt, int off) {
    return as_bf8(__builtin_amdgcn_raw_buffer_load_b128(rt, off, 0, 0));
}
__device__ __forceinline__ float4 ld_f4(__amdgpu_buffer_rsrc_t rt, int off) {
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rt, off, 0, 0);
    return make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]), __uint_as_float(x[2]),
                       __uint_as_float(x[3]));
}

// S[a][jb] holds S[32cw + 16a + 4q4 + e][16jb + r] of the slice.
typedef f32x4 StateFrag[2][2];

// The state operand of a chunk's products: G = 2^R * S, with 2^R = max(Gam,
// 2^-RLIM) the chunk's reference (kda_chunk_ops.h): Gam itself wherever the
// chunk decays by less than 2^-RLIM.
__device__ __forceinline__ float4 ref_of(const float4& gam) {
    constexpr float MIN_REF = 3.4694469519536142e-18f;  // 2^-RLIM
    return make_float4(fmaxf(gam.x, MIN_REF), fmaxf(gam.y, MIN_REF), fmaxf(gam.z, MIN_REF),
                       fmaxf(gam.w, MIN_REF));
}
__device__ __forceinline__ f32x4 scale4(f32x4 x, const float4& m) {
    return f32x4{x[0] * m.x, x[1] * m.y, x[2] * m.z, x[3] * m.w};
}

// The chunk's state operand G = 2^R * S in bf16 into Gt, and S *= Gam (per
// row): the accumulators then hold Gam * S, to which the chunk's update adds.
__device__ __forceinline__ void chain_scale_store(StateLds& sm, StateFrag& S, const float4 (&gam)[2],
                                                  int cw, int lane) {
    const int r = lane & 15, q4 = lane >> 4;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const float4 er = ref_of(gam[a]);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            st4(sm.Gt + (16 * jb + r) * LDK + 32 * cw + 16 * a + 4 * q4, scale4(S[a][jb], er));
            S[a][jb] = scale4(S[a][jb], gam[a]);
        }
    }
}

// Stage this wave's V rows (read back by the same wave only).
__device__ __forceinline__ void chain_stage_v(StateLds& sm, const uint4& v, int xrow, int xcol) {
    *reinterpret_cast<uint4*>(sm.V + xrow * LDX + xcol) = v;
    __builtin_amdgcn_wave_barrier();
}

// [A] Y = Kt G; R = diag(beta)(V - Y) into Rt.
template <typename Frags>
__device__ __forceinline__ void chain_yr(StateLds& sm, const Frags& cur, int cw, int lane) {
    const int r = lane & 15, q4 = lane >> 4;
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
}

// [B] U = T R into Ut.
__device__ __forceinline__ void chain_u(StateLds& sm, const ChainFrags& cur, int cw, int lane) {
    const int r = lane & 15, q4 = lane >> 4;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
        f32x4 u = mma32(cur.T[0], ld8(sm.Rt + (16 * jb + r) * LDT + 8 * q4), Z4);
        if (cw >= 2) u = mma32(cur.T[1], ld8(sm.Rt + (16 * jb + r) * LDT + 32 + 8 * q4), u);
        st4(sm.Ut + (16 * jb + r) * LDT + 16 * cw + 4 * q4, u);
    }
}

// [C] S <- Gam S + Kb^T U; the raw S to snp (a snapshot) when snp is set; with
// more, the next chunk's operand G' = 2^R' S into Gt and Gam' S into S.
__device__ __forceinline__ void chain_s(StateLds& sm, const ChainFrags& cur,
                                        const float4 (&gam_next)[2], bool more, StateFrag& S,
                                        float* snp, int j0, int cw, int lane) {
    const int r = lane & 15, q4 = lane >> 4;
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
                st4(sm.Gt + (16 * jb + r) * LDK + 32 * cw + 16 * a + 4 * q4,
                    scale4(s, ref_of(gam_next[a])));
                s = scale4(s, gam_next[a]);
            }
            S[a][jb] = s;
        }
    }
}

// [A] Z = Qt G.
__device__ __forceinline__ void out_z(StateLds& sm, const OutFrags& cur, f32x4 (&Zc)[2], int lane) {
    const int r = lane & 15, q4 = lane >> 4;
    Zc[0] = Z4;
    Zc[1] = Z4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        Zc[0] = mma32(cur.Q[kk], ld8(sm.Gt + r * LDK + 32 * kk + 8 * q4), Zc[0]);
        Zc[1] = mma32(cur.Q[kk], ld8(sm.Gt + (16 + r) * LDK + 32 * kk + 8 * q4), Zc[1]);
    }
}

// This wave's 16 output rows, fp32 in the accumulator layout (acc[jb][e]: row
// 16cw + 4q4 + e, column 16jb + r), to this lane's 16-byte piece of them (row
// xrow, columns xcol ..) in bf16, through the wave's rows of the staging tile.
// GATED: each output is first multiplied by sigmoid(z), the output gate, with z
// this lane's 16-byte piece of the gate projection (same rows and columns): z
// takes the same way through the staging rows into the accumulator layout, so
// that the gated value is rounded to bf16 once.  Only the wave itself touches
// these rows, and a wave's LDS accesses complete in order.
template <bool GATED>
__device__ __forceinline__ u32x4 stage_out(StateLds& sm, f32x4 (&acc)[2], const uint4& z, int cw,
                                           int lane, int xrow, int xcol) {
    const int r = lane & 15, q4 = lane >> 4;
    if constexpr (GATED) {
        *reinterpret_cast<uint4*>(sm.O + xrow * LDX + xcol) = z;
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc[jb][e] *= sigmoid_f(
                    bf16_bits_to_f32(sm.O[(16 * cw + 4 * q4 + e) * LDX + 16 * jb + r]));
        __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            sm.O[(16 * cw + 4 * q4 + e) * LDX + 16 * jb + r] = f32_to_bf16_bits(acc[jb][e]);
    __builtin_amdgcn_wave_barrier();
    const uint4 x = *reinterpret_cast<const uint4*>(sm.O + xrow * LDX + xcol);
    return u32x4{x.x, x.y, x.z, x.w};
}

// [C] O = Z + P U (gated by sigmoid(z) with GATED), staged through this wave's
// rows; returns this lane's 16-byte piece (row xrow, columns xcol ..) for one
// store.
template <bool GATED>
__device__ __forceinline__ u32x4 out_o(StateLds& sm, const OutFrags& cur, const f32x4 (&Zc)[2],
                                       const uint4& z, int cw, int lane, int xrow, int xcol) {
    const int r = lane & 15, q4 = lane >> 4;
    f32x4 acc[2];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
        acc[jb] = mma32(cur.P[0], ld8(sm.Ut + (16 * jb + r) * LDT + 8 * q4), Zc[jb]);
        if (cw >= 2) acc[jb] = mma32(cur.P[1], ld8(sm.Ut + (16 * jb + r) * LDT + 32 + 8 * q4), acc[jb]);
    }
    return stage_out<GATED>(sm, acc, z, cw, lane, xrow, xcol);
}

// ------------------------------------------------ two-kernel path, T folded in
// With U = T R:  S <- Gam S + Kb^T U = Gam S + Wb^T R  and  O = Z + P U = Z + PT R.  The
// chain then needs no U, and a chunk takes two barriers.
struct ChainFragsW {
    bf16x8 K[4], W[2][2];
    float4 bet, gam[2];
    uint4 v;  // V[16c + (lane >> 2)][8 (lane & 3) + 0..7]
};

// Kt, beta, Gam and this lane's piece of V (first half); Wb^T (second half).
__device__ __forceinline__ void chainw_load_a(ChainFragsW& f, __amdgpu_buffer_rsrc_t rt,
                                              __amdgpu_buffer_rsrc_t rv, int xoff, int cw,
                                              int lane) {
    const int q4 = lane >> 4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) f.K[kk] = ld_frag(rt, OFF_KT + ((cw * 4 + kk) * 64 + lane) * 16);
    f.bet = ld_f4(rt, OFF_BETA + (16 * cw + 4 * q4) * 4);
#pragma unroll
    for (int a = 0; a < 2; ++a) f.gam[a] = ld_f4(rt, OFF_GAM + (32 * cw + 16 * a + 4 * q4) * 4);
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rv, xoff, 0, 0);
    f.v = make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void chainw_load_b(ChainFragsW& f, __amdgpu_buffer_rsrc_t rt, int cw,
                                              int lane) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
            f.W[a][kk] = ld_frag(rt, OFF_WBT + ((cw * 4 + a * 2 + kk) * 64 + lane) * 16);
}
__device__ __forceinline__ void outw_load_a(OutFrags& f, __amdgpu_buffer_rsrc_t rt, int cw,
                                            int lane) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) f.Q[kk] = ld_frag(rt, OFF_QT + ((cw * 4 + kk) * 64 + lane) * 16);
}
__device__ __forceinline__ void outw_load_b(OutFrags& f, __amdgpu_buffer_rsrc_t rt, int cw,
                                            int lane) {
    f.P[0] = ld_frag(rt, OFF_PT + (cw * 2 * 64 + lane) * 16);
    if (cw >= 2) f.P[1] = ld_frag(rt, OFF_PT + ((cw * 2 + 1) * 64 + lane) * 16);  // else zero
}
// This lane's 16-byte piece of the chunk's gate projection (row xrow, columns
// xcol ..; a window of zero rows past the chunk).
__device__ __forceinline__ void out_load_z(OutFrags& f, __amdgpu_buffer_rsrc_t rz, int xoff) {
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rz, xoff, 0, 0);
    f.z = make_uint4(x[0], x[1], x[2], x[3]);
}

// [C] S <- Gam S + Wb^T R (R from Rt); the raw S to snp (a snapshot) when snp is
// set; with more, the next chunk's operand G' = 2^R' S into Gt and Gam' S into S.
__device__ __forceinline__ void chainw_s(StateLds& sm, const ChainFragsW& cur,
                                         const float4 (&gam_next)[2], bool more, StateFrag& S,
                                         float* snp, int j0, int cw, int lane) {
    const int r = lane & 15, q4 = lane >> 4;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
        const bf16x8 r0 = ld8(sm.Rt + (16 * jb + r) * LDT + 8 * q4);
        const bf16x8 r1 = ld8(sm.Rt + (16 * jb + r) * LDT + 32 + 8 * q4);
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            f32x4 s = mma32(cur.W[a][1], r1, mma32(cur.W[a][0], r0, S[a][jb]));
            if (snp) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    snp[(size_t)(32 * cw + 16 * a + 4 * q4 + e) * D + j0 + 16 * jb + r] = s[e];
            }
            if (more) {
                st4(sm.Gt + (16 * jb + r) * LDK + 32 * cw + 16 * a + 4 * q4,
                    scale4(s, ref_of(gam_next[a])));
                s = scale4(s, gam_next[a]);
            }
            S[a][jb] = s;
        }
    }
}

// [C] O = Z + PT R (gated by sigmoid(z) with GATED), staged through this
// wave's rows; returns this lane's 16-byte piece (row xrow, columns xcol ..)
// for one store.
template <bool GATED>
__device__ __forceinline__ u32x4 outw_o(StateLds& sm, const OutFrags& cur, const f32x4 (&Zc)[2],
                                        const uint4& z, int cw, int lane, int xrow, int xcol) {
    const int r = lane & 15, q4 = lane >> 4;
    f32x4 acc[2];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
        acc[jb] = mma32(cur.P[0], ld8(sm.Rt + (16 * jb + r) * LDT + 8 * q4), Zc[jb]);
        if (cw >= 2) acc[jb] = mma32(cur.P[1], ld8(sm.Rt + (16 * jb + r) * LDT + 32 + 8 * q4), acc[jb]);
    }
    return stage_out<GATED>(sm, acc, z, cw, lane, xrow, xcol);
}

}  // namespace co
}  // namespace kda
