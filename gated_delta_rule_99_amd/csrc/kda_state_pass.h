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
// State pass of one (sequence, head, DV-column slice of the state; DV = 32:
// four slices per head), 8 waves
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
// V and O move with DV / 32 16-byte accesses per lane (16 rows x DV columns per
// wave) and are turned into the accumulator layout (lane (r, q4) holds rows
// 4q4 + e of column r) through a staging tile that only the wave itself touches.
#pragma once

#include "kda_chunk_ops.h"

namespace kda {
namespace co {

constexpr int DVS = 32, NS = D / DVS;  // state columns per workgroup, slices per head
constexpr int TILE = 58112;
constexpr int OFF_KT = 0, OFF_QT = 16384, OFF_WBT = 32768, OFF_PT = 49152, OFF_BETA = 57344,
              OFF_GAM = 57600;
static_assert(TILE % 256 == 0, "tiles stay 256-byte aligned");

// This lane's 16-byte pieces of its wave's 16 x DV block of V or O (16 rows of
// the chunk, DV columns of the slice): piece u is row 16 cw + pi / (DV / 8),
// columns 8 (pi % (DV / 8)) .. + 8, with pi = lane + 64 u.
template <int DV>
struct VoPieces {
    static constexpr int N = DV / 32;
    int row[N], col[N];
    __device__ __forceinline__ VoPieces(int cw, int lane) {
#pragma unroll
        for (int u = 0; u < N; ++u) {
            const int pi = lane + 64 * u;
            row[u] = 16 * cw + pi / (DV / 8);
            col[u] = 8 * (pi % (DV / 8));
        }
    }
    // byte offset of piece u from the slice's first element of the chunk's first row
    __device__ __forceinline__ int off(int u, int rowb) const { return row[u] * rowb + col[u] * 2; }
};

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
template <int DV>
struct StateLdsT {
    static constexpr int LDX = DV + 8;   // row stride (bf16) of the V and O staging tiles
    static constexpr int LDXF = DV + 4;  // row stride (fp32) of the gated O staging tile
    uint16_t Gt[DV * LDK];  // bf16 (2^R * S)^T [j][i]
    uint16_t Rt[DV * LDT];  // R^T [j][t]
    uint16_t Ut[DV * LDT];  // U^T [j][t] (fused path)
    uint16_t V[C * LDX];    // V slice [t][j]: each chain wave stages its own 16 rows
    uint16_t O[C * LDX];    // O slice [t][j]: each output wave stages its own 16 rows
    float Of[C * LDXF];     // O slice in fp32, for the output gate (same rows)
};
using StateLds = StateLdsT<DVS>;

struct ChainFrags {
    bf16x8 K[4], Kb[2][2], T[2];
    float4 bet, gam[2];
    uint4 v[1];  // this lane's piece of V (VoPieces<32>)
};
template <int DV = DVS>
struct OutFragsT {
    bf16x8 Q[4], P[2];
    uint4 z[DV / 32];  // output gate: this lane's pieces of the gate projection
};
using OutFrags = OutFragsT<DVS>;

// S[a][jb] holds S[32cw + 16a + 4q4 + e][16jb + r] of the slice.
template <int DV>
using StateFragT = f32x4[2][DV / 16];
typedef StateFragT<DVS> StateFrag;

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
template <int DV>
__device__ __forceinline__ void chain_scale_store(StateLdsT<DV>& sm, StateFragT<DV>& S,
                                                  const float4 (&gam)[2], int cw, int lane) {
    const int r = lane & 15, q4 = lane >> 4;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const float4 er = ref_of(gam[a]);
#pragma unroll
        for (int jb = 0; jb < DV / 16; ++jb) {
            st4(sm.Gt + (16 * jb + r) * LDK + 32 * cw + 16 * a + 4 * q4, scale4(S[a][jb], er));
            S[a][jb] = scale4(S[a][jb], gam[a]);
        }
    }
}

// Stage this wave's V rows (read back by the same wave only).
template <int DV>
__device__ __forceinline__ void chain_stage_v(StateLdsT<DV>& sm, const uint4 (&v)[DV / 32],
                                              const VoPieces<DV>& vp) {
#pragma unroll
    for (int u = 0; u < DV / 32; ++u)
        *reinterpret_cast<uint4*>(sm.V + vp.row[u] * StateLdsT<DV>::LDX + vp.col[u]) = v[u];
    __builtin_amdgcn_wave_barrier();
}

// [A] Y = Kt G; R = diag(beta)(V - Y) into Rt.
template <int DV, typename Frags>
__device__ __forceinline__ void chain_yr(StateLdsT<DV>& sm, const Frags& cur, int cw, int lane) {
    constexpr int NJB = DV / 16, LDX = StateLdsT<DV>::LDX;
    const int r = lane & 15, q4 = lane >> 4;
    f32x4 Y[NJB];
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) Y[jb] = Z4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb)
            Y[jb] = mma32(cur.K[kk], ld8(sm.Gt + (16 * jb + r) * LDK + 32 * kk + 8 * q4), Y[jb]);
    const float bb[4] = {cur.bet.x, cur.bet.y, cur.bet.z, cur.bet.w};
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) {
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
template <int DV>
__device__ __forceinline__ void out_z(StateLdsT<DV>& sm, const OutFragsT<DV>& cur,
                                      f32x4 (&Zc)[DV / 16], int lane) {
    const int r = lane & 15, q4 = lane >> 4;
#pragma unroll
    for (int jb = 0; jb < DV / 16; ++jb) Zc[jb] = Z4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int jb = 0; jb < DV / 16; ++jb)
            Zc[jb] = mma32(cur.Q[kk], ld8(sm.Gt + (16 * jb + r) * LDK + 32 * kk + 8 * q4), Zc[jb]);
}

// This wave's 16 output rows, fp32 in the accumulator layout (acc[jb][e]: row
// 16cw + 4q4 + e, column 16jb + r), to this lane's 16-byte pieces of them
// (VoPieces) in bf16, through the wave's rows of a staging tile.  GATED: each
// output is multiplied by sigmoid(z), the output gate, z this lane's pieces of
// the gate projection (same rows and columns): the rows are staged in fp32,
// the gate applied in the piece layout (where z already is) and the product
// rounded to bf16 once.  Only the wave itself touches these rows, and a wave's
// LDS accesses complete in order.
template <bool GATED, int DV>
__device__ __forceinline__ void stage_out(StateLdsT<DV>& sm, f32x4 (&acc)[DV / 16],
                                          const uint4 (&z)[DV / 32], int cw, int lane,
                                          const VoPieces<DV>& vp, u32x4 (&out)[DV / 32]) {
    constexpr int NJB = DV / 16, LDX = StateLdsT<DV>::LDX, LDXF = StateLdsT<DV>::LDXF;
    const int r = lane & 15, q4 = lane >> 4;
    if constexpr (GATED) {
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sm.Of[(16 * cw + 4 * q4 + e) * LDXF + 16 * jb + r] = acc[jb][e];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int u = 0; u < DV / 32; ++u) {
            const float* row = sm.Of + vp.row[u] * LDXF + vp.col[u];
            const float4 a = *reinterpret_cast<const float4*>(row);
            const float4 b = *reinterpret_cast<const float4*>(row + 4);
            const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            const uint32_t zw[4] = {z[u].x, z[u].y, z[u].z, z[u].w};
#pragma unroll
            for (int w = 0; w < 4; ++w)
                out[u][w] = pack2(x[2 * w] * sigmoid_f(bf_lo(zw[w])),
                                  x[2 * w + 1] * sigmoid_f(bf_hi(zw[w])));
        }
    } else {
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sm.O[(16 * cw + 4 * q4 + e) * LDX + 16 * jb + r] = f32_to_bf16_bits(acc[jb][e]);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int u = 0; u < DV / 32; ++u) {
            const uint4 x = *reinterpret_cast<const uint4*>(sm.O + vp.row[u] * LDX + vp.col[u]);
            out[u] = u32x4{x.x, x.y, x.z, x.w};
        }
    }
}

// [C] O = Z + P U (gated by sigmoid(z) with GATED), staged through this wave's
// rows; this lane's 16-byte piece (VoPieces<32>) for one store into out.
template <bool GATED>
__device__ __forceinline__ void out_o(StateLds& sm, const OutFrags& cur, const f32x4 (&Zc)[2],
                                      const uint4 (&z)[1], int cw, int lane,
                                      const VoPieces<DVS>& vp, u32x4 (&out)[1]) {
    const int r = lane & 15, q4 = lane >> 4;
    f32x4 acc[2];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
        acc[jb] = mma32(cur.P[0], ld8(sm.Ut + (16 * jb + r) * LDT + 8 * q4), Zc[jb]);
        if (cw >= 2) acc[jb] = mma32(cur.P[1], ld8(sm.Ut + (16 * jb + r) * LDT + 32 + 8 * q4), acc[jb]);
    }
    stage_out<GATED, DVS>(sm, acc, z, cw, lane, vp, out);
}

// ------------------------------------------------ two-kernel path, T folded in
// With U = T R:  S <- Gam S + Kb^T U = Gam S + Wb^T R  and  O = Z + P U = Z + PT R.  The
// chain then needs no U, and a chunk takes two barriers.
template <int DV = DVS>
struct ChainFragsWT {
    bf16x8 K[4], W[2][2];
    float4 bet, gam[2];
    uint4 v[DV / 32];  // this lane's pieces of V (VoPieces<DV>)
};
using ChainFragsW = ChainFragsWT<DVS>;

// Kt, beta, Gam and this lane's pieces of V (first half); Wb^T (second half).
// AUX: the cache policy bits of the tile loads.
template <int DV, int AUX = 0>
__device__ __forceinline__ void chainw_load_a(ChainFragsWT<DV>& f, __amdgpu_buffer_rsrc_t rt,
                                              __amdgpu_buffer_rsrc_t rv, const VoPieces<DV>& vp,
                                              int rowb, int cw, int lane) {
    const int q4 = lane >> 4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        f.K[kk] = as_bf8(__builtin_amdgcn_raw_buffer_load_b128(
            rt, OFF_KT + ((cw * 4 + kk) * 64 + lane) * 16, 0, AUX));
    {
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rt, OFF_BETA + (16 * cw + 4 * q4) * 4,
                                                              0, AUX);
        f.bet = make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]), __uint_as_float(x[2]),
                            __uint_as_float(x[3]));
    }
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(
            rt, OFF_GAM + (32 * cw + 16 * a + 4 * q4) * 4, 0, AUX);
        f.gam[a] = make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]),
                               __uint_as_float(x[2]), __uint_as_float(x[3]));
    }
#pragma unroll
    for (int u = 0; u < DV / 32; ++u) {
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rv, vp.off(u, rowb), 0, 0);
        f.v[u] = make_uint4(x[0], x[1], x[2], x[3]);
    }
}
template <int DV, int AUX = 0>
__device__ __forceinline__ void chainw_load_b(ChainFragsWT<DV>& f, __amdgpu_buffer_rsrc_t rt,
                                              int cw, int lane) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
            f.W[a][kk] = as_bf8(__builtin_amdgcn_raw_buffer_load_b128(
                rt, OFF_WBT + ((cw * 4 + a * 2 + kk) * 64 + lane) * 16, 0, AUX));
}
template <int DV, int AUX = 0>
__device__ __forceinline__ void outw_load_a(OutFragsT<DV>& f, __amdgpu_buffer_rsrc_t rt, int cw,
                                            int lane) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        f.Q[kk] = as_bf8(__builtin_amdgcn_raw_buffer_load_b128(
            rt, OFF_QT + ((cw * 4 + kk) * 64 + lane) * 16, 0, AUX));
}
template <int DV, int AUX = 0>
__device__ __forceinline__ void outw_load_b(OutFragsT<DV>& f, __amdgpu_buffer_rsrc_t rt, int cw,
                                            int lane) {
    f.P[0] = as_bf8(__builtin_amdgcn_raw_buffer_load_b128(rt, OFF_PT + (cw * 2 * 64 + lane) * 16,
                                                          0, AUX));
    if (cw >= 2)  // else zero
        f.P[1] = as_bf8(__builtin_amdgcn_raw_buffer_load_b128(
            rt, OFF_PT + ((cw * 2 + 1) * 64 + lane) * 16, 0, AUX));
}
// This lane's 16-byte pieces of the chunk's gate projection (VoPieces; a window
// of zero rows past the chunk).
template <int DV>
__device__ __forceinline__ void out_load_z(OutFragsT<DV>& f, __amdgpu_buffer_rsrc_t rz,
                                           const VoPieces<DV>& vp, int rowb) {
#pragma unroll
    for (int u = 0; u < DV / 32; ++u) {
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rz, vp.off(u, rowb), 0, 0);
        f.z[u] = make_uint4(x[0], x[1], x[2], x[3]);
    }
}

// [C] S <- Gam S + Wb^T R (R from Rt); the raw S to snp (a snapshot) when snp is
// set; with more, the next chunk's operand G' = 2^R' S into Gt and Gam' S into S.
template <int DV>
__device__ __forceinline__ void chainw_s(StateLdsT<DV>& sm, const ChainFragsWT<DV>& cur,
                                         const float4 (&gam_next)[2], bool more,
                                         StateFragT<DV>& S, float* snp, int j0, int cw, int lane) {
    const int r = lane & 15, q4 = lane >> 4;
#pragma unroll
    for (int jb = 0; jb < DV / 16; ++jb) {
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
// wave's rows; this lane's 16-byte pieces (VoPieces) for the stores, into out.
template <bool GATED, int DV>
__device__ __forceinline__ void outw_o(StateLdsT<DV>& sm, const OutFragsT<DV>& cur,
                                       const f32x4 (&Zc)[DV / 16], int cw, int lane,
                                       const VoPieces<DV>& vp, u32x4 (&out)[DV / 32]) {
    const int r = lane & 15, q4 = lane >> 4;
    f32x4 acc[DV / 16];
#pragma unroll
    for (int jb = 0; jb < DV / 16; ++jb) {
        acc[jb] = mma32(cur.P[0], ld8(sm.Rt + (16 * jb + r) * LDT + 8 * q4), Zc[jb]);
        if (cw >= 2) acc[jb] = mma32(cur.P[1], ld8(sm.Rt + (16 * jb + r) * LDT + 32 + 8 * q4), acc[jb]);
    }
    stage_out<GATED, DV>(sm, acc, cur.z, cw, lane, vp, out);
}

}  // namespace co
}  // namespace kda
