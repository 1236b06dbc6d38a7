// KDA chunked prefill on gfx950 matrix cores: bf16 q/k/v, d_k = d_v = 128,
// chunk C = 64, fp32 state, bf16 MFMA operands with fp32 accumulation.
//
// The recurrence (page "Ling-3.1-flash: a 560B hybrid-attention MoE, counted from
// its safetensors headers", section "How KDA and MLA split the work"):
//   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
//   o_t = S_t^T q_t,  alpha_t = exp(g_t) per key channel, beta_t per head.
//
// Chunked (WY / UT-transform) form, exact algebra derived from the recurrence,
// with the decay referenced to the END of the chunk.  For a chunk of 64 tokens
// with per-channel decays alpha_t (padding tokens: alpha = 1, k = q = v = 0,
// beta = 0):
//   e^{b_t} = prod_{s<=t} alpha_s,  Gam = e^{b_63},
//   D_t = e^{b_t - b_63} (>= 1),    F_t = e^{b_63 - b_t} = prod_{s>t} alpha_s (<= 1)
//   Kt = K * D,  Qt = Q * D,  Kb = K * F                       (bf16 operands)
//   N  = strict_lower(diag(beta) Kt Kb^T)   (N_ts = beta_t k_t.k_s e^{b_t-b_s})
//   T  = (I + N)^{-1}                        (unit lower triangular)
//   P  = lower(Qt Kb^T)
//   G  = Gam * S                             (state rows scaled by the chunk decay)
//   U  = T diag(beta) (V - Kt G)
//   O  = Qt G + P U
//   S <- G + Kb^T U
// Only three scaled copies of the inputs are needed, each element of the decay
// comes from one exponential and running products (no exp(-b)), and every
// product stays in range as long as the chunk's log decay stays above ~-80.
//
// Workgroup = 8 waves for one (sequence, head, 32-column slice of the state).
// Value columns evolve independently, so the four slices of a head never talk.
//   waves 0-3 ("producer") prepare chunk i+1: decay products, Kt/Qt/Kb in LDS,
//             N, T and P with MFMA;
//   waves 4-7 ("state")    run chunk i's state pass: Y = Kt G, Z = Qt G, R, U,
//             O, S with MFMA; the fp32 state slice lives in their registers.
// Both groups meet at four workgroup barriers per chunk; between barriers they
// work on different chunks, so the producer's vector-ALU work overlaps the
// state pass's matrix-core work.  The four slices of a head are placed on one
// XCD so q, k and g come from HBM once and from that XCD's L2 three times.
//
// T's 16 x 16 diagonal blocks come from the nilpotent product form
//   (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8)
// evaluated in registers on 16x16x16 MFMA, and two levels of block merges
//   T_10 = -T_11 N_10 T_00,  T[32:64, 0:32] = -T_hi N[32:64, 0:32] T_lo.
// A product and its transpose are obtained by swapping the MFMA operands, so
// every operand is available in both lane layouts without an LDS transpose.
//
// MFMA operand layouts (gfx950, lane l, r = l % 16, q4 = l / 16):
//   16x16x32 bf16: A[r][8 q4 + e], B[8 q4 + e][r], D[4 q4 + e][r]
//   16x16x16 bf16: A[r][4 q4 + e], B[4 q4 + e][r], D[4 q4 + e][r]
#include "kda_internal.h"

namespace kda {
namespace mf {

constexpr int D = 128, C = 64, DVS = 32, NS = D / DVS, NT = 512;
constexpr int LDK = 136;  // bf16 row stride of [*][128] tiles (272 B)
constexpr int LDT = 72;   // bf16 row stride of [*][64] tiles (144 B)
constexpr int LDO = 40;   // bf16 row stride of the output staging tile [64][32]
constexpr int LDV = 68;   // fp32 row stride of the V^T tile [32][64]
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ s16x4 ld4(const uint16_t* p) {
    return *reinterpret_cast<const s16x4*>(p);
}
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// two floats -> two bf16 (RNE) in one register: a in the low half
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    const f32x2 x = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}
__device__ __forceinline__ s16x4 cvt4(f32x4 x) {
    const uint32_t lo = pack2(x[0], x[1]), hi = pack2(x[2], x[3]);
    s16x4 r;
    r[0] = (short)(lo & 0xffffu);
    r[1] = (short)(lo >> 16);
    r[2] = (short)(hi & 0xffffu);
    r[3] = (short)(hi >> 16);
    return r;
}
__device__ __forceinline__ f32x4 neg4(f32x4 x) { return f32x4{-x[0], -x[1], -x[2], -x[3]}; }
__device__ __forceinline__ void st4(uint16_t* p, f32x4 x) {
    uint2 v;
    v.x = pack2(x[0], x[1]);
    v.y = pack2(x[2], x[3]);
    *reinterpret_cast<uint2*>(p) = v;
}
__device__ __forceinline__ float bf_lo(uint32_t v) { return bf16_bits_to_f32(v & 0xffffu); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return bf16_bits_to_f32(v >> 16); }

constexpr f32x4 Z4 = {0.f, 0.f, 0.f, 0.f};

// Buffer resource for a window of global memory: loads past num_bytes return
// zero and stores past it are dropped, so rows past a chunk's end need no mask.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t window(const void* base, int num_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, num_bytes,
                                             0x00020000);
}
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));


struct Smem {
    uint16_t Kt[C * LDK];    // Kt = K * D        [t][i]
    uint16_t Qt[C * LDK];    // Qt = Q * D        [t][i]
    uint16_t Kb[C * LDK];    // Kb = K * F        [t][i]
    uint16_t KbT[D * LDT];   // Kb^T              [i][t]
    uint16_t T[C * LDT];     // T                 [t][s]
    uint16_t Tt[C * LDT];    // T^T               [s][t]
    uint16_t P[C * LDT];     // P                 [t][s]
    uint16_t N[C * LDT];     // N, off-diagonal 16x16 blocks   [t][s]
    uint16_t Gt[DVS * LDK];  // bf16 (Gam * S)^T  [j][i]
    uint16_t Rt[DVS * LDT];  // R^T               [j][t]
    uint16_t Ut[DVS * LDT];  // U^T               [j][t]
    uint16_t O[C * LDO];     // output staging    [t][j]
    float Vt[DVS * LDV];     // V^T slice (fp32) [j][t]
    float Gam[D];
    float Beta[C];
};

}  // namespace mf

using namespace mf;

__global__ void __launch_bounds__(NT)
prefill_mfma_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                    const bf16_t* __restrict__ v, const float* __restrict__ g,
                    const float* __restrict__ beta, const int32_t* __restrict__ cu, int64_t T,
                    int H, int n_pairs, const float* __restrict__ s0,
                    float* __restrict__ s_final, bf16_t* __restrict__ o) {
    __shared__ __attribute__((aligned(16))) Smem sm;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int r = lane & 15, q4 = lane >> 4;
    const bool producer = wave < 4;

    // XCD-aware placement: workgroup ids are dealt round-robin over 8 XCDs, so
    // the NS slices of one (sequence, head) pair take ids b, b+8, b+16, ...
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
    seq_range(cu, n, T, tb, te);
    const int nC = (int)((te - tb + C - 1) / C);
    const size_t row = (size_t)H * D;  // element stride between tokens
    const size_t hoff = (size_t)h * D;
    const size_t sidx = (size_t)pair * D * D;
    auto chunk_len = [&](int c) -> int {
        const int64_t rem = te - (tb + (int64_t)c * C);
        return rem < C ? (int)rem : C;
    };

    // ---- one-time set-up: the triangular tiles' upper blocks stay zero
    for (int e = tid; e < C * LDT / 2; e += NT) {
        reinterpret_cast<uint32_t*>(sm.T)[e] = 0u;
        reinterpret_cast<uint32_t*>(sm.Tt)[e] = 0u;
        reinterpret_cast<uint32_t*>(sm.P)[e] = 0u;
    }

    // ---- state waves: fp32 state slice in registers.  Wave 4+c owns rows
    // [32c, 32c+32) x 32 columns as tiles (a, jb); lane holds
    // S[32c + 16a + 4 q4 + e][16 jb + r].
    const int cw = wave - 4;  // state-wave index (valid for !producer)
    f32x4 S[2][2];
    if (!producer) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 32 * cw + 16 * a + 4 * q4 + e, j = 16 * jb + r;
                    S[a][jb][e] = s0 ? s0[sidx + (size_t)i * D + j0 + j] : 0.f;
                }
    }
    if (nC == 0) {  // empty sequence: the final state is the initial state
        if (!producer && s_final) {
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
        return;
    }

    if (producer) {
        // ================================================================ producer
        // Lane (cg, tg) of producer wave p handles channels [32p + 4cg, +4) of
        // tokens [8tg, 8tg + 8) of a chunk.  In iteration it it prepares chunk
        // it+1; segment by segment:
        //   0: decay products and scaled operands in registers
        //   1: scaled operands, Gam and beta to LDS; prefetch chunk it+2
        //   2: diagonal blocks of N and of T (product form), off-diagonal N
        //   3: wave 0 merges T's off-diagonal blocks, waves 1-3 compute P
        const int p = wave;
        const int cg = lane & 7, tg = lane >> 3;
        const int ch0 = 32 * p + 4 * cg;
        float4 pg[8];
        uint2 pk[8], pq[8];
        float pb = 0.f;
        // per-lane byte offsets inside a chunk window; the row step is scalar
        const int rowb2 = (int)(row * 2), rowb4 = (int)(row * 4);
        const int voff_kq = 8 * tg * rowb2 + ch0 * 2, voff_g = 8 * tg * rowb4 + ch0 * 4;
        auto prefetch = [&](int c) {
            const size_t c0 = (size_t)(tb + (int64_t)c * C) * row + hoff;
            const int L = chunk_len(c);
            const auto rg = window(g + c0, L * rowb4);
            const auto rk = window(k + c0, L * rowb2);
            const auto rq = window(q + c0, L * rowb2);
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
                const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rg, voff_g, rr * rowb4, 0);
                pg[rr] = make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]),
                                     __uint_as_float(x[2]), __uint_as_float(x[3]));
                const u32x2 y = __builtin_amdgcn_raw_buffer_load_b64(rk, voff_kq, rr * rowb2, 0);
                const u32x2 z = __builtin_amdgcn_raw_buffer_load_b64(rq, voff_kq, rr * rowb2, 0);
                pk[rr] = make_uint2(y[0], y[1]);
                pq[rr] = make_uint2(z[0], z[1]);
            }
            if (p == 0) {
                const auto rb = window(beta + (size_t)(tb + (int64_t)c * C) * H + h, L * H * 4);
                pb = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, lane * H * 4, 0, 0));
            }
        };
        prefetch(0);

        for (int it = -1; it < nC; ++it) {
            const bool work = it + 1 < nC;
            uint2 wkt[8], wqt[8], wkb[8];
            uint4 wkbt[4];
            float wgam[4];
            // ---------------------------------------------------- segment 0
            if (work) {
                // rows past the chunk's end were read as zero: alpha = 1, k = q = 0
                // alpha = exp(g), per element; thread totals over its 8 tokens
                float al[8][4], tot[4] = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
                for (int rr = 0; rr < 8; ++rr) {
                    al[rr][0] = __builtin_amdgcn_exp2f(pg[rr].x * LOG2E);
                    al[rr][1] = __builtin_amdgcn_exp2f(pg[rr].y * LOG2E);
                    al[rr][2] = __builtin_amdgcn_exp2f(pg[rr].z * LOG2E);
                    al[rr][3] = __builtin_amdgcn_exp2f(pg[rr].w * LOG2E);
#pragma unroll
                    for (int e = 0; e < 4; ++e) tot[e] *= al[rr][e];
                }
                // products over the other token groups (lanes cg + 8 tg'):
                // dsc = prod_{tg' < tg} / Gam,  fsc = prod_{tg' > tg}
                float dsc[4], fsc[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float xp = tot[e], xs = tot[e];
#pragma unroll
                    for (int dd = 8; dd < 64; dd <<= 1) {
                        const float yp = __shfl_up(xp, dd);
                        const float ys = __shfl_down(xs, dd);
                        if (lane >= dd) xp *= yp;
                        if (lane + dd < 64) xs *= ys;
                    }
                    const float epre = __shfl_up(xp, 8);
                    const float esuf = __shfl_down(xs, 8);
                    const float gam = __shfl(xp, 56 + cg);
                    wgam[e] = gam;
                    dsc[e] = (tg > 0 ? epre : 1.f) * __builtin_amdgcn_rcpf(gam);
                    fsc[e] = tg < 7 ? esuf : 1.f;
                }
                // forward: D_t = e^{b_t - b_63} -> Kt = K D, Qt = Q D
#pragma unroll
                for (int rr = 0; rr < 8; ++rr) {
                    float kt[4], qt[4];
                    const float kx[4] = {bf_lo(pk[rr].x), bf_hi(pk[rr].x), bf_lo(pk[rr].y),
                                         bf_hi(pk[rr].y)};
                    const float qx[4] = {bf_lo(pq[rr].x), bf_hi(pq[rr].x), bf_lo(pq[rr].y),
                                         bf_hi(pq[rr].y)};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        dsc[e] *= al[rr][e];
                        kt[e] = kx[e] * dsc[e];
                        qt[e] = qx[e] * dsc[e];
                    }
                    wkt[rr] = make_uint2(pack2(kt[0], kt[1]), pack2(kt[2], kt[3]));
                    wqt[rr] = make_uint2(pack2(qt[0], qt[1]), pack2(qt[2], qt[3]));
                }
                // backward: F_t = e^{b_63 - b_t} -> Kb = K F (row-major and transposed)
                float kb4[4][8];
#pragma unroll
                for (int rr = 7; rr >= 0; --rr) {
                    const float kx[4] = {bf_lo(pk[rr].x), bf_hi(pk[rr].x), bf_lo(pk[rr].y),
                                         bf_hi(pk[rr].y)};
                    float kb[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        kb[e] = kx[e] * fsc[e];
                        kb4[e][rr] = kb[e];
                        fsc[e] *= al[rr][e];
                    }
                    wkb[rr] = make_uint2(pack2(kb[0], kb[1]), pack2(kb[2], kb[3]));
                }
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    wkbt[e] = make_uint4(pack2(kb4[e][0], kb4[e][1]), pack2(kb4[e][2], kb4[e][3]),
                                         pack2(kb4[e][4], kb4[e][5]), pack2(kb4[e][6], kb4[e][7]));
            }
            __syncthreads();
            // ---------------------------------------------------- segment 1
            if (work) {
#pragma unroll
                for (int rr = 0; rr < 8; ++rr) {
                    const int t = 8 * tg + rr;
                    const int a = t * LDK + ch0;
                    *reinterpret_cast<uint2*>(sm.Kt + a) = wkt[rr];
                    *reinterpret_cast<uint2*>(sm.Qt + a) = wqt[rr];
                    *reinterpret_cast<uint2*>(sm.Kb + a) = wkb[rr];
                }
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    *reinterpret_cast<uint4*>(sm.KbT + (ch0 + e) * LDT + 8 * tg) = wkbt[e];
                if (tg == 0) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) sm.Gam[ch0 + e] = wgam[e];
                }
                if (p == 0) sm.Beta[lane] = pb;
                if (it + 2 < nC) prefetch(it + 2);
            }
            __syncthreads();
            // ---------------------------------------------------- segment 2
            if (work) {
                // diagonal block p of N in both lane layouts, from Kt and Kb
                f32x4 acc1 = Z4, acc2 = Z4;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const bf16x8 xt = ld8(sm.Kt + (16 * p + r) * LDK + 32 * kk + 8 * q4);
                    const bf16x8 xb = ld8(sm.Kb + (16 * p + r) * LDK + 32 * kk + 8 * q4);
                    acc1 = mma32(xt, xb, acc1);  // [4q4+e][r]  (B layout)
                    acc2 = mma32(xb, xt, acc2);  // [r][4q4+e]  (A layout)
                }
                const float4 b4 = *reinterpret_cast<const float4*>(sm.Beta + 16 * p + 4 * q4);
                const float bw[4] = {b4.x, b4.y, b4.z, b4.w};
                const float br = sm.Beta[16 * p + r];
                f32x4 Nb, Na, X0b, X0a;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int rowb = 4 * q4 + e;
                    Nb[e] = rowb > r ? bw[e] * acc1[e] : 0.f;
                    Na[e] = r > rowb ? br * acc2[e] : 0.f;
                    X0b[e] = (rowb == r ? 1.f : 0.f) - Nb[e];
                    X0a[e] = (rowb == r ? 1.f : 0.f) - Na[e];
                }
                // (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8), both layouts
                const s16x4 na = cvt4(Na), nb = cvt4(Nb);
                const f32x4 N2b = mma16(na, nb, Z4), N2a = mma16(nb, na, Z4);
                const s16x4 n2a = cvt4(N2a), n2b = cvt4(N2b);
                const f32x4 N4b = mma16(n2a, n2b, Z4), N4a = mma16(n2b, n2a, Z4);
                const s16x4 x0a = cvt4(X0a);
                const f32x4 X1b = mma16(x0a, n2b, X0b), X1a = mma16(n2b, x0a, X0a);
                const s16x4 n4a = cvt4(N4a), n4b = cvt4(N4b);
                const f32x4 N8b = mma16(n4a, n4b, Z4);
                const s16x4 x1a = cvt4(X1a);
                const f32x4 X2b = mma16(x1a, n4b, X1b), X2a = mma16(n4b, x1a, X1a);
                const s16x4 n8b = cvt4(N8b), x2a = cvt4(X2a);
                const f32x4 Tb = mma16(x2a, n8b, X2b), Ta = mma16(n8b, x2a, X2a);
                st4(sm.T + (16 * p + r) * LDT + 16 * p + 4 * q4, Ta);   // T[16p + r][16p + 4q4 + e]
                st4(sm.Tt + (16 * p + r) * LDT + 16 * p + 4 * q4, Tb);  // T^T rows
                // off-diagonal blocks of N (row-major, bf16): computed transposed so
                // each lane holds 4 consecutive columns of one row
                auto offdiag = [&](int rb, int cb) {
                    f32x4 acc = Z4;
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        acc = mma32(ld8(sm.Kb + (16 * cb + r) * LDK + 32 * kk + 8 * q4),
                                    ld8(sm.Kt + (16 * rb + r) * LDK + 32 * kk + 8 * q4), acc);
                    const float bt = sm.Beta[16 * rb + r];
                    acc[0] *= bt; acc[1] *= bt; acc[2] *= bt; acc[3] *= bt;
                    st4(sm.N + (16 * rb + r) * LDT + 16 * cb + 4 * q4, acc);
                };
                if (p == 0) { offdiag(1, 0); offdiag(2, 0); }
                else if (p == 1) { offdiag(2, 1); offdiag(3, 0); }
                else if (p == 2) { offdiag(3, 1); }
                else { offdiag(3, 2); }
            }
            __syncthreads();
            // ---------------------------------------------------- segment 3
            if (work) {
                if (p == 0) {
                    // level 32: T_10 = -T_11 N_10 T_00 and T_32 = -T_33 N_32 T_22
                    s16x4 bT10 = {0, 0, 0, 0}, aT32 = {0, 0, 0, 0};
#pragma unroll
                    for (int p2 = 0; p2 < 2; ++p2) {
                        const int o0 = 32 * p2;
                        const s16x4 aN = ld4(sm.N + (o0 + 16 + r) * LDT + o0 + 4 * q4);
                        const s16x4 bTlo = ld4(sm.Tt + (o0 + r) * LDT + o0 + 4 * q4);
                        const s16x4 aThi = ld4(sm.T + (o0 + 16 + r) * LDT + o0 + 16 + 4 * q4);
                        const f32x4 X = mma16(aN, bTlo, Z4);
                        const s16x4 xb = cvt4(X);
                        const f32x4 Yb = neg4(mma16(aThi, xb, Z4));  // T block, B layout
                        const f32x4 Ya = neg4(mma16(xb, aThi, Z4));  // T block, A layout
                        st4(sm.T + (o0 + 16 + r) * LDT + o0 + 4 * q4, Ya);
                        st4(sm.Tt + (o0 + r) * LDT + o0 + 16 + 4 * q4, Yb);
                        if (p2 == 0) bT10 = cvt4(Yb);
                        else aT32 = cvt4(Ya);
                    }
                    // level 64: T[32:64, 0:32] = -T_hi (N[32:64, 0:32] T_lo)
                    const s16x4 bT00 = ld4(sm.Tt + r * LDT + 4 * q4);
                    const s16x4 bT11 = ld4(sm.Tt + (16 + r) * LDT + 16 + 4 * q4);
                    const s16x4 aT22 = ld4(sm.T + (32 + r) * LDT + 32 + 4 * q4);
                    const s16x4 aT33 = ld4(sm.T + (48 + r) * LDT + 48 + 4 * q4);
                    s16x4 xm[2][2];
#pragma unroll
                    for (int a = 0; a < 2; ++a) {
                        const s16x4 n0 = ld4(sm.N + (32 + 16 * a + r) * LDT + 4 * q4);
                        const s16x4 n1 = ld4(sm.N + (32 + 16 * a + r) * LDT + 16 + 4 * q4);
                        xm[a][0] = cvt4(mma16(n1, bT10, mma16(n0, bT00, Z4)));
                        xm[a][1] = cvt4(mma16(n1, bT11, Z4));
                    }
#pragma unroll
                    for (int bb = 0; bb < 2; ++bb) {
                        const f32x4 y0 = mma16(xm[0][bb], aT22, Z4);
                        const f32x4 y1 = mma16(xm[1][bb], aT33, mma16(xm[0][bb], aT32, Z4));
                        st4(sm.T + (32 + r) * LDT + 16 * bb + 4 * q4, neg4(y0));
                        st4(sm.T + (48 + r) * LDT + 16 * bb + 4 * q4, neg4(y1));
                    }
                } else {
                    // P tiles, lower incl. diagonal, computed transposed (row-major out)
                    auto ptile = [&](int rb, int cb) {
                        f32x4 acc = Z4;
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk)
                            acc = mma32(ld8(sm.Kb + (16 * cb + r) * LDK + 32 * kk + 8 * q4),
                                        ld8(sm.Qt + (16 * rb + r) * LDK + 32 * kk + 8 * q4), acc);
                        if (rb == cb) {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (4 * q4 + e > r) acc[e] = 0.f;
                        }
                        st4(sm.P + (16 * rb + r) * LDT + 16 * cb + 4 * q4, acc);
                    };
                    if (p == 1) { ptile(0, 0); ptile(1, 0); ptile(1, 1); }
                    else if (p == 2) { ptile(2, 0); ptile(2, 1); ptile(2, 2); }
                    else { ptile(3, 0); ptile(3, 1); ptile(3, 2); ptile(3, 3); }
                }
            }
            __syncthreads();
        }
    } else {
        // ================================================================ state pass
        // Wave 4+c owns output/U rows [16c, 16c+16) and state rows [32c, 32c+32).
        // In iteration it it runs chunk it; segment by segment:
        //   0: flush chunk it-1's output; chunk it's operands into registers
        //   1: Y = Kt G, Z = Qt G; R = diag(beta)(V - Y) to LDS
        //   2: U = T R to LDS  (iteration -1: G_0 = Gam_0 * S_0)
        //   3: O = Z + P U staged; S <- G + Kb^T U; next G to LDS
        const int cw = wave - 4;
        bf16x8 aK[4], aQ[4], aKb[2][2], aT[2], aP[2];
        float4 bet = make_float4(0.f, 0.f, 0.f, 0.f);
        f32x4 Zc[2] = {Z4, Z4};
        // V slice of a chunk: thread st = tid - 256 loads row st >> 2, columns
        // 8 (st & 3) .. +8 as one 16-byte vector; unpacked into LDS one segment later
        const int st = tid - 256, vrow = st >> 2, vcol = 8 * (st & 3);
        uint4 vraw = make_uint4(0u, 0u, 0u, 0u);
        const int rowb = (int)(row * 2), voff_v = vrow * rowb + vcol * 2;
        auto load_v = [&](int c) {
            const auto rv = window(v + (size_t)(tb + (int64_t)c * C) * row + hoff + j0,
                                   chunk_len(c) * rowb);
            const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rv, voff_v, 0, 0);
            vraw = make_uint4(x[0], x[1], x[2], x[3]);
        };
        auto flush_o = [&](int c) {  // staged output tile of chunk c -> HBM, 16 B per thread
            const auto ro = window(o + (size_t)(tb + (int64_t)c * C) * row + hoff + j0,
                                   chunk_len(c) * rowb);
            const uint4 x = *reinterpret_cast<const uint4*>(sm.O + vrow * LDO + vcol);
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{x.x, x.y, x.z, x.w}, ro, voff_v, 0, 0);
        };
        load_v(0);

        for (int it = -1; it < nC; ++it) {
            const bool work = it >= 0;
            // ---------------------------------------------------- segment 0
            if (work) {
                if (it > 0) flush_o(it - 1);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    aK[kk] = ld8(sm.Kt + (16 * cw + r) * LDK + 32 * kk + 8 * q4);
                    aQ[kk] = ld8(sm.Qt + (16 * cw + r) * LDK + 32 * kk + 8 * q4);
                }
#pragma unroll
                for (int a = 0; a < 2; ++a)
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
                        aKb[a][kk] = ld8(sm.KbT + (32 * cw + 16 * a + r) * LDT + 32 * kk + 8 * q4);
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    aT[kk] = ld8(sm.T + (16 * cw + r) * LDT + 32 * kk + 8 * q4);
                    aP[kk] = ld8(sm.P + (16 * cw + r) * LDT + 32 * kk + 8 * q4);
                }
                bet = *reinterpret_cast<const float4*>(sm.Beta + 16 * cw + 4 * q4);
                {
                    const uint32_t w4[4] = {vraw.x, vraw.y, vraw.z, vraw.w};
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        sm.Vt[(vcol + 2 * m) * LDV + vrow] = bf_lo(w4[m]);
                        sm.Vt[(vcol + 2 * m + 1) * LDV + vrow] = bf_hi(w4[m]);
                    }
                }
            }
            __syncthreads();
            // ---------------------------------------------------- segment 1
            if (work) {
                f32x4 Y[2] = {Z4, Z4};
                Zc[0] = Zc[1] = Z4;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const bf16x8 b0 = ld8(sm.Gt + r * LDK + 32 * kk + 8 * q4);
                    const bf16x8 b1 = ld8(sm.Gt + (16 + r) * LDK + 32 * kk + 8 * q4);
                    Y[0] = mma32(aK[kk], b0, Y[0]);
                    Y[1] = mma32(aK[kk], b1, Y[1]);
                    Zc[0] = mma32(aQ[kk], b0, Zc[0]);
                    Zc[1] = mma32(aQ[kk], b1, Zc[1]);
                }
                const float bb[4] = {bet.x, bet.y, bet.z, bet.w};
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) {
                    const float4 vv = *reinterpret_cast<const float4*>(
                        sm.Vt + (16 * jb + r) * LDV + 16 * cw + 4 * q4);
                    const float vx[4] = {vv.x, vv.y, vv.z, vv.w};
                    f32x4 rv;
#pragma unroll
                    for (int e = 0; e < 4; ++e) rv[e] = bb[e] * (vx[e] - Y[jb][e]);
                    st4(sm.Rt + (16 * jb + r) * LDT + 16 * cw + 4 * q4, rv);
                }
                if (it + 1 < nC) load_v(it + 1);
            }
            __syncthreads();
            // ---------------------------------------------------- segment 2
            if (work) {
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) {
                    f32x4 u = mma32(aT[0], ld8(sm.Rt + (16 * jb + r) * LDT + 8 * q4), Z4);
                    if (cw >= 2)
                        u = mma32(aT[1], ld8(sm.Rt + (16 * jb + r) * LDT + 32 + 8 * q4), u);
                    st4(sm.Ut + (16 * jb + r) * LDT + 16 * cw + 4 * q4, u);
                }
            } else {
                // G_0 = Gam_0 * S_0 (Gam_0 was written in segment 1)
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    const float4 gm =
                        *reinterpret_cast<const float4*>(sm.Gam + 32 * cw + 16 * a + 4 * q4);
#pragma unroll
                    for (int jb = 0; jb < 2; ++jb) {
                        S[a][jb][0] *= gm.x; S[a][jb][1] *= gm.y;
                        S[a][jb][2] *= gm.z; S[a][jb][3] *= gm.w;
                        st4(sm.Gt + (16 * jb + r) * LDK + 32 * cw + 16 * a + 4 * q4, S[a][jb]);
                    }
                }
            }
            __syncthreads();
            // ---------------------------------------------------- segment 3
            if (work) {
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) {
                    f32x4 acc = mma32(aP[0], ld8(sm.Ut + (16 * jb + r) * LDT + 8 * q4), Zc[jb]);
                    if (cw >= 2)
                        acc = mma32(aP[1], ld8(sm.Ut + (16 * jb + r) * LDT + 32 + 8 * q4), acc);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sm.O[(16 * cw + 4 * q4 + e) * LDO + 16 * jb + r] = f32_to_bf16_bits(acc[e]);
                }
                // S <- G + Kb^T U ; then G for the next chunk = Gam_next * S
                const bool last = it + 1 >= nC;
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    float4 gm = make_float4(1.f, 1.f, 1.f, 1.f);
                    if (!last)
                        gm = *reinterpret_cast<const float4*>(sm.Gam + 32 * cw + 16 * a + 4 * q4);
#pragma unroll
                    for (int jb = 0; jb < 2; ++jb) {
                        const bf16x8 u0 = ld8(sm.Ut + (16 * jb + r) * LDT + 8 * q4);
                        const bf16x8 u1 = ld8(sm.Ut + (16 * jb + r) * LDT + 32 + 8 * q4);
                        f32x4 s = mma32(aKb[a][1], u1, mma32(aKb[a][0], u0, S[a][jb]));
                        if (!last) {
                            s[0] *= gm.x; s[1] *= gm.y; s[2] *= gm.z; s[3] *= gm.w;
                            st4(sm.Gt + (16 * jb + r) * LDK + 32 * cw + 16 * a + 4 * q4, s);
                        }
                        S[a][jb] = s;
                    }
                }
            }
            __syncthreads();
        }

        flush_o(nC - 1);
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
    }
}

hipError_t launch_prefill_mfma(const void* q, const void* k, const void* v, const float* g,
                               const float* beta, const int32_t* cu, int n_seqs, int64_t T,
                               int H, const float* s0, float* s_final, void* o,
                               hipStream_t stream) {
    const int64_t n_pairs = (int64_t)n_seqs * H;
    const int64_t blocks = n_pairs * NS;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(prefill_mfma_kernel, dim3((unsigned)blocks), dim3(NT), 0, stream,
                       (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, g, beta, cu, T, H,
                       (int)n_pairs, s0, s_final, (bf16_t*)o);
    return hipGetLastError();
}

}  // namespace kda
