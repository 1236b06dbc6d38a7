// KDA chunked prefill on gfx950 matrix cores: bf16 q/k/v, d_k = d_v = 128,
// chunk C = 64, fp32 state, bf16 MFMA operands with fp32 accumulation.
//
// The recurrence (page "Ling-3.1-flash: a 560B hybrid-attention MoE, counted from
// its safetensors headers", section "How KDA and MLA split the work"):
//   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
//   o_t = S_t^T q_t,  alpha_t = exp(g_t) per key channel, beta_t per head.
// It is evaluated chunk by chunk in the WY / UT-transform form (exact algebra,
// derived from the recurrence): with b_t the in-chunk cumulative sum of g_t,
//   Kt = K e^{b}, Kh = K e^{-b}, Qt = Q e^{b}, Kb = K e^{b_C - b}, Gam = e^{b_C}
//   N  = strict_lower(diag(beta) Kt Kh^T)             (MFMA)
//   T  = (I + N)^{-1}                                  (unit lower triangular)
//   P  = lower(Qt Kh^T)                                (MFMA)
//   U  = T diag(beta) (V - Kt S)                       (MFMA, S from the last chunk)
//   O  = Qt S + P U                                    (MFMA)
//   S <- Gam * S + Kb^T U                              (MFMA, fp32 accumulate)
//
// Mapping: one workgroup of 4 waves per (sequence, head, 32-column slice of the
// state).  Value columns evolve independently, so the four slices of a head never
// talk; each recomputes the chunk's decay factors, N, T and P, and the four
// workgroups of a head are placed on the same XCD so that q, k and g come from
// HBM once and from that XCD's L2 three times.  The fp32 state slice (128 x 32)
// lives in MFMA accumulator registers for the whole sequence; a bf16 copy in LDS
// feeds the products that read it.  The next chunk's q, k, g, v, beta are loaded
// into registers while the current chunk computes.
//
// T is built in fp32 on the diagonal 16 x 16 blocks (forward substitution, one
// lane per column) and completed with two levels of block products on bf16 MFMA:
//   T_10 = -T_11 N_10 T_00 (and T_32),  T_[2:4,0:2] = -T_hi N_[2:4,0:2] T_lo.
//
// MFMA operand layouts (gfx950, lane l, r = l % 16, q4 = l / 16):
//   16x16x32 bf16: A[r][8 q4 + e], B[8 q4 + e][r], D[4 q4 + e][r]
//   16x16x16 bf16: A[r][4 q4 + e], B[4 q4 + e][r], D[4 q4 + e][r]
// so a 16x16x16 result is already laid out as the B operand of the next one.
#include "kda_internal.h"

namespace kda {
namespace mf {

constexpr int D = 128, C = 64, DVS = 32, NS = D / DVS, NT = 256;
constexpr int LDK = 136;  // bf16 row stride of [64 or 32][128] tiles (272 B)
constexpr int LDT = 72;   // bf16 row stride of [*][64] tiles (144 B)
constexpr int LDN = 68;   // fp32 row stride of N [64][64]
constexpr int LDV = 68;   // fp32 row stride of V^T [32][64]
constexpr int LDO = 40;   // bf16 row stride of the output staging tile [64][32]

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
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return (uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16);
}
__device__ __forceinline__ s16x4 cvt4(float a, float b, float c, float d) {
    s16x4 r;
    r[0] = (short)f32_to_bf16_bits(a);
    r[1] = (short)f32_to_bf16_bits(b);
    r[2] = (short)f32_to_bf16_bits(c);
    r[3] = (short)f32_to_bf16_bits(d);
    return r;
}
__device__ __forceinline__ s16x4 cvt4(f32x4 x) { return cvt4(x[0], x[1], x[2], x[3]); }
__device__ __forceinline__ s16x4 cvt4n(f32x4 x) { return cvt4(-x[0], -x[1], -x[2], -x[3]); }
__device__ __forceinline__ s16x4 ld4f(const float* p) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    return cvt4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st4(uint16_t* p, f32x4 x) {
    uint2 v;
    v.x = pack2(x[0], x[1]);
    v.y = pack2(x[2], x[3]);
    *reinterpret_cast<uint2*>(p) = v;
}
// Order this wave's LDS traffic: everything before is visible to every lane of
// the wave after (single-wave phases, no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// acc += A[16 rows][32*NK] * Bt[16 rows][32*NK]^T, both row-major bf16 in LDS
// (contraction over the contiguous axis of both).
template <int NK>
__device__ __forceinline__ f32x4 mm(const uint16_t* A, int lda, const uint16_t* Bt, int ldb,
                                   f32x4 acc, int r, int q4) {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
        acc = mma32(ld8(A + r * lda + 32 * kk + 8 * q4), ld8(Bt + r * ldb + 32 * kk + 8 * q4),
                    acc);
    return acc;
}

struct Smem {
    uint16_t Kt[C * LDK];    // Kt = K e^{b}          [t][i]
    uint16_t Kh[C * LDK];    // Kh = K e^{-b}         [t][i]
    uint16_t Qt[C * LDK];    // Qt = Q e^{b}          [t][i]
    uint16_t KbT[D * LDT];   // Kb^T, Kb = K e^{b_C-b} [i][t]
    uint16_t T[C * LDT];     // T                      [t][s]
    uint16_t Tt[C * LDT];    // T^T                    [s][t]
    uint16_t P[C * LDT];     // P                      [t][s]
    uint16_t Rt[DVS * LDT];  // R^T, R = diag(beta)(V - Kt S)   [j][t]
    uint16_t Ut[DVS * LDT];  // U^T                    [j][t]
    uint16_t St[DVS * LDK];  // bf16 copy of the state slice, S^T [j][i]
    uint16_t O[C * LDO];     // output staging         [t][j]
    float N[C * LDN];        // N (fp32)               [t][s]
    float Vt[DVS * LDV];     // V^T slice (fp32)       [j][t]
    float Gam[D];
    float Beta[C];
};

}  // namespace mf

using namespace mf;

__global__ void __launch_bounds__(NT, 1)
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
    const size_t row = (size_t)H * D;  // stride between tokens
    const size_t hoff = (size_t)h * D;
    const size_t sidx = (size_t)pair * D * D;

    // ---- one-time set-up: zero the triangular tiles' upper parts
    for (int e = tid; e < C * LDT / 2; e += NT) {
        reinterpret_cast<uint32_t*>(sm.T)[e] = 0u;
        reinterpret_cast<uint32_t*>(sm.Tt)[e] = 0u;
        reinterpret_cast<uint32_t*>(sm.P)[e] = 0u;
    }

    // ---- state slice in registers: wave w owns rows [32w, 32w+32) x 32 columns,
    // as 4 tiles (ib = 2w + a, jb), lane holds S[16 ib + 4 q4 + e][16 jb + r]
    f32x4 S[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * (2 * wave + a) + 4 * q4 + e, j = 16 * jb + r;
                S[a][jb][e] = s0 ? s0[sidx + (size_t)i * D + j0 + j] : 0.f;
            }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
            st4(sm.St + (16 * jb + r) * LDK + 16 * (2 * wave + a) + 4 * q4, S[a][jb]);

    // ---- prefetch registers: lane (cg, tg) of wave w holds channels
    // [32w + 4cg, +4) of tokens [8tg, 8tg+8) of the chunk; v and beta separately.
    const int cg = lane & 7, tg = lane >> 3;
    const int ch0 = 32 * wave + 4 * cg;
    const int tv = tid >> 2, jv = 8 * (tid & 3);
    float4 pg[8];
    uint2 pk[8], pq[8];
    uint4 pv;
    float pb = 0.f;

    auto prefetch = [&](int64_t c0, int L) {
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            const int t = 8 * tg + rr;
            if (t < L) {
                const size_t off = (size_t)(c0 + t) * row + hoff + ch0;
                pg[rr] = *reinterpret_cast<const float4*>(g + off);
                pk[rr] = *reinterpret_cast<const uint2*>(k + off);
                pq[rr] = *reinterpret_cast<const uint2*>(q + off);
            } else {
                pg[rr] = make_float4(0.f, 0.f, 0.f, 0.f);
                pk[rr] = make_uint2(0u, 0u);
                pq[rr] = make_uint2(0u, 0u);
            }
        }
        if (tv < L)
            pv = *reinterpret_cast<const uint4*>(v + (size_t)(c0 + tv) * row + hoff + j0 + jv);
        else
            pv = make_uint4(0u, 0u, 0u, 0u);
        if (tid < 64) pb = tid < L ? beta[(size_t)(c0 + tid) * H + h] : 0.f;
    };

    if (tb < te) prefetch(tb, (int)((te - tb) < C ? (te - tb) : C));

    int64_t prev_c0 = -1;
    int prev_L = 0;
    // copy the staged output tile of the previous chunk to HBM (16 B per thread)
    auto flush_o = [&]() {
        if (prev_c0 >= 0 && tv < prev_L)
            *reinterpret_cast<uint4*>(o + (size_t)(prev_c0 + tv) * row + hoff + j0 + jv) =
                *reinterpret_cast<const uint4*>(sm.O + tv * LDO + jv);
    };

    for (int64_t c0 = tb; c0 < te; c0 += C) {
        const int L = (int)((te - c0) < C ? (te - c0) : C);

        // ---- A: cumulative decay and scaled operands, in registers
        float bcum[8][4];
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            bcum[rr][0] = (rr ? bcum[rr - 1][0] : 0.f) + pg[rr].x;
            bcum[rr][1] = (rr ? bcum[rr - 1][1] : 0.f) + pg[rr].y;
            bcum[rr][2] = (rr ? bcum[rr - 1][2] : 0.f) + pg[rr].z;
            bcum[rr][3] = (rr ? bcum[rr - 1][3] : 0.f) + pg[rr].w;
        }
        float gam[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float tot = bcum[7][e];
            float x = tot;
#pragma unroll
            for (int dd = 8; dd < 64; dd <<= 1) {
                const float y = __shfl_up(x, dd);
                if (lane >= dd) x += y;
            }
            const float excl = x - tot;
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) bcum[rr][e] += excl;
            gam[e] = __expf(__shfl(x, 56 + cg));
        }
        uint2 wkt[8], wkh[8], wqt[8];
        uint4 wkb[4];
        float kbv[4][8];
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            float kx[4], qx[4], kt[4], kh[4], qt[4];
            kx[0] = bf16_bits_to_f32(pk[rr].x & 0xffffu); kx[1] = bf16_bits_to_f32(pk[rr].x >> 16);
            kx[2] = bf16_bits_to_f32(pk[rr].y & 0xffffu); kx[3] = bf16_bits_to_f32(pk[rr].y >> 16);
            qx[0] = bf16_bits_to_f32(pq[rr].x & 0xffffu); qx[1] = bf16_bits_to_f32(pq[rr].x >> 16);
            qx[2] = bf16_bits_to_f32(pq[rr].y & 0xffffu); qx[3] = bf16_bits_to_f32(pq[rr].y >> 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float eb = __expf(bcum[rr][e]), ebi = __expf(-bcum[rr][e]);
                kt[e] = kx[e] * eb;
                kh[e] = kx[e] * ebi;
                qt[e] = qx[e] * eb;
                kbv[e][rr] = kx[e] * (ebi * gam[e]);
            }
            wkt[rr] = make_uint2(pack2(kt[0], kt[1]), pack2(kt[2], kt[3]));
            wkh[rr] = make_uint2(pack2(kh[0], kh[1]), pack2(kh[2], kh[3]));
            wqt[rr] = make_uint2(pack2(qt[0], qt[1]), pack2(qt[2], qt[3]));
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            wkb[e] = make_uint4(pack2(kbv[e][0], kbv[e][1]), pack2(kbv[e][2], kbv[e][3]),
                                pack2(kbv[e][4], kbv[e][5]), pack2(kbv[e][6], kbv[e][7]));
        float vf[8];
        vf[0] = bf16_bits_to_f32(pv.x & 0xffffu); vf[1] = bf16_bits_to_f32(pv.x >> 16);
        vf[2] = bf16_bits_to_f32(pv.y & 0xffffu); vf[3] = bf16_bits_to_f32(pv.y >> 16);
        vf[4] = bf16_bits_to_f32(pv.z & 0xffffu); vf[5] = bf16_bits_to_f32(pv.z >> 16);
        vf[6] = bf16_bits_to_f32(pv.w & 0xffffu); vf[7] = bf16_bits_to_f32(pv.w >> 16);
        const float bt_reg = pb;

        __syncthreads();  // previous chunk finished reading KbT, Gam and staging O
        flush_o();
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            const int t = 8 * tg + rr;
            *reinterpret_cast<uint2*>(sm.Kt + t * LDK + ch0) = wkt[rr];
            *reinterpret_cast<uint2*>(sm.Kh + t * LDK + ch0) = wkh[rr];
            *reinterpret_cast<uint2*>(sm.Qt + t * LDK + ch0) = wqt[rr];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            *reinterpret_cast<uint4*>(sm.KbT + (ch0 + e) * LDT + 8 * tg) = wkb[e];
        if (tg == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.Gam[ch0 + e] = gam[e];
        }
#pragma unroll
        for (int m = 0; m < 8; ++m) sm.Vt[(jv + m) * LDV + tv] = vf[m];
        if (tid < 64) sm.Beta[tid] = bt_reg;
        prev_c0 = c0;
        prev_L = L;
        if (c0 + C < te) prefetch(c0 + C, (int)((te - c0 - C) < C ? (te - c0 - C) : C));
        __syncthreads();

        // ---- B: N = strict_lower(diag(beta) Kt Kh^T), 10 tiles over 4 waves
        {
            // tiles (rb, cb) per wave: w0 {(0,0),(1,0),(1,1)}, w1 {(2,0),(2,1),(2,2)},
            // w2 {(3,0),(3,1)}, w3 {(3,2),(3,3)}
            const int cnt = wave < 2 ? 3 : 2;
            for (int ti = 0; ti < cnt; ++ti) {
                int rb, cb;
                if (wave == 0) { rb = ti == 0 ? 0 : 1; cb = ti == 2 ? 1 : 0; }
                else if (wave == 1) { rb = 2; cb = ti; }
                else if (wave == 2) { rb = 3; cb = ti; }
                else { rb = 3; cb = 2 + ti; }
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mm<4>(sm.Kt + 16 * rb * LDK, LDK, sm.Kh + 16 * cb * LDK, LDK, acc, r, q4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * rb + 4 * q4 + e, s = 16 * cb + r;
                    sm.N[t * LDN + s] = s < t ? sm.Beta[t] * acc[e] : 0.f;
                }
            }
        }
        __syncthreads();

        // ---- C: wave 0 builds T; waves 1-3 compute P, R = diag(beta)(V - Kt S), Z = Qt S
        f32x4 Z[3];
        if (wave == 0) {
            // (a) diagonal 16x16 blocks, fp32 forward substitution, lane = (block, column)
            {
                const int blk = lane >> 4, col = lane & 15;
                float x[16];
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    const float* nrow = sm.N + (16 * blk + t) * LDN + 16 * blk;
                    float acc = (t == col) ? 1.f : 0.f;
#pragma unroll
                    for (int s = 0; s < t; ++s) acc -= nrow[s] * x[s];
                    x[t] = acc;
                }
#pragma unroll
                for (int t = 0; t < 16; ++t)
                    sm.T[(16 * blk + t) * LDT + 16 * blk + col] = f32_to_bf16_bits(x[t]);
                uint4 w0, w1;
                w0 = make_uint4(pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]),
                                pack2(x[6], x[7]));
                w1 = make_uint4(pack2(x[8], x[9]), pack2(x[10], x[11]), pack2(x[12], x[13]),
                                pack2(x[14], x[15]));
                *reinterpret_cast<uint4*>(sm.Tt + (16 * blk + col) * LDT + 16 * blk) = w0;
                *reinterpret_cast<uint4*>(sm.Tt + (16 * blk + col) * LDT + 16 * blk + 8) = w1;
            }
            wave_lds_sync();
            // (b) T_{2p+1,2p} = -T_{2p+1,2p+1} N_{2p+1,2p} T_{2p,2p}, p = 0, 1
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int o0 = 32 * p;
                f32x4 X = {0.f, 0.f, 0.f, 0.f};
                X = mma16(ld4f(sm.N + (o0 + 16 + r) * LDN + o0 + 4 * q4),
                          ld4(sm.Tt + (o0 + r) * LDT + o0 + 4 * q4), X);
                f32x4 Y = {0.f, 0.f, 0.f, 0.f};
                Y = mma16(ld4(sm.T + (o0 + 16 + r) * LDT + o0 + 16 + 4 * q4), cvt4(X), Y);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sm.T[(o0 + 16 + 4 * q4 + e) * LDT + o0 + r] = f32_to_bf16_bits(-Y[e]);
                *reinterpret_cast<s16x4*>(sm.Tt + (o0 + r) * LDT + o0 + 16 + 4 * q4) = cvt4n(Y);
            }
            wave_lds_sync();
            // (c) T[32:64, 0:32] = -T_hi (N[32:64, 0:32] T_lo), 16-blocks a (rows), bb (cols)
            {
                f32x4 X[2][2];
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    const float* nr = sm.N + (32 + 16 * a + r) * LDN;
                    const s16x4 n0 = ld4f(nr + 4 * q4), n1 = ld4f(nr + 16 + 4 * q4);
                    f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
                    // X_a0 = N_{a,0} T_00 + N_{a,1} T_10 ; X_a1 = N_{a,1} T_11
                    x0 = mma16(n0, ld4(sm.Tt + r * LDT + 4 * q4), x0);
                    x0 = mma16(n1, ld4(sm.Tt + r * LDT + 16 + 4 * q4), x0);
                    x1 = mma16(n1, ld4(sm.Tt + (16 + r) * LDT + 16 + 4 * q4), x1);
                    X[a][0] = x0;
                    X[a][1] = x1;
                }
#pragma unroll
                for (int bb = 0; bb < 2; ++bb) {
                    const s16x4 xb0 = cvt4(X[0][bb]), xb1 = cvt4(X[1][bb]);
                    f32x4 y0 = {0.f, 0.f, 0.f, 0.f}, y1 = {0.f, 0.f, 0.f, 0.f};
                    // Y_0b = T_22 X_0b ; Y_1b = T_32 X_0b + T_33 X_1b
                    y0 = mma16(ld4(sm.T + (32 + r) * LDT + 32 + 4 * q4), xb0, y0);
                    y1 = mma16(ld4(sm.T + (48 + r) * LDT + 32 + 4 * q4), xb0, y1);
                    y1 = mma16(ld4(sm.T + (48 + r) * LDT + 48 + 4 * q4), xb1, y1);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        sm.T[(32 + 4 * q4 + e) * LDT + 16 * bb + r] = f32_to_bf16_bits(-y0[e]);
                        sm.T[(48 + 4 * q4 + e) * LDT + 16 * bb + r] = f32_to_bf16_bits(-y1[e]);
                    }
                    *reinterpret_cast<s16x4*>(sm.Tt + (16 * bb + r) * LDT + 32 + 4 * q4) =
                        cvt4n(y0);
                    *reinterpret_cast<s16x4*>(sm.Tt + (16 * bb + r) * LDT + 48 + 4 * q4) =
                        cvt4n(y1);
                }
            }
        } else {
            // Z/Y tiles (tb, jb): w1 {(0,0),(0,1),(1,0)}, w2 {(1,1),(2,0),(2,1)}, w3 {(3,0),(3,1)}
            const int w = wave - 1;
            const int nz = w < 2 ? 3 : 2;
#pragma unroll
            for (int zi = 0; zi < 3; ++zi) {
                if (zi < nz) {
                    const int idx = 3 * w + zi;  // 0..7 -> (tb, jb) = (idx / 2, idx % 2)
                    const int tbk = idx >> 1, jb = idx & 1;
                    f32x4 y = {0.f, 0.f, 0.f, 0.f}, z = {0.f, 0.f, 0.f, 0.f};
                    y = mm<4>(sm.Kt + 16 * tbk * LDK, LDK, sm.St + 16 * jb * LDK, LDK, y, r, q4);
                    z = mm<4>(sm.Qt + 16 * tbk * LDK, LDK, sm.St + 16 * jb * LDK, LDK, z, r, q4);
                    Z[zi] = z;
                    const int t0 = 16 * tbk + 4 * q4, j = 16 * jb + r;
                    const float4 vv = *reinterpret_cast<const float4*>(sm.Vt + j * LDV + t0);
                    const float4 bb = *reinterpret_cast<const float4*>(sm.Beta + t0);
                    f32x4 rv;
                    rv[0] = bb.x * (vv.x - y[0]);
                    rv[1] = bb.y * (vv.y - y[1]);
                    rv[2] = bb.z * (vv.z - y[2]);
                    rv[3] = bb.w * (vv.w - y[3]);
                    st4(sm.Rt + j * LDT + t0, rv);
                }
            }
            // P tiles: w1 {(0,0),(1,0),(1,1)}, w2 {(2,0),(2,1),(2,2)}, w3 {(3,0),...,(3,3)}
            const int np = w < 2 ? 3 : 4;
            for (int pi = 0; pi < np; ++pi) {
                int rb, cb;
                if (w == 0) { rb = pi == 0 ? 0 : 1; cb = pi == 2 ? 1 : 0; }
                else if (w == 1) { rb = 2; cb = pi; }
                else { rb = 3; cb = pi; }
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mm<4>(sm.Qt + 16 * rb * LDK, LDK, sm.Kh + 16 * cb * LDK, LDK, acc, r, q4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * rb + 4 * q4 + e, s = 16 * cb + r;
                    sm.P[t * LDT + s] = f32_to_bf16_bits(s <= t ? acc[e] : 0.f);
                }
            }
        }
        __syncthreads();

        // ---- D: U = T R, 8 tiles: w0 {(3,0),(3,1)}, w1 {(2,0),(2,1)}, w2 {(0,0),(1,0)},
        // w3 {(0,1),(1,1)}
#pragma unroll
        for (int ui = 0; ui < 2; ++ui) {
            int tbk, jb;
            if (wave == 0) { tbk = 3; jb = ui; }
            else if (wave == 1) { tbk = 2; jb = ui; }
            else if (wave == 2) { tbk = ui; jb = 0; }
            else { tbk = ui; jb = 1; }
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (tbk >= 2)
                acc = mm<2>(sm.T + 16 * tbk * LDT, LDT, sm.Rt + 16 * jb * LDT, LDT, acc, r, q4);
            else
                acc = mm<1>(sm.T + 16 * tbk * LDT, LDT, sm.Rt + 16 * jb * LDT, LDT, acc, r, q4);
            st4(sm.Ut + (16 * jb + r) * LDT + 16 * tbk + 4 * q4, acc);
        }
        __syncthreads();

        // ---- E: O = Z + P U (Z owners), S <- Gam S + Kb^T U (all waves)
        if (wave > 0) {
            const int w = wave - 1;
            const int nz = w < 2 ? 3 : 2;
#pragma unroll
            for (int zi = 0; zi < 3; ++zi) {
                if (zi < nz) {
                    const int idx = 3 * w + zi;
                    const int tbk = idx >> 1, jb = idx & 1;
                    f32x4 acc = Z[zi];
                    if (tbk >= 2)
                        acc = mm<2>(sm.P + 16 * tbk * LDT, LDT, sm.Ut + 16 * jb * LDT, LDT, acc,
                                    r, q4);
                    else
                        acc = mm<1>(sm.P + 16 * tbk * LDT, LDT, sm.Ut + 16 * jb * LDT, LDT, acc,
                                    r, q4);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sm.O[(16 * tbk + 4 * q4 + e) * LDO + 16 * jb + r] =
                            f32_to_bf16_bits(acc[e]);
                }
            }
        }
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const int ib = 2 * wave + a;
            const float4 gm = *reinterpret_cast<const float4*>(sm.Gam + 16 * ib + 4 * q4);
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                f32x4 acc = S[a][jb];
                acc[0] *= gm.x;
                acc[1] *= gm.y;
                acc[2] *= gm.z;
                acc[3] *= gm.w;
                acc = mm<2>(sm.KbT + 16 * ib * LDT, LDT, sm.Ut + 16 * jb * LDT, LDT, acc, r, q4);
                S[a][jb] = acc;
                st4(sm.St + (16 * jb + r) * LDK + 16 * ib + 4 * q4, acc);
            }
        }
    }
    __syncthreads();
    flush_o();
    if (s_final) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 16 * (2 * wave + a) + 4 * q4 + e, j = 16 * jb + r;
                    s_final[sidx + (size_t)i * D + j0 + j] = S[a][jb][e];
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
