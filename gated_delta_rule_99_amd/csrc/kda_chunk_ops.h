// Per-chunk operand stages of the matrix-core prefill (bf16, d_k = d_v = 128,
// chunk C = 64), shared by the chunk-parallel operand kernel of the two-kernel
// path and by the producer waves of the fused kernel.
//
// Recurrence from page "Ling-3.1-flash: a 560B hybrid-attention MoE, counted
// from its safetensors headers", section "How KDA and MLA split the work".  B
// is the in-chunk cumulative log2 decay (B_t = sum over tokens u <= t of log2
// alpha_u, per key channel) and B_C its value at the chunk's end.  Every
// channel gets a reference R = max(B_C, -RLIM): the scaled operands
//   Kt = K * 2^{B - R},  Qt = Q * 2^{B - R},  Kb = K * 2^{R - B},
//   Kbar = K * 2^{B_C - B}  (<= 1),   Gam = 2^{B_C},
// give N = strict_lower(diag(beta) Kt Kb^T), T = (I + N)^{-1},
// P = lower(Qt Kb^T), and with G = 2^R * S the state products Kt G, Qt G.
// R = B_C (the chunk's end) wherever the chunk decays by less than 2^-RLIM;
// the clamp keeps Kt and Qt below 2^RLIM and 2^R * S representable however
// strong the decay.  Kt Kb^T factors e^{b_t - b_s} exactly when both factors
// stay in range, which holds while B_C >= -SLOW on every channel; a chunk with
// a stronger decay takes the pairwise path (slow_products), which forms N and
// P from 2^{B_t - B_s} directly.  The state pass recovers 2^R as
// max(Gam, 2^-RLIM).
// Four waves (p = 0..3) run each stage; callers place the barriers between
// stages.  MFMA operand layouts (gfx950, lane l, r = l % 16, q4 = l / 16):
//   16x16x32 bf16: A[r][8 q4 + e], B[8 q4 + e][r], D[4 q4 + e][r]
//   16x16x16 bf16: A[r][4 q4 + e], B[4 q4 + e][r], D[4 q4 + e][r]
#pragma once

#include "kda_internal.h"

namespace kda {
namespace co {

constexpr int D = 128, C = 64;
constexpr int LDK = 136, LDT = 72;  // LDS row strides (bf16) of the C x D and C x C tiles
constexpr float LOG2E = 1.4426950408889634f;
// log2 bounds of the scaled operands: the reference R >= -RLIM, and the
// factored products hold while every channel's chunk decay B_C >= -SLOW
// (Kt <= 2^RLIM, Kb <= 2^(SLOW - RLIM) = 2^102, both far inside fp32 and bf16).
constexpr float RLIM = 58.f, SLOW = 160.f;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr f32x4 Z4 = {0.f, 0.f, 0.f, 0.f};

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
    *reinterpret_cast<uint2*>(p) = make_uint2(pack2(x[0], x[1]), pack2(x[2], x[3]));
}
__device__ __forceinline__ float bf_lo(uint32_t v) { return bf16_bits_to_f32(v & 0xffffu); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return bf16_bits_to_f32(v >> 16); }
__device__ __forceinline__ bf16x8 as_bf8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ u32x4 as_u4(bf16x8 x) { return __builtin_bit_cast(u32x4, x); }

// Sequence n's token range (clamped to [0, T)) and chunk count.
__device__ __forceinline__ void seq_chunks(const int32_t* cu, int n, int64_t T, int64_t& tb,
                                           int64_t& te, int& nc) {
    seq_range(cu, n, T, tb, te);
    nc = (int)((te - tb + C - 1) / C);
}

// LDS of the operand stages.
struct ChunkLds {
    uint16_t Kt[C * LDK];  // [t][i]
    uint16_t Qt[C * LDK];  // [t][i]
    uint16_t Kb[C * LDK];  // [t][i]
    uint16_t T[C * LDT];   // T [t][s]; upper blocks stay zero
    uint16_t Tt[C * LDT];  // T^T [s][t] on the diagonal blocks, N [t][s] below them
    uint16_t P[C * LDT];   // P [t][s]; upper blocks stay zero
    float beta[C];
};

// Zero T and P once: only their diagonal and lower blocks are ever written.
__device__ __forceinline__ void zero_tp(ChunkLds& sm, int tid, int nthreads) {
    for (int e = tid; e < C * LDT / 2; e += nthreads) {
        reinterpret_cast<uint32_t*>(sm.T)[e] = 0u;
        reinterpret_cast<uint32_t*>(sm.P)[e] = 0u;
    }
}

// One lane's inputs of a chunk: channels [32p + 4cg, +4) of tokens [8tg, 8tg+8).
struct ChunkIn {
    float4 g[8];
    uint2 f[8];   // GATE_PROJ: the decay projection (bf16 pairs) in place of g
    float a_log;  // GATE_PROJ: the head's log rate
    int L;        // GATE_PROJ: rows of the chunk (rows past it keep alpha = 1)
    uint2 k[8], q[8];
    float beta;  // beta of token `lane` (wave 0 only); logits with GATE_PROJ
};

// Issue the loads of chunk rows [c0, c0 + L) of head h; rows past L (and every
// row when L = 0) read as zero, i.e. alpha = 1 and k = q = 0.  GM (GateMode):
// GATE_HEAD broadcasts one g per (token, head) to the channels; GATE_PROJ loads
// the bf16 decay projection, turned into alpha by the decay stage.
template <int GM>
__device__ __forceinline__ void load_chunk(ChunkIn& in, const bf16_t* q, const bf16_t* k,
                                           const Gate& gt, const float* beta, int64_t c0, int L,
                                           int H, int h, int p, int lane) {
    const int cg = lane & 7, tg = lane >> 3, ch0 = 32 * p + 4 * cg;
    const size_t row = (size_t)H * D;
    const int64_t cc0 = L > 0 ? c0 : 0;  // keep the base address inside the tensors
    const size_t base = (size_t)cc0 * row + (size_t)h * D;
    const int rowb2 = (int)(row * 2), rowb4 = (int)(row * 4);
    const float* g = static_cast<const float*>(gt.g);
    const auto rg = GM == GATE_HEAD ? window(g + (size_t)cc0 * H + h, L * H * 4)
                    : GM == GATE_PROJ
                        ? window(static_cast<const bf16_t*>(gt.g) + base, L * rowb2)
                        : window(g + base, L * rowb4);
    const auto rk = window(k + base, L * rowb2);
    const auto rq = window(q + base, L * rowb2);
    const int vkq = 8 * tg * rowb2 + ch0 * 2, vg = 8 * tg * rowb4 + ch0 * 4;
    if constexpr (GM == GATE_PROJ) {
        in.a_log = gt.a_log[h];
        in.L = L;
    }
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
        if constexpr (GM == GATE_HEAD) {
            const float x = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(rg, 8 * tg * H * 4, rr * H * 4, 0));
            in.g[rr] = make_float4(x, x, x, x);
        } else if constexpr (GM == GATE_PROJ) {
            const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rg, vkq, rr * rowb2, 0);
            in.f[rr] = make_uint2(x[0], x[1]);
        } else {
            const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rg, vg, rr * rowb4, 0);
            in.g[rr] = make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]),
                                   __uint_as_float(x[2]), __uint_as_float(x[3]));
        }
        const u32x2 y = __builtin_amdgcn_raw_buffer_load_b64(rk, vkq, rr * rowb2, 0);
        const u32x2 z = __builtin_amdgcn_raw_buffer_load_b64(rq, vkq, rr * rowb2, 0);
        in.k[rr] = make_uint2(y[0], y[1]);
        in.q[rr] = make_uint2(z[0], z[1]);
    }
    const auto rb = window(beta + (size_t)cc0 * H + h, L * H * 4);
    in.beta = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, lane * H * 4, 0, 0));
}

// beta of token `lane` of the chunk (wave 0); zero on padding rows.
template <int GM>
__device__ __forceinline__ float chunk_beta(const ChunkIn& in, int lane) {
    if constexpr (GM == GATE_PROJ) return lane < in.L ? sigmoid_f(in.beta) : 0.f;
    return in.beta;
}

// log2 of the decay of element (token 8tg + rr, channel ch0 + e) of a lane's
// inputs: g * log2(e) per channel or per head, or from the projection (padding
// rows of a partial chunk keep alpha = 1).
template <int GM>
__device__ __forceinline__ void log2_decays(const ChunkIn& in, int lane, float (&lg)[8][4]) {
    const int tg = lane >> 3;
    float rate = 0.f;
    if constexpr (GM == GATE_PROJ) rate = __builtin_amdgcn_exp2f(in.a_log * LOG2E);
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
        if constexpr (GM == GATE_PROJ) {
            const float fx[4] = {bf_lo(in.f[rr].x), bf_hi(in.f[rr].x), bf_lo(in.f[rr].y),
                                 bf_hi(in.f[rr].y)};
            const bool live = 8 * tg + rr < in.L;
#pragma unroll
            for (int e = 0; e < 4; ++e) lg[rr][e] = live ? proj_log2_decay(fx[e], rate) : 0.f;
        } else {
            lg[rr][0] = in.g[rr].x * LOG2E;
            lg[rr][1] = in.g[rr].y * LOG2E;
            lg[rr][2] = in.g[rr].z * LOG2E;
            lg[rr][3] = in.g[rr].w * LOG2E;
        }
    }
}

// The cumulative log2 decay of a lane's elements: B[rr][e] for token 8tg + rr
// and channel ch0 + e (inclusive of the token), and the chunk's total bc[e]
// (B at the last token), by running sums within the lane's 8 tokens and a scan
// across the 8 token groups (lanes 8 apart).
template <int GM>
__device__ __forceinline__ void log2_prefix(const ChunkIn& in, int lane, float (&B)[8][4],
                                            float (&bc)[4]) {
    const int cg = lane & 7, tg = lane >> 3;
    log2_decays<GM>(in, lane, B);
#pragma unroll
    for (int rr = 1; rr < 8; ++rr)
#pragma unroll
        for (int e = 0; e < 4; ++e) B[rr][e] += B[rr - 1][e];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float xp = B[7][e];  // inclusive prefix over token groups
#pragma unroll
        for (int dd = 8; dd < 64; dd <<= 1) {
            const float yp = __shfl_up(xp, dd);
            if (lane >= dd) xp += yp;
        }
        // (every lane takes part in the shuffles: a lane that skipped one would
        // hand its neighbour an undefined value)
        const float up = __shfl_up(xp, 8);
        const float epre = tg > 0 ? up : 0.f;
        bc[e] = __shfl(xp, 56 + cg);
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) B[rr][e] += epre;
    }
}

// Decay stage: the cumulative log2 decay, the scaled operands Kt, Qt, Kb (rows
// into LDS) and beta into LDS.  Hands Gam[ch0 + e] (lanes with tg == 0) to
// gam_sink(ch0, gam4) and, for every lane, the Kbar^T piece of channel ch0 + e,
// tokens [8tg, 8tg + 8) as 8 packed bf16 to kbt_sink(i, tg, u32x4).  Returns
// (wave-uniform) whether some channel of this wave decays below 2^-SLOW over
// the chunk, so that the factored N and P do not hold.  Each factor costs one
// exponential and one reciprocal per element; where every channel of the wave
// is in range, Kbar = Kb * 2^{B_C - R}, else one more exponential.
template <int GM, typename L, typename GamSink, typename KbtSink>
__device__ __forceinline__ bool decay_stage(L& sm, const ChunkIn& in, int p, int lane,
                                            GamSink gam_sink, KbtSink kbt_sink) {
    const int cg = lane & 7, tg = lane >> 3, ch0 = 32 * p + 4 * cg;
    if (p == 0) sm.beta[lane] = chunk_beta<GM>(in, lane);
    float B[8][4], bc[4];
    log2_prefix<GM>(in, lane, B, bc);
    float R[4], c[4], gam[4];
    bool in_range = true;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        R[e] = fmaxf(bc[e], -RLIM);
        c[e] = __builtin_amdgcn_exp2f(bc[e] - R[e]);
        gam[e] = __builtin_amdgcn_exp2f(bc[e]);
        in_range = in_range && bc[e] >= -SLOW;
    }
    const bool wave_in_range = __all(in_range);
    if (tg == 0) gam_sink(ch0, gam);
    u32x4 kbt[4];     // Kbar^T pieces: channel ch0 + e, token pairs (2j, 2j + 1) packed
    float kb_even[4];  // Kbar of the even token of the pair being formed
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
        const float kx[4] = {bf_lo(in.k[rr].x), bf_hi(in.k[rr].x), bf_lo(in.k[rr].y),
                             bf_hi(in.k[rr].y)};
        const float qx[4] = {bf_lo(in.q[rr].x), bf_hi(in.q[rr].x), bf_lo(in.q[rr].y),
                             bf_hi(in.q[rr].y)};
        float kt[4], qt[4], kb[4], kbar[4];  // Kbar = Kb * 2^{B_C - R} while in range
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float f = __builtin_amdgcn_exp2f(B[rr][e] - R[e]);
            const float fi = __builtin_amdgcn_rcpf(f);
            kt[e] = kx[e] * f;
            qt[e] = qx[e] * f;
            kb[e] = kx[e] * fi;
            kbar[e] = kb[e] * c[e];
            if (rr & 1) kbt[e][rr >> 1] = pack2(kb_even[e], kbar[e]);
            else kb_even[e] = kbar[e];
        }
        const int t = 8 * tg + rr;
        *reinterpret_cast<uint2*>(sm.Kt + t * LDK + ch0) =
            make_uint2(pack2(kt[0], kt[1]), pack2(kt[2], kt[3]));
        *reinterpret_cast<uint2*>(sm.Qt + t * LDK + ch0) =
            make_uint2(pack2(qt[0], qt[1]), pack2(qt[2], qt[3]));
        *reinterpret_cast<uint2*>(sm.Kb + t * LDK + ch0) =
            make_uint2(pack2(kb[0], kb[1]), pack2(kb[2], kb[3]));
    }
    if (!wave_in_range) {  // Kb may have overflowed: Kbar from the decay directly
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            const float kx[4] = {bf_lo(in.k[rr].x), bf_hi(in.k[rr].x), bf_lo(in.k[rr].y),
                                 bf_hi(in.k[rr].y)};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float kbar = kx[e] * __builtin_amdgcn_exp2f(bc[e] - B[rr][e]);
                if (rr & 1) kbt[e][rr >> 1] = pack2(kb_even[e], kbar);
                else kb_even[e] = kbar;
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) kbt_sink(ch0 + e, tg, kbt[e]);
    return !wave_in_range;
}

// N stage (after the decay stage is visible): wave p forms diagonal block p of
// N in both layouts and T's diagonal block by the nilpotent product
// (I - N)(I + N^2)(I + N^4)(I + N^8) (a product and its transpose are one MFMA
// with the operands swapped); off-diagonal blocks of N go to Tt's lower part.
// n_raw forms wave p's raw products (Kt Kb^T entries, before beta and the
// causal mask) from LDS on the matrix cores; the pairwise path forms the same
// entries directly (slow_products).  n_finish applies beta and the mask and
// forms T's diagonal block; n_store writes them to T and Tt.
struct NRaw {
    f32x4 d1, d2;   // diagonal block p: d1[e] at (t, s) = (16p + 4q4 + e, 16p + r),
                    // d2[e] at (16p + r, 16p + 4q4 + e)
    f32x4 off[2];   // off-diagonal block k of wave p: off[k][e] at (16rb + r, 16cb + 4q4 + e)
};
struct NRegs {
    f32x4 Ta, Tb;   // T's diagonal block p, A and B layouts
    f32x4 off[2];   // off-diagonal N blocks of wave p (n_off(p) of them)
};
__device__ __forceinline__ int n_off(int p) { return p < 2 ? 2 : 1; }
// off-diagonal N block k of wave p: (1,0) (2,0) | (2,1) (3,0) | (3,1) | (3,2)
__device__ __forceinline__ void n_off_block(int p, int k, int& rb, int& cb) {
    rb = p == 0 ? 1 + k : p == 1 ? 2 + k : 3;
    cb = p == 0 ? 0 : p == 1 ? 1 - k : p - 1;
}

template <typename L>
__device__ __forceinline__ void n_raw(const L& sm, int p, int lane, NRaw& nw) {
    const int r = lane & 15, q4 = lane >> 4;
    f32x4 acc1 = Z4, acc2 = Z4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 xt = ld8(sm.Kt + (16 * p + r) * LDK + 32 * kk + 8 * q4);
        const bf16x8 xb = ld8(sm.Kb + (16 * p + r) * LDK + 32 * kk + 8 * q4);
        acc1 = mma32(xt, xb, acc1);  // (Kt Kb^T)[4q4+e][r]
        acc2 = mma32(xb, xt, acc2);  // (Kt Kb^T)[r][4q4+e]
    }
    nw.d1 = acc1;
    nw.d2 = acc2;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        if (k >= n_off(p)) break;
        int rb, cb;
        n_off_block(p, k, rb, cb);
        f32x4 acc = Z4;  // (Kt Kb^T) block (rb, cb), row-major
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            acc = mma32(ld8(sm.Kb + (16 * cb + r) * LDK + 32 * kk + 8 * q4),
                        ld8(sm.Kt + (16 * rb + r) * LDK + 32 * kk + 8 * q4), acc);
        nw.off[k] = acc;
    }
}

// beta: the chunk's write strengths (LDS, or wherever the caller keeps them).
__device__ __forceinline__ void n_finish(const float* beta, int p, int lane, const NRaw& nw,
                                         NRegs& nr) {
    const int r = lane & 15, q4 = lane >> 4;
    const float4 b4 = *reinterpret_cast<const float4*>(beta + 16 * p + 4 * q4);
    const float bw[4] = {b4.x, b4.y, b4.z, b4.w};
    const float br = beta[16 * p + r];
    f32x4 Nb, Na, X0b, X0a;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int rowb = 4 * q4 + e;
        Nb[e] = rowb > r ? bw[e] * nw.d1[e] : 0.f;
        Na[e] = r > rowb ? br * nw.d2[e] : 0.f;
        X0b[e] = (rowb == r ? 1.f : 0.f) - Nb[e];
        X0a[e] = (rowb == r ? 1.f : 0.f) - Na[e];
    }
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
    nr.Tb = mma16(x2a, n8b, X2b);
    nr.Ta = mma16(n8b, x2a, X2a);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        if (k >= n_off(p)) break;
        int rb, cb;
        n_off_block(p, k, rb, cb);
        const float bt = beta[16 * rb + r];
        f32x4 acc = nw.off[k];
        acc[0] *= bt; acc[1] *= bt; acc[2] *= bt; acc[3] *= bt;
        nr.off[k] = acc;
    }
}

template <typename L>
__device__ __forceinline__ void n_regs(const L& sm, int p, int lane, NRegs& nr) {
    NRaw nw;
    n_raw(sm, p, lane, nw);
    n_finish(sm.beta, p, lane, nw, nr);
}

// Block k (row order) of the 16x16 blocks on and below the diagonal of a 4x4
// grid: (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) ...
__device__ __forceinline__ void lower_block(int k, int& rb, int& cb) {
    rb = k < 1 ? 0 : k < 3 ? 1 : k < 6 ? 2 : 3;
    cb = k - rb * (rb + 1) / 2;
}
// P blocks formed by wave p beside its N blocks: blocks pk0(p) .. pk0(p) + pn(p) - 1
// of lower_block's order (2, 2, 3, 3 of the ten).
__device__ __forceinline__ int p_count(int p) { return p < 2 ? 2 : 3; }
__device__ __forceinline__ int p_first(int p) { return p == 0 ? 0 : p == 1 ? 2 : p == 2 ? 4 : 7; }

// ---------------------------------------------------------------- pairwise path
// A chunk in which some channel decays below 2^-SLOW: N and P from the decay
// between each pair of tokens directly,
//   (Kt Kb^T)[t][s] = sum_i K[t][i] K[s][i] 2^{B[t][i] - B[s][i]},
//   (Qt Kb^T)[t][s] = sum_i Q[t][i] K[s][i] 2^{B[t][i] - B[s][i]}   (s <= t),
// every factor at most 1 whatever the decay.  The entries each lane forms are
// those the matrix-core products give it (NRaw; P blocks p_first(p) ..), so the
// rest of the operand stages is shared.  Raw k, q and B go through LDS one half
// of the channels at a time (PairLds, 35 840 bytes over the stage rows).
constexpr int LDH = 72, LDB = 68;  // row strides of PairLds's bf16 and fp32 arrays
struct PairLds {
    uint16_t K[C * LDH];  // raw k of channels [64h, 64h + 64) [t][i]
    uint16_t Q[C * LDH];  // raw q
    float B[C * LDB];     // cumulative log2 decay
};

// Accumulates this half's channels into the lane's entries.  Entry (t, s) with
// X the row source (K for N, Q for P); entries above the diagonal (s > t, or
// s == t for N) stay zero.
__device__ __forceinline__ float pair_dot(const PairLds& pl, const uint16_t* X, int t, int s,
                                          bool valid) {
    float acc = 0.f;
#pragma unroll 1
    for (int j = 0; j < 16; ++j) {
        const uint2 xt = *reinterpret_cast<const uint2*>(X + t * LDH + 4 * j);
        const uint2 ks = *reinterpret_cast<const uint2*>(pl.K + s * LDH + 4 * j);
        const float4 bt = *reinterpret_cast<const float4*>(pl.B + t * LDB + 4 * j);
        const float4 bs = *reinterpret_cast<const float4*>(pl.B + s * LDB + 4 * j);
        acc += bf_lo(xt.x) * bf_lo(ks.x) * __builtin_amdgcn_exp2f(bt.x - bs.x);
        acc += bf_hi(xt.x) * bf_hi(ks.x) * __builtin_amdgcn_exp2f(bt.y - bs.y);
        acc += bf_lo(xt.y) * bf_lo(ks.y) * __builtin_amdgcn_exp2f(bt.z - bs.z);
        acc += bf_hi(xt.y) * bf_hi(ks.y) * __builtin_amdgcn_exp2f(bt.w - bs.w);
    }
    return valid ? acc : 0.f;
}

// The pairwise path for wave p: NRaw (as n_raw gives it) and P blocks pb[j]
// (block p_first(p) + j, diagonal masked as p_tile's).  `in` holds the chunk's
// inputs as load_chunk gives them (the caller reloads them); sync() is the
// workgroup barrier, called four times (the caller's other waves, if any, must
// call it as often).  Overwrites the LDS at pl.  Every loop over the lane's
// entries has a constant trip count, so that the accumulators stay in
// registers.
template <int GM, typename Sync>
__device__ __forceinline__ void slow_products(PairLds& pl, const ChunkIn& in, int p, int lane,
                                              NRaw& nw, f32x4 (&pb)[3], Sync sync) {
    const int r = lane & 15, q4 = lane >> 4, cg = lane & 7, tg = lane >> 3;
    float B[8][4], bc[4];
    log2_prefix<GM>(in, lane, B, bc);
    f32x4 d1 = Z4, d2 = Z4, off0 = Z4, off1 = Z4, p0 = Z4, p1 = Z4, p2 = Z4;
    int rb[5], cb[5];  // blocks of off0, off1, p0, p1, p2
    n_off_block(p, 0, rb[0], cb[0]);
    n_off_block(p, n_off(p) > 1 ? 1 : 0, rb[1], cb[1]);
    lower_block(p_first(p), rb[2], cb[2]);
    lower_block(p_first(p) + 1, rb[3], cb[3]);
    lower_block(p_first(p) + (p_count(p) > 2 ? 2 : 1), rb[4], cb[4]);
    const bool has_off1 = n_off(p) > 1, has_p2 = p_count(p) > 2;
    sync();  // every wave is done with the stage rows
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        if ((p >> 1) == hh) {  // waves 2hh, 2hh + 1 hold these channels
            const int lc = 32 * (p & 1) + 4 * cg;
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
                const int t = 8 * tg + rr;
                *reinterpret_cast<uint2*>(pl.K + t * LDH + lc) = in.k[rr];
                *reinterpret_cast<uint2*>(pl.Q + t * LDH + lc) = in.q[rr];
                *reinterpret_cast<float4*>(pl.B + t * LDB + lc) =
                    make_float4(B[rr][0], B[rr][1], B[rr][2], B[rr][3]);
            }
        }
        sync();
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int a = 16 * p + 4 * q4 + e, b = 16 * p + r;
            d1[e] += pair_dot(pl, pl.K, a, b, a > b);
            d2[e] += pair_dot(pl, pl.K, b, a, b > a);
            off0[e] += pair_dot(pl, pl.K, 16 * rb[0] + r, 16 * cb[0] + 4 * q4 + e, true);
            if (has_off1)
                off1[e] += pair_dot(pl, pl.K, 16 * rb[1] + r, 16 * cb[1] + 4 * q4 + e, true);
            {
                const int t = 16 * rb[2] + r, s = 16 * cb[2] + 4 * q4 + e;
                p0[e] += pair_dot(pl, pl.Q, t, s, s <= t);
            }
            {
                const int t = 16 * rb[3] + r, s = 16 * cb[3] + 4 * q4 + e;
                p1[e] += pair_dot(pl, pl.Q, t, s, s <= t);
            }
            if (has_p2) {
                const int t = 16 * rb[4] + r, s = 16 * cb[4] + 4 * q4 + e;
                p2[e] += pair_dot(pl, pl.Q, t, s, s <= t);
            }
        }
        if (hh == 0) sync();  // the first half is read in full
    }
    nw.d1 = d1;
    nw.d2 = d2;
    nw.off[0] = off0;
    nw.off[1] = off1;
    pb[0] = p0;
    pb[1] = p1;
    pb[2] = p2;
}

template <typename L>
__device__ __forceinline__ void n_store(L& sm, int p, int lane, const NRegs& nr) {
    const int r = lane & 15, q4 = lane >> 4;
    st4(sm.T + (16 * p + r) * LDT + 16 * p + 4 * q4, nr.Ta);
    st4(sm.Tt + (16 * p + r) * LDT + 16 * p + 4 * q4, nr.Tb);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        if (k >= n_off(p)) break;
        int rb, cb;
        n_off_block(p, k, rb, cb);
        st4(sm.Tt + (16 * rb + r) * LDT + 16 * cb + 4 * q4, nr.off[k]);
    }
}

__device__ __forceinline__ void n_stage(ChunkLds& sm, int p, int lane) {
    NRegs nr;
    n_regs(sm, p, lane, nr);
    n_store(sm, p, lane, nr);
}

// Merge stage (after the N stage is visible): wave 0 forms T's off-diagonal
// blocks, T21 = -T22 N21 T11 at the 32- and 64-row levels (merge_t); waves 1-3
// form P (p_tile: block (rb, cb) of lower(Qt Kb^T), p_store).  With FORM_TT,
// merge_t also leaves all of T^T in Tt: each N block is zeroed once read (T^T
// is zero below its diagonal; Tt's diagonal blocks already hold T's diagonal
// blocks transposed) and each T block it forms is also written transposed.
// Store 4 values of one row of an A-layout block into a transposed block:
// x[e] (row r, column 4 q4 + e) to base[(4 q4 + e) * LDT + r].
__device__ __forceinline__ void st4_tr(uint16_t* base, f32x4 x, int r, int q4) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
        base[(4 * q4 + e) * LDT + r] = __builtin_bit_cast(uint16_t, (__bf16)x[e]);
}

template <bool FORM_TT = false, typename L>
__device__ __forceinline__ void merge_t(L& sm, int lane) {
    const int r = lane & 15, q4 = lane >> 4;
    s16x4 bT10 = {0, 0, 0, 0}, aT32 = {0, 0, 0, 0};
    s16x4 nblk[2];  // N_10, N_32
#pragma unroll
    for (int p2 = 0; p2 < 2; ++p2) {
        const int o0 = 32 * p2;
        nblk[p2] = ld4(sm.Tt + (o0 + 16 + r) * LDT + o0 + 4 * q4);
    }
    const s16x4 n20 = ld4(sm.Tt + (32 + r) * LDT + 4 * q4);
    const s16x4 n21 = ld4(sm.Tt + (32 + r) * LDT + 16 + 4 * q4);
    const s16x4 n30 = ld4(sm.Tt + (48 + r) * LDT + 4 * q4);
    const s16x4 n31 = ld4(sm.Tt + (48 + r) * LDT + 16 + 4 * q4);
    const s16x4 bT00 = ld4(sm.Tt + r * LDT + 4 * q4);
    const s16x4 bT11 = ld4(sm.Tt + (16 + r) * LDT + 16 + 4 * q4);
    const s16x4 aT22 = ld4(sm.T + (32 + r) * LDT + 32 + 4 * q4);
    const s16x4 aT33 = ld4(sm.T + (48 + r) * LDT + 48 + 4 * q4);
    if constexpr (FORM_TT) {  // the N blocks this lane read: zero (below T^T's diagonal)
        st4(sm.Tt + (16 + r) * LDT + 4 * q4, Z4);
        st4(sm.Tt + (48 + r) * LDT + 32 + 4 * q4, Z4);
        st4(sm.Tt + (32 + r) * LDT + 4 * q4, Z4);
        st4(sm.Tt + (32 + r) * LDT + 16 + 4 * q4, Z4);
        st4(sm.Tt + (48 + r) * LDT + 4 * q4, Z4);
        st4(sm.Tt + (48 + r) * LDT + 16 + 4 * q4, Z4);
    }
#pragma unroll
    for (int p2 = 0; p2 < 2; ++p2) {
        const int o0 = 32 * p2;
        const s16x4 bTlo = p2 == 0 ? bT00 : ld4(sm.Tt + (32 + r) * LDT + 32 + 4 * q4);
        const s16x4 aThi = p2 == 0 ? ld4(sm.T + (16 + r) * LDT + 16 + 4 * q4) : aT33;
        const f32x4 X = mma16(nblk[p2], bTlo, Z4);
        const s16x4 xb = cvt4(X);
        const f32x4 Ya = neg4(mma16(xb, aThi, Z4));  // T block, A layout
        st4(sm.T + (o0 + 16 + r) * LDT + o0 + 4 * q4, Ya);
        if constexpr (FORM_TT) st4_tr(sm.Tt + o0 * LDT + o0 + 16, Ya, r, q4);
        if (p2 == 0) bT10 = cvt4(neg4(mma16(aThi, xb, Z4)));  // B layout
        else aT32 = cvt4(Ya);
    }
    s16x4 xm[2][2];
    xm[0][0] = cvt4(mma16(n21, bT10, mma16(n20, bT00, Z4)));
    xm[0][1] = cvt4(mma16(n21, bT11, Z4));
    xm[1][0] = cvt4(mma16(n31, bT10, mma16(n30, bT00, Z4)));
    xm[1][1] = cvt4(mma16(n31, bT11, Z4));
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
        const f32x4 y0 = neg4(mma16(xm[0][bb], aT22, Z4));
        const f32x4 y1 = neg4(mma16(xm[1][bb], aT33, mma16(xm[0][bb], aT32, Z4)));
        st4(sm.T + (32 + r) * LDT + 16 * bb + 4 * q4, y0);
        st4(sm.T + (48 + r) * LDT + 16 * bb + 4 * q4, y1);
        if constexpr (FORM_TT) {
            st4_tr(sm.Tt + (16 * bb) * LDT + 32, y0, r, q4);
            st4_tr(sm.Tt + (16 * bb) * LDT + 48, y1, r, q4);
        }
    }
}

template <typename L>
__device__ __forceinline__ f32x4 p_tile(const L& sm, int rb, int cb, int lane) {
    const int r = lane & 15, q4 = lane >> 4;
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
    return acc;
}
template <typename L>
__device__ __forceinline__ void p_store(L& sm, int rb, int cb, int lane, f32x4 acc) {
    const int r = lane & 15, q4 = lane >> 4;
    st4(sm.P + (16 * rb + r) * LDT + 16 * cb + 4 * q4, acc);
}

// with_p: waves 1-3 also form P (a chunk on the pairwise path has it already).
__device__ __forceinline__ void merge_stage(ChunkLds& sm, int p, int lane, bool with_p = true) {
    if (p == 0) {
        merge_t(sm, lane);
    } else if (with_p) {
        auto ptile = [&](int rb, int cb) { p_store(sm, rb, cb, lane, p_tile(sm, rb, cb, lane)); };
        if (p == 1) { ptile(0, 0); ptile(1, 0); ptile(1, 1); }
        else if (p == 2) { ptile(2, 0); ptile(2, 1); ptile(2, 2); }
        else { ptile(3, 0); ptile(3, 1); ptile(3, 2); ptile(3, 3); }
    }
}

}  // namespace co
}  // namespace kda
