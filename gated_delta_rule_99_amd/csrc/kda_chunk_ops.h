// Per-chunk operand stages of the matrix-core prefill (bf16, d_k = d_v = 128,
// chunk C = 64), shared by the chunk-parallel operand kernel of the two-kernel
// path and by the producer waves of the fused kernel.
//
// With the decay referenced to the chunk's end (recurrence from page
// "Ling-3.1-flash: a 560B hybrid-attention MoE, counted from its safetensors
// headers", section "How KDA and MLA split the work"; b the in-chunk cumulative
// log decay):
//   Kt = K * e^{b - b_C},  Qt = Q * e^{b - b_C},  Kb = K * e^{b_C - b},
//   Gam = e^{b_C},  N = strict_lower(diag(beta) Kt Kb^T),
//   T = (I + N)^{-1},  P = lower(Qt Kb^T).
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

// Window of global memory as a buffer resource: loads past num_bytes read zero,
// stores past it are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t window(const void* base, int num_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, num_bytes,
                                             0x00020000);
}

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

// Decay stage: alpha = exp(g), in-chunk running products, the scaled operands
// Kt, Qt, Kb (rows into LDS) and beta into LDS.  Hands Gam[ch0 + e] (lanes with
// tg == 0) to gam_sink(ch0, gam4) and, for every lane, the Kb^T piece of channel
// ch0 + e, tokens [8tg, 8tg + 8) as 8 packed bf16 to kbt_sink(i, tg, u32x4).
template <int GM, typename L, typename GamSink, typename KbtSink>
__device__ __forceinline__ void decay_stage(L& sm, const ChunkIn& in, int p, int lane,
                                            GamSink gam_sink, KbtSink kbt_sink) {
    const int cg = lane & 7, tg = lane >> 3, ch0 = 32 * p + 4 * cg;
    if (p == 0) sm.beta[lane] = chunk_beta<GM>(in, lane);
    float al[8][4], tot[4] = {1.f, 1.f, 1.f, 1.f};
    float rate = 0.f;
    if constexpr (GM == GATE_PROJ) rate = __builtin_amdgcn_exp2f(in.a_log * LOG2E);
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
        if constexpr (GM == GATE_PROJ) {
            const float fx[4] = {bf_lo(in.f[rr].x), bf_hi(in.f[rr].x), bf_lo(in.f[rr].y),
                                 bf_hi(in.f[rr].y)};
            const bool live = 8 * tg + rr < in.L;  // padding rows keep alpha = 1
#pragma unroll
            for (int e = 0; e < 4; ++e)
                al[rr][e] = live ? __builtin_amdgcn_exp2f(proj_log2_decay(fx[e], rate)) : 1.f;
        } else {
            al[rr][0] = __builtin_amdgcn_exp2f(in.g[rr].x * LOG2E);
            al[rr][1] = __builtin_amdgcn_exp2f(in.g[rr].y * LOG2E);
            al[rr][2] = __builtin_amdgcn_exp2f(in.g[rr].z * LOG2E);
            al[rr][3] = __builtin_amdgcn_exp2f(in.g[rr].w * LOG2E);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) tot[e] *= al[rr][e];
    }
    // products across the 8 token groups of a channel group (lanes 8 apart)
    float dsc[4], fsc[4], gam[4];
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
        gam[e] = __shfl(xp, 56 + cg);
        dsc[e] = (tg > 0 ? epre : 1.f) * __builtin_amdgcn_rcpf(gam[e]);
        fsc[e] = tg < 7 ? esuf : 1.f;
    }
    if (tg == 0) gam_sink(ch0, gam);
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
        const float kx[4] = {bf_lo(in.k[rr].x), bf_hi(in.k[rr].x), bf_lo(in.k[rr].y),
                             bf_hi(in.k[rr].y)};
        const float qx[4] = {bf_lo(in.q[rr].x), bf_hi(in.q[rr].x), bf_lo(in.q[rr].y),
                             bf_hi(in.q[rr].y)};
        float kt[4], qt[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            dsc[e] *= al[rr][e];
            kt[e] = kx[e] * dsc[e];
            qt[e] = qx[e] * dsc[e];
        }
        const int t = 8 * tg + rr;
        *reinterpret_cast<uint2*>(sm.Kt + t * LDK + ch0) =
            make_uint2(pack2(kt[0], kt[1]), pack2(kt[2], kt[3]));
        *reinterpret_cast<uint2*>(sm.Qt + t * LDK + ch0) =
            make_uint2(pack2(qt[0], qt[1]), pack2(qt[2], qt[3]));
    }
    u32x4 kbt[4];     // Kb^T pieces: channel ch0 + e, token pairs (2j, 2j + 1) packed
    float kb_odd[4];  // Kb of the odd token of the pair being formed
#pragma unroll
    for (int rr = 7; rr >= 0; --rr) {
        const float kx[4] = {bf_lo(in.k[rr].x), bf_hi(in.k[rr].x), bf_lo(in.k[rr].y),
                             bf_hi(in.k[rr].y)};
        float kb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kb[e] = kx[e] * fsc[e];
            if (rr & 1) kb_odd[e] = kb[e];
            else kbt[e][rr >> 1] = pack2(kb[e], kb_odd[e]);
            fsc[e] *= al[rr][e];
        }
        *reinterpret_cast<uint2*>(sm.Kb + (8 * tg + rr) * LDK + ch0) =
            make_uint2(pack2(kb[0], kb[1]), pack2(kb[2], kb[3]));
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) kbt_sink(ch0 + e, tg, kbt[e]);
}

// N stage (after the decay stage is visible): wave p forms diagonal block p of
// N in both layouts and T's diagonal block by the nilpotent product
// (I - N)(I + N^2)(I + N^4)(I + N^8) (a product and its transpose are one MFMA
// with the operands swapped); off-diagonal blocks of N go to Tt's lower part.
// n_regs forms wave p's blocks in registers (reading Kt, Kb and beta), n_store
// writes them to T and Tt.
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
__device__ __forceinline__ void n_regs(const L& sm, int p, int lane, NRegs& nr) {
    const int r = lane & 15, q4 = lane >> 4;
    f32x4 acc1 = Z4, acc2 = Z4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 xt = ld8(sm.Kt + (16 * p + r) * LDK + 32 * kk + 8 * q4);
        const bf16x8 xb = ld8(sm.Kb + (16 * p + r) * LDK + 32 * kk + 8 * q4);
        acc1 = mma32(xt, xb, acc1);  // (Kt Kb^T)[4q4+e][r]
        acc2 = mma32(xb, xt, acc2);  // (Kt Kb^T)[r][4q4+e]
    }
    const float4 b4 = *reinterpret_cast<const float4*>(sm.beta + 16 * p + 4 * q4);
    const float bw[4] = {b4.x, b4.y, b4.z, b4.w};
    const float br = sm.beta[16 * p + r];
    f32x4 Nb, Na, X0b, X0a;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int rowb = 4 * q4 + e;
        Nb[e] = rowb > r ? bw[e] * acc1[e] : 0.f;
        Na[e] = r > rowb ? br * acc2[e] : 0.f;
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
        f32x4 acc = Z4;  // N block (rb, cb), row-major
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            acc = mma32(ld8(sm.Kb + (16 * cb + r) * LDK + 32 * kk + 8 * q4),
                        ld8(sm.Kt + (16 * rb + r) * LDK + 32 * kk + 8 * q4), acc);
        const float bt = sm.beta[16 * rb + r];
        acc[0] *= bt; acc[1] *= bt; acc[2] *= bt; acc[3] *= bt;
        nr.off[k] = acc;
    }
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

__device__ __forceinline__ void merge_stage(ChunkLds& sm, int p, int lane) {
    if (p == 0) {
        merge_t(sm, lane);
    } else {
        auto ptile = [&](int rb, int cb) { p_store(sm, rb, cb, lane, p_tile(sm, rb, cb, lane)); };
        if (p == 1) { ptile(0, 0); ptile(1, 0); ptile(1, 1); }
        else if (p == 2) { ptile(2, 0); ptile(2, 1); ptile(2, 2); }
        else { ptile(3, 0); ptile(3, 1); ptile(3, 2); ptile(3, 3); }
    }
}

}  // namespace co
}  // namespace kda
