// KDA chunked prefill, split form for gfx950: bf16 q/k/v, d_k = d_v = 128,
// chunk C = 64, fp32 state.  Same algebra as the fused kernel
// (kda_prefill_mfma.hip): per chunk, with the decay referenced to the chunk end,
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
#include "kda_internal.h"

namespace kda {
namespace sp {

constexpr int D = 128, C = 64, DVS = 32, NS = D / DVS;
constexpr int MAX_WIN = 32;                 // chunks per window, at most
constexpr size_t TILE_BUDGET = 192u << 20;  // bytes of one window's tiles, at most
constexpr int LDK = 136, LDT = 72, LDO = 40, LDV = 68;
constexpr int TILE = 66304;
constexpr int OFF_KT = 0, OFF_QT = 16384, OFF_KBT = 32768, OFF_T = 49152, OFF_P = 57344,
              OFF_BETA = 65536, OFF_GAM = 65792;
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

// Window of global memory as a buffer resource: loads past num_bytes read zero,
// stores past it are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t window(const void* base, int num_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, num_bytes,
                                             0x00020000);
}
__device__ __forceinline__ bf16x8 as_bf8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ u32x4 as_u4(bf16x8 x) { return __builtin_bit_cast(u32x4, x); }

// Chunk count of sequence n (clamped to [0, T)).
__device__ __forceinline__ void seq_chunks(const int32_t* cu, int n, int64_t T, int64_t& tb,
                                           int64_t& te, int& nc) {
    seq_range(cu, n, T, tb, te);
    nc = (int)((te - tb + C - 1) / C);
}

struct PrepSmem {
    uint16_t Kt[C * LDK];   // [t][i]
    uint16_t Qt[C * LDK];   // [t][i]
    uint16_t Kb[C * LDK];   // [t][i]
    uint16_t T[C * LDT];    // T [t][s]
    uint16_t Tt[C * LDT];   // T^T [s][t]; its strictly-lower 16x16 blocks hold N
    uint16_t P[C * LDT];    // P [t][s]
    float beta[C];
};

}  // namespace sp

using namespace sp;

// ---------------------------------------------------------------- prep
// grid (n_seqs * H, chunks in the window): one workgroup of 4 waves per
// (sequence, head, window chunk).  Lane (cg, tg) of wave p handles channels [32p + 4cg, +4) of
// tokens [8tg, 8tg + 8) for the decay stage.
__global__ void __launch_bounds__(256, 2)
prep_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
            const float* __restrict__ g, const float* __restrict__ beta,
            const int32_t* __restrict__ cu, int64_t T, int H, int w0, int win,
            uint8_t* __restrict__ ws_tiles) {
    __shared__ __attribute__((aligned(16))) PrepSmem sm;
    const int pair = blockIdx.x, cl = blockIdx.y, n = pair / H, h = pair - n * H;
    int64_t tb, te;
    int nc;
    seq_chunks(cu, n, T, tb, te, nc);
    const int c = w0 + cl;
    if (c >= nc) return;
    const int tid = threadIdx.x, p = tid >> 6, lane = tid & 63;
    const int r = lane & 15, q4 = lane >> 4;
    const int cg = lane & 7, tg = lane >> 3, ch0 = 32 * p + 4 * cg;
    const size_t row = (size_t)H * D;
    const int64_t c0 = tb + (int64_t)c * C;
    const int L = (te - c0) < C ? (int)(te - c0) : C;
    uint8_t* tile = ws_tiles + ((size_t)(n * win + cl) * H + h) * TILE;
    const auto rt = window(tile, TILE);

    // zero the upper blocks of T and P (T^T's upper blocks are overwritten by data)
    for (int e = tid; e < C * LDT / 2; e += 256) {
        reinterpret_cast<uint32_t*>(sm.T)[e] = 0u;
        reinterpret_cast<uint32_t*>(sm.P)[e] = 0u;
    }

    // ---- load: rows past the chunk's end read as zero (alpha = 1, k = q = 0)
    float4 pg[8];
    uint2 pk[8], pq[8];
    {
        const size_t base = (size_t)c0 * row + (size_t)h * D;
        const int rowb2 = (int)(row * 2), rowb4 = (int)(row * 4);
        const auto rg = window(g + base, L * rowb4);
        const auto rk = window(k + base, L * rowb2);
        const auto rq = window(q + base, L * rowb2);
        const int vkq = 8 * tg * rowb2 + ch0 * 2, vg = 8 * tg * rowb4 + ch0 * 4;
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rg, vg, rr * rowb4, 0);
            pg[rr] = make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]),
                                 __uint_as_float(x[2]), __uint_as_float(x[3]));
            const u32x2 y = __builtin_amdgcn_raw_buffer_load_b64(rk, vkq, rr * rowb2, 0);
            const u32x2 z = __builtin_amdgcn_raw_buffer_load_b64(rq, vkq, rr * rowb2, 0);
            pk[rr] = make_uint2(y[0], y[1]);
            pq[rr] = make_uint2(z[0], z[1]);
        }
        if (p == 0) {
            const auto rb = window(beta + (size_t)c0 * H + h, L * H * 4);
            const float bv =
                __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, lane * H * 4, 0, 0));
            sm.beta[lane] = bv;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(bv), rt, OFF_BETA + 4 * lane, 0,
                                                  0);
        }
    }

    // ---- decay: alpha = exp(g); D and F from running products
    {
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
        if (tg == 0)
            __builtin_amdgcn_raw_buffer_store_b128(
                u32x4{__float_as_uint(gam[0]), __float_as_uint(gam[1]), __float_as_uint(gam[2]),
                      __float_as_uint(gam[3])},
                rt, OFF_GAM + 4 * ch0, 0, 0);
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            const float kx[4] = {bf_lo(pk[rr].x), bf_hi(pk[rr].x), bf_lo(pk[rr].y),
                                 bf_hi(pk[rr].y)};
            const float qx[4] = {bf_lo(pq[rr].x), bf_hi(pq[rr].x), bf_lo(pq[rr].y),
                                 bf_hi(pq[rr].y)};
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
            *reinterpret_cast<uint2*>(sm.Kb + (8 * tg + rr) * LDK + ch0) =
                make_uint2(pack2(kb[0], kb[1]), pack2(kb[2], kb[3]));
        }
        // Kb^T fragments straight from registers: channel row i = ch0 + e holds
        // tokens [8tg, 8tg + 8), exactly one lane's 16-byte fragment
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = ch0 + e;
            const int blk = (i >> 5) * 4 + ((i >> 4) & 1) * 2 + (tg >> 2);
            const int ln = (i & 15) + 16 * (tg & 3);
            __builtin_amdgcn_raw_buffer_store_b128(
                u32x4{pack2(kb4[e][0], kb4[e][1]), pack2(kb4[e][2], kb4[e][3]),
                      pack2(kb4[e][4], kb4[e][5]), pack2(kb4[e][6], kb4[e][7])},
                rt, OFF_KBT + (blk * 64 + ln) * 16, 0, 0);
        }
    }
    __syncthreads();

    // ---- Kt and Qt fragments out (wave p exports row block p)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 a = ld8(sm.Kt + (16 * p + r) * LDK + 32 * kk + 8 * q4);
        const bf16x8 b = ld8(sm.Qt + (16 * p + r) * LDK + 32 * kk + 8 * q4);
        __builtin_amdgcn_raw_buffer_store_b128(as_u4(a), rt, OFF_KT + ((p * 4 + kk) * 64 + lane) * 16,
                                               0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(as_u4(b), rt, OFF_QT + ((p * 4 + kk) * 64 + lane) * 16,
                                               0, 0);
    }

    // ---- N: diagonal block p in both layouts -> T_pp by the product form;
    // off-diagonal blocks into T^T's strictly-lower blocks
    {
        f32x4 acc1 = Z4, acc2 = Z4;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const bf16x8 xt = ld8(sm.Kt + (16 * p + r) * LDK + 32 * kk + 8 * q4);
            const bf16x8 xb = ld8(sm.Kb + (16 * p + r) * LDK + 32 * kk + 8 * q4);
            acc1 = mma32(xt, xb, acc1);  // [4q4+e][r]
            acc2 = mma32(xb, xt, acc2);  // [r][4q4+e]
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
        const f32x4 Tb = mma16(x2a, n8b, X2b), Ta = mma16(n8b, x2a, X2a);
        st4(sm.T + (16 * p + r) * LDT + 16 * p + 4 * q4, Ta);
        st4(sm.Tt + (16 * p + r) * LDT + 16 * p + 4 * q4, Tb);
        auto offdiag = [&](int rb, int cb) {  // N block (rb, cb), row-major, in T^T's lower part
            f32x4 acc = Z4;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                acc = mma32(ld8(sm.Kb + (16 * cb + r) * LDK + 32 * kk + 8 * q4),
                            ld8(sm.Kt + (16 * rb + r) * LDK + 32 * kk + 8 * q4), acc);
            const float bt = sm.beta[16 * rb + r];
            acc[0] *= bt; acc[1] *= bt; acc[2] *= bt; acc[3] *= bt;
            st4(sm.Tt + (16 * rb + r) * LDT + 16 * cb + 4 * q4, acc);
        };
        if (p == 0) { offdiag(1, 0); offdiag(2, 0); }
        else if (p == 1) { offdiag(2, 1); offdiag(3, 0); }
        else if (p == 2) { offdiag(3, 1); }
        else { offdiag(3, 2); }
    }
    __syncthreads();

    // ---- wave 0: T's off-diagonal blocks; waves 1-3: P
    if (p == 0) {
        s16x4 bT10 = {0, 0, 0, 0}, aT32 = {0, 0, 0, 0};
        s16x4 nblk[4];  // N_10, N_32, then N_20/N_21, N_30/N_31 read below
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
#pragma unroll
        for (int p2 = 0; p2 < 2; ++p2) {
            const int o0 = 32 * p2;
            const s16x4 bTlo = p2 == 0 ? bT00 : ld4(sm.Tt + (32 + r) * LDT + 32 + 4 * q4);
            const s16x4 aThi = p2 == 0 ? ld4(sm.T + (16 + r) * LDT + 16 + 4 * q4) : aT33;
            const f32x4 X = mma16(nblk[p2], bTlo, Z4);
            const s16x4 xb = cvt4(X);
            const f32x4 Ya = neg4(mma16(xb, aThi, Z4));  // T block, A layout
            st4(sm.T + (o0 + 16 + r) * LDT + o0 + 4 * q4, Ya);
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
            const f32x4 y0 = mma16(xm[0][bb], aT22, Z4);
            const f32x4 y1 = mma16(xm[1][bb], aT33, mma16(xm[0][bb], aT32, Z4));
            st4(sm.T + (32 + r) * LDT + 16 * bb + 4 * q4, neg4(y0));
            st4(sm.T + (48 + r) * LDT + 16 * bb + 4 * q4, neg4(y1));
        }
    } else {
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
    __syncthreads();

    // ---- T and P fragments out (wave p exports row block p)
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
// grid n_seqs * H * NS (slices of one head placed on one XCD); 4 waves.  Wave c
// owns output rows [16c, 16c+16) and state rows [32c, 32c+32) of its slice.
struct StateSmem {
    uint16_t Gt[DVS * LDK];  // bf16 (Gam * S)^T [j][i]
    uint16_t Rt[DVS * LDT];  // R^T [j][t]
    uint16_t Ut[DVS * LDT];  // U^T [j][t]
    uint16_t O[C * LDO];     // output staging [t][j]
    float Vt[DVS * LDV];     // V^T [j][t]
};

struct Frags {
    bf16x8 K[4], Q[4], Kb[2][2], T[2], P[2];
    float4 bet, gam[2];
    uint4 v;  // this thread's 8 bf16 of the chunk's V slice
};

__global__ void __launch_bounds__(256)
state_kernel(const bf16_t* __restrict__ v, const int32_t* __restrict__ cu, int64_t T, int H,
             int n_pairs, int w0, int win, const uint8_t* __restrict__ ws_tiles, float* __restrict__ ws_state,
             const float* __restrict__ s0, float* __restrict__ s_final, bf16_t* __restrict__ o) {
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
    const int tid = threadIdx.x, cw = tid >> 6, lane = tid & 63;
    const int r = lane & 15, q4 = lane >> 4;
    const size_t sidx = (size_t)pair * D * D;
    const float* s_in = first_window ? s0 : ws_state;
    float* s_out = last_here ? s_final : ws_state;

    if (c_beg >= c_end) {  // nothing in this window (ended earlier, or empty sequence)
        if (first_window && nc == 0 && s_final) {
            for (int e = tid; e < D * DVS; e += 256) {
                const size_t at = sidx + (size_t)(e / DVS) * D + j0 + e % DVS;
                s_final[at] = s0 ? s0[at] : 0.f;
            }
        }
        return;
    }
    // state slice, lane holds S[32c + 16a + 4q4 + e][16jb + r]
    f32x4 S[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 32 * cw + 16 * a + 4 * q4 + e, j = 16 * jb + r;
                S[a][jb][e] = s_in ? s_in[sidx + (size_t)i * D + j0 + j] : 0.f;
            }

    const size_t row = (size_t)H * D;
    const size_t hoff = (size_t)h * D;
    const int rowb = (int)(row * 2);
    const int vrow = tid >> 2, vcol = 8 * (tid & 3), voff_v = vrow * rowb + vcol * 2;
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
    // Fragment loads of chunk c, in four groups so that they can be spread over
    // the segments of a step (a group is ~5 loads of 1 KB per wave).
    auto tile_rsrc = [&](int c) {
        const int cc = c < c_end ? c : c_beg;  // keep the address inside the workspace
        return window(ws_tiles + ((size_t)(n * win + (cc - w0)) * H + h) * TILE,
                      c < c_end ? TILE : 0);
    };
    auto load_a = [&](int c, Frags& f) {  // K, beta, Gam, V
        const auto rt = tile_rsrc(c);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            f.K[kk] = as_bf8(__builtin_amdgcn_raw_buffer_load_b128(
                rt, OFF_KT + ((cw * 4 + kk) * 64 + lane) * 16, 0, 0));
        const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rt, OFF_BETA + (16 * cw + 4 * q4) * 4,
                                                              0, 0);
        f.bet = make_float4(__uint_as_float(b[0]), __uint_as_float(b[1]), __uint_as_float(b[2]),
                            __uint_as_float(b[3]));
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const u32x4 gg = __builtin_amdgcn_raw_buffer_load_b128(
                rt, OFF_GAM + (32 * cw + 16 * a + 4 * q4) * 4, 0, 0);
            f.gam[a] = make_float4(__uint_as_float(gg[0]), __uint_as_float(gg[1]),
                                   __uint_as_float(gg[2]), __uint_as_float(gg[3]));
        }
        const int cc = c < c_end ? c : c_beg;
        const auto rv = window(v + (size_t)(tb + (int64_t)cc * C) * row + hoff + j0,
                               chunk_len(c) * rowb);
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rv, voff_v, 0, 0);
        f.v = make_uint4(x[0], x[1], x[2], x[3]);
    };
    auto load_b = [&](int c, Frags& f) {  // Q
        const auto rt = tile_rsrc(c);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            f.Q[kk] = as_bf8(__builtin_amdgcn_raw_buffer_load_b128(
                rt, OFF_QT + ((cw * 4 + kk) * 64 + lane) * 16, 0, 0));
    };
    auto load_c = [&](int c, Frags& f) {  // Kb^T
        const auto rt = tile_rsrc(c);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                f.Kb[a][kk] = as_bf8(__builtin_amdgcn_raw_buffer_load_b128(
                    rt, OFF_KBT + ((cw * 4 + a * 2 + kk) * 64 + lane) * 16, 0, 0));
    };
    auto load_d = [&](int c, Frags& f) {  // T, P
        const auto rt = tile_rsrc(c);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            f.T[kk] = as_bf8(__builtin_amdgcn_raw_buffer_load_b128(
                rt, OFF_T + ((cw * 2 + kk) * 64 + lane) * 16, 0, 0));
            f.P[kk] = as_bf8(__builtin_amdgcn_raw_buffer_load_b128(
                rt, OFF_P + ((cw * 2 + kk) * 64 + lane) * 16, 0, 0));
        }
    };
    auto load_frags = [&](int c, Frags& f) {
        load_a(c, f);
        load_b(c, f);
        load_c(c, f);
        load_d(c, f);
    };
    auto flush_o = [&](int c) {
        const int cc = c >= c_beg ? c : c_beg;
        const auto ro = window(o + (size_t)(tb + (int64_t)cc * C) * row + hoff + j0,
                               chunk_len(c) * rowb);
        const uint4 x = *reinterpret_cast<const uint4*>(sm.O + vrow * LDO + vcol);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{x.x, x.y, x.z, x.w}, ro, voff_v, 0, 0);
    };

    // Three fragment sets in rotation: while chunk c runs, the loads of chunk
    // c + 1 are in flight since one chunk and those of c + 2 are being issued.
    Frags F0, F1, F2;
    load_frags(c_beg, F0);
    load_frags(c_beg + 1, F1);
    // G = Gam * S for the first chunk of the window
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            S[a][jb][0] *= F0.gam[a].x; S[a][jb][1] *= F0.gam[a].y;
            S[a][jb][2] *= F0.gam[a].z; S[a][jb][3] *= F0.gam[a].w;
            st4(sm.Gt + (16 * jb + r) * LDK + 32 * cw + 16 * a + 4 * q4, S[a][jb]);
        }

    auto step = [&](int c, const Frags& cur, const Frags& nxt, Frags& later) {
        const bool more = c + 1 < c_end;
        // ---- segment 0: V into LDS, previous output out, prefetch chunk c + 2
        {
            const uint32_t w4[4] = {cur.v.x, cur.v.y, cur.v.z, cur.v.w};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                sm.Vt[(vcol + 2 * m) * LDV + vrow] = bf_lo(w4[m]);
                sm.Vt[(vcol + 2 * m + 1) * LDV + vrow] = bf_hi(w4[m]);
            }
        }
        flush_o(c - 1);
        load_a(c + 2, later);
        __syncthreads();
        // ---- segment 1: Y = Kt G, Z = Qt G, R = diag(beta)(V - Y)
        f32x4 Y[2] = {Z4, Z4}, Zc[2] = {Z4, Z4};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const bf16x8 b0 = ld8(sm.Gt + r * LDK + 32 * kk + 8 * q4);
            const bf16x8 b1 = ld8(sm.Gt + (16 + r) * LDK + 32 * kk + 8 * q4);
            Y[0] = mma32(cur.K[kk], b0, Y[0]);
            Y[1] = mma32(cur.K[kk], b1, Y[1]);
            Zc[0] = mma32(cur.Q[kk], b0, Zc[0]);
            Zc[1] = mma32(cur.Q[kk], b1, Zc[1]);
        }
        load_b(c + 2, later);
        {
            const float bb[4] = {cur.bet.x, cur.bet.y, cur.bet.z, cur.bet.w};
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
        }
        __syncthreads();
        // ---- segment 2: U = T R
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            f32x4 u = mma32(cur.T[0], ld8(sm.Rt + (16 * jb + r) * LDT + 8 * q4), Z4);
            if (cw >= 2) u = mma32(cur.T[1], ld8(sm.Rt + (16 * jb + r) * LDT + 32 + 8 * q4), u);
            st4(sm.Ut + (16 * jb + r) * LDT + 16 * cw + 4 * q4, u);
        }
        load_c(c + 2, later);
        __syncthreads();
        // ---- segment 3: O = Z + P U; S <- G + Kb^T U; next G
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            f32x4 acc = mma32(cur.P[0], ld8(sm.Ut + (16 * jb + r) * LDT + 8 * q4), Zc[jb]);
            if (cw >= 2) acc = mma32(cur.P[1], ld8(sm.Ut + (16 * jb + r) * LDT + 32 + 8 * q4), acc);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sm.O[(16 * cw + 4 * q4 + e) * LDO + 16 * jb + r] = f32_to_bf16_bits(acc[e]);
        }
#pragma unroll
        for (int a = 0; a < 2; ++a) {
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                const bf16x8 u0 = ld8(sm.Ut + (16 * jb + r) * LDT + 8 * q4);
                const bf16x8 u1 = ld8(sm.Ut + (16 * jb + r) * LDT + 32 + 8 * q4);
                f32x4 s = mma32(cur.Kb[a][1], u1, mma32(cur.Kb[a][0], u0, S[a][jb]));
                if (more) {
                    s[0] *= nxt.gam[a].x; s[1] *= nxt.gam[a].y;
                    s[2] *= nxt.gam[a].z; s[3] *= nxt.gam[a].w;
                    st4(sm.Gt + (16 * jb + r) * LDK + 32 * cw + 16 * a + 4 * q4, s);
                }
                S[a][jb] = s;
            }
        }
        load_d(c + 2, later);
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
    flush_o(c_end - 1);
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
                                const float* beta, const int32_t* cu, int n_seqs, int64_t T,
                                int H, int max_chunks, const float* s0, float* s_final, void* o,
                                void* workspace, hipStream_t stream) {
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
            hipLaunchKernelGGL(prep_kernel, dim3((unsigned)n_pairs, (unsigned)rows), dim3(256), 0,
                               stream, (const bf16_t*)q, (const bf16_t*)k, g, beta, cu, T, H, w0,
                               win, tiles);
            hipError_t err = hipGetLastError();
            if (err != hipSuccess) return err;
        }
        hipLaunchKernelGGL(state_kernel, dim3((unsigned)(n_pairs * NS)), dim3(256), 0, stream,
                           (const bf16_t*)v, cu, T, H, (int)n_pairs, w0, win, tiles, ws_state, s0,
                           s_final, (bf16_t*)o);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace kda
