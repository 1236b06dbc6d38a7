// KDA decode step and state initialisation for gfx950.
//
// One recurrence step per sequence (page "Ling-3.1-flash: a 560B hybrid-attention
// MoE, counted from its safetensors headers", section "How KDA and MLA split the
// work": per-channel decay alpha_t, per-head write strength beta_t) in the fused
// form that touches the state once:
//
//   a     = exp(g_t)                       per key channel
//   y_k   = S^T (a * k_t)                  = (Diag(a) S)^T k_t
//   y_q   = S^T (a * q_t)
//   u     = beta_t (v_t - y_k)
//   o_t   = y_q + (q_t . k_t) u            = S_t^T q_t
//   S_t   = Diag(a) S + k_t u^T
//
// Several consecutive tokens of one sequence (speculative-decoding drafts) run
// in one launch: the state is read once, stepped token by token in registers,
// optionally copied out after every token, and written once.
//
// Decode is bandwidth bound (page "Ling-3.1-flash and the 7:1 hybrid: how much
// KV cache does a 560B model need at 1M tokens?", section "Why would a model keep
// only 9 full-attention layers?"): each 64 KiB fp32 state (d = 128) is streamed
// in once with 128-bit loads, kept in registers while the two column reductions
// run, and streamed out once with 128-bit stores.  Both carry the non-temporal
// hint: a state is touched once per step, and keeping it out of the caches was
// measured at 5.68 TB/s against 5.10 TB/s without the hint (B=256, H=64).
// A state may also be stored in bf16 (half the bytes; the page warns that
// linear-attention state is sensitive to precision, page "Ling-3.1-flash and
// the 7:1 hybrid: how much KV cache does a 560B model need at 1M tokens?",
// section "How fast did the community react?"): it is widened to fp32 on load,
// stepped in fp32 and rounded to nearest even once per call when stored.
#include "kda_internal.h"

namespace kda {

// State access: VEC consecutive state elements of one row (4 or 8), with the
// non-temporal (streaming) hint, widened to / narrowed from fp32.  fp32 states
// move 4 elements in 16 bytes; bf16 states 4 elements in 8 bytes or 8 in 16,
// rounded to nearest even when stored.  Two addressing forms: 64-bit
// pointers, or a head's state as a buffer window (the lane's offset voff plus
// a constant row-group offset soff), which keeps no 64-bit address live
// between the state's load and its store.
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
template <typename TS>
struct StateIO;
template <>
struct StateIO<float> {
    template <int VEC>
    static __device__ __forceinline__ void load(const float* p, float (&x)[VEC]) {
        static_assert(VEC == 4, "fp32 states move 4 elements per access");
        const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
        x[0] = v[0]; x[1] = v[1]; x[2] = v[2]; x[3] = v[3];
    }
    template <int VEC>
    static __device__ __forceinline__ void store(float* p, const float (&x)[VEC]) {
        static_assert(VEC == 4, "fp32 states move 4 elements per access");
        const f32x4 v = {x[0], x[1], x[2], x[3]};
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
    }
    template <int VEC>
    static __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int voff, int soff,
                                                float (&x)[VEC]) {
        static_assert(VEC == 4, "fp32 states move 4 elements per access");
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, BUF_NT);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(v[e]);
    }
    template <int VEC>
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, int voff, int soff,
                                                 const float (&x)[VEC]) {
        static_assert(VEC == 4, "fp32 states move 4 elements per access");
        const u32x4 v = {__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                         __float_as_uint(x[3])};
        __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, BUF_NT);
    }
};
template <>
struct StateIO<bf16_t> {
    static __device__ __forceinline__ uint32_t pack(float a, float b) {
        return (uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16);
    }
    template <int VEC>
    static __device__ __forceinline__ void load(const bf16_t* p, float (&x)[VEC]) {
        if constexpr (VEC == 4) {
            const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                x[2 * e] = bf16_bits_to_f32(v[e] & 0xffffu);
                x[2 * e + 1] = bf16_bits_to_f32(v[e] >> 16);
            }
        } else {
            static_assert(VEC == 8, "bf16 states move 4 or 8 elements per access");
            const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[2 * e] = bf16_bits_to_f32(v[e] & 0xffffu);
                x[2 * e + 1] = bf16_bits_to_f32(v[e] >> 16);
            }
        }
    }
    template <int VEC>
    static __device__ __forceinline__ void store(bf16_t* p, const float (&x)[VEC]) {
        if constexpr (VEC == 4) {
            const u32x2 v = {pack(x[0], x[1]), pack(x[2], x[3])};
            __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
        } else {
            static_assert(VEC == 8, "bf16 states move 4 or 8 elements per access");
            const u32x4 v = {pack(x[0], x[1]), pack(x[2], x[3]), pack(x[4], x[5]),
                             pack(x[6], x[7])};
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
        }
    }
    template <int VEC>
    static __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int voff, int soff,
                                                float (&x)[VEC]) {
        if constexpr (VEC == 4) {
            const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, BUF_NT);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                x[2 * e] = bf16_bits_to_f32(v[e] & 0xffffu);
                x[2 * e + 1] = bf16_bits_to_f32(v[e] >> 16);
            }
        } else {
            static_assert(VEC == 8, "bf16 states move 4 or 8 elements per access");
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, BUF_NT);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[2 * e] = bf16_bits_to_f32(v[e] & 0xffffu);
                x[2 * e + 1] = bf16_bits_to_f32(v[e] >> 16);
            }
        }
    }
    template <int VEC>
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, int voff, int soff,
                                                 const float (&x)[VEC]) {
        if constexpr (VEC == 4) {
            const u32x2 v = {pack(x[0], x[1]), pack(x[2], x[3])};
            __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, soff, BUF_NT);
        } else {
            static_assert(VEC == 8, "bf16 states move 4 or 8 elements per access");
            const u32x4 v = {pack(x[0], x[1]), pack(x[2], x[3]), pack(x[4], x[5]),
                             pack(x[6], x[7])};
            __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, BUF_NT);
        }
    }
};

// ---------------------------------------------------------------- state init

// dst[i] = src[i] (converted between fp32 and bf16 as the types say) or zero.
template <typename TD, typename TSRC>
__global__ void __launch_bounds__(256) state_fill_kernel(TD* __restrict__ dst,
                                                         const TSRC* __restrict__ src,
                                                         int64_t n4) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        float x[4] = {0.f, 0.f, 0.f, 0.f};
        if (src) StateIO<TSRC>::load(src + 4 * i, x);
        StateIO<TD>::store(dst + 4 * i, x);
    }
}

template <typename TD, typename TSRC>
static hipError_t launch_fill_t(void* dst, const void* src, int64_t n4, hipStream_t stream) {
    int64_t blocks = (n4 + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL((state_fill_kernel<TD, TSRC>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<TD*>(dst), reinterpret_cast<const TSRC*>(src), n4);
    return hipGetLastError();
}

hipError_t launch_state_init(void* state, kda_dtype state_dtype, int64_t n_elems, const void* src,
                             kda_dtype src_dtype, hipStream_t stream) {
    if (n_elems == 0) return hipSuccess;
    const int64_t n4 = n_elems / 4;  // n_elems is a multiple of 16 (d >= 16)
    const bool db = state_dtype == KDA_BF16, sb = src_dtype == KDA_BF16;
    if (db) return sb ? launch_fill_t<bf16_t, bf16_t>(state, src, n4, stream)
                      : launch_fill_t<bf16_t, float>(state, src, n4, stream);
    return sb ? launch_fill_t<float, bf16_t>(state, src, n4, stream)
              : launch_fill_t<float, float>(state, src, n4, stream);
}

// ---------------------------------------------------------------- decode

// Thread layout for one (sequence, head) state of D x D elements:
//   CG = D/VEC column groups (VEC consecutive value columns per thread and row,
//   one 16-byte access: VEC = 4 for fp32 states, 8 for bf16 states of D >= 64),
//   RG row groups; thread (rg, cg) owns rows rg, rg+RG, rg+2RG, ... (RPT rows).
// The 64 lanes of a wave read 1 KiB of consecutive rows per load instruction.
// For D = 128:
//   fp32 state, one token per call: 1024 threads of 16 elements each, compiled
//     for at least 8 waves per SIMD (at most 64 VGPRs), so two workgroups share
//     a CU.  Measured at 256 sequences x 64 heads: 0.334 ms per step against
//     0.385 ms for 256 threads of 64 elements; 6 or 12 waves per SIMD, and 512
//     threads, were 0.36-0.38 ms.
//   fp32 state, several tokens: 256 threads of 64 elements (1024 threads were
//     0.63 ms against 0.41 ms for four tokens: the per-token reductions and
//     barriers then span 16 waves).
//   bf16 state, one token per call: 1024 threads of 16 elements (2 rows of 8
//     columns), at least 8 waves per SIMD, and the column sums formed once per
//     column (as with several tokens): 0.1775 ms against 0.1833 ms for 256
//     threads of 64 elements; 512 threads of 32 were 0.187-0.29 ms.
//   bf16 state, several tokens: 256 threads of 64 elements.
// COL_SUMS: the column sums over the row groups are formed once per column into
// LDS and read back (faster with several tokens, or with 64 row groups), rather
// than by every thread for its own columns.
template <int D, int VEC, bool MULTI>
struct DecodeShape {
    static constexpr int CG = D / VEC;
    static constexpr int RG = VEC == 4 ? (CG < 8 ? CG : (CG == 32 && !MULTI ? 32 : 8))
                                       : (CG == 16 && !MULTI ? 64 : (2 * CG < 16 ? 2 * CG : 16));
    static constexpr int NT = CG * RG;
    static constexpr int RPT = D / RG;
    static constexpr int MIN_WAVES = NT == 1024 ? 8 : 1;  // per SIMD
    static constexpr bool COL_SUMS = MULTI || RG >= 64;
};
template <int D, typename TS>
constexpr int decode_vec() { return sizeof(TS) == 2 && D >= 64 ? 8 : 4; }

// VEC consecutive input elements (v) or outputs (o).
template <typename Tin, int VEC>
__device__ __forceinline__ void in_load(const Tin* p, float (&x)[VEC]) {
#pragma unroll
    for (int h = 0; h < VEC / 4; ++h) {
        float y[4];
        In<Tin>::load4(p + 4 * h, y);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * h + e] = y[e];
    }
}
template <typename Tin, int VEC>
__device__ __forceinline__ void in_store(Tin* p, const float (&x)[VEC]) {
#pragma unroll
    for (int h = 0; h < VEC / 4; ++h) {
        const float y[4] = {x[4 * h], x[4 * h + 1], x[4 * h + 2], x[4 * h + 3]};
        In<Tin>::store4(p + 4 * h, y);
    }
}

// TS: the stored state's type (fp32, or bf16 widened to fp32 while it is in
// registers and rounded once when it is written back).  MULTI: n_tok may
// exceed 1 (the token loop then also holds the partial-sum reads to fewer
// registers, which was measured faster for several tokens and slower for one).
// PROJ: g is the decay projection in Tin, with one log rate a_log per head,
// and beta holds logits (GATE_PROJ); otherwise g is fp32, per key channel or,
// with g_head, per head.
template <int D, typename Tin, typename TS, bool MULTI, bool PROJ>
__global__ void __launch_bounds__((DecodeShape<D, decode_vec<D, TS>(), MULTI>::NT),
                                  (DecodeShape<D, decode_vec<D, TS>(), MULTI>::MIN_WAVES))
decode_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
              const float* __restrict__ g, const float* __restrict__ a_log,
              const float* __restrict__ beta, int g_head, TS* __restrict__ state, int64_t n_slots,
              const int32_t* __restrict__ slot_idx, int H, int n_tok,
              TS* __restrict__ token_states, const Tin* __restrict__ zg, Tin* __restrict__ o) {
    constexpr int VEC = decode_vec<D, TS>();
    using S = DecodeShape<D, VEC, MULTI>;
    constexpr int NT = S::NT, CG = S::CG, RG = S::RG, RPT = S::RPT;
    constexpr int NWAVE = (NT + 63) / 64;

    __shared__ float s_ak[D];   // alpha * k
    __shared__ float s_aq[D];   // alpha * q
    __shared__ float s_a[D];    // alpha
    __shared__ float s_k[D];    // k
    __shared__ float s_qk[NWAVE];
    __shared__ float s_qkp[D];  // q_i * k_i (only summed directly when NT < 64)
    __shared__ __attribute__((aligned(16))) float s_part[2][RG][D];  // per-row-group partial sums
    __shared__ __attribute__((aligned(16))) float s_y[2][D];         // full column sums

    const int tid = threadIdx.x;
    const int bh = blockIdx.x;           // b * H + h
    const int b = bh / H, h = bh - b * H;
    const int64_t slot = slot_idx ? (int64_t)slot_idx[b] : (int64_t)b;
    // token j of sequence b is row (b * n_tok + j) * H + h of the activations
    auto token_row = [&](int j) { return ((int64_t)b * n_tok + j) * H + h; };

    if (slot < 0 || slot >= n_slots) {
        // invalid slot: leave every state untouched, flag the outputs
        for (int j = 0; j < n_tok; ++j)
            for (int c = tid; c < D; c += NT)
                In<Tin>::store1(o + token_row(j) * D + c, __builtin_nanf(""));
        return;
    }

    TS* st = state + ((size_t)slot * H + h) * (size_t)(D * D);
    float rate = 0.f;
    if constexpr (PROJ) rate = __expf(a_log[h]);
    const int cg = tid % CG, rg = tid / CG, c0 = VEC * cg;

    // The state's addressing.  Several tokens: a buffer window, which frees the
    // 64-bit addresses otherwise live across the token loop (d = 128: 162-164
    // -> 118-130 VGPRs, four waves per SIMD instead of three; four tokens at
    // 256 sequences x 64 heads 0.404 -> 0.399 ms).  One token: 64-bit pointers
    // (the window measured 0.333 -> 0.343 ms there, fp32 states).
    constexpr int SB = D * D * (int)sizeof(TS);      // bytes of one state
    constexpr int MSTEP = RG * D * (int)sizeof(TS);  // between a thread's rows
    const int voff = (rg * D + c0) * (int)sizeof(TS);

    // 1. stream the state in: RPT independent 16-byte loads per thread
    float s[RPT][VEC];
    if constexpr (MULTI) {
#pragma unroll
        for (int m = 0; m < RPT; ++m) StateIO<TS>::load(window(st, SB), voff, MSTEP * m, s[m]);
    } else {
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            StateIO<TS>::load(st + (size_t)(rg + RG * m) * D + c0, s[m]);
    }

    // 2-5 once per token, the state staying in registers
    const int nt = MULTI ? n_tok : 1;
    for (int j = 0; j < nt; ++j) {
        const int64_t row = token_row(j), vec = row * D;
        if (j > 0) __syncthreads();  // the previous token's reads of the LDS vectors are done

        // 2. gate vectors (small, cooperative)
        float qk_part = 0.f;
        for (int i = tid; i < D; i += NT) {
            float a;
            if constexpr (PROJ)
                a = __builtin_amdgcn_exp2f(proj_log2_decay(
                    In<Tin>::load1(reinterpret_cast<const Tin*>(g) + vec + i), rate));
            else
                a = __expf(g_head ? g[row] : g[vec + i]);
            const float kv = In<Tin>::load1(k + vec + i);
            const float qv = In<Tin>::load1(q + vec + i);
            s_a[i] = a;
            s_k[i] = kv;
            s_ak[i] = a * kv;
            s_aq[i] = a * qv;
            s_qkp[i] = qv * kv;
            qk_part += qv * kv;
        }
        if constexpr (NT % 64 == 0) {  // whole waves: reduce across lanes
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) qk_part += __shfl_xor(qk_part, off);
            if ((tid & 63) == 0) s_qk[tid >> 6] = qk_part;
        }
        float bt = beta[row];
        if constexpr (PROJ) bt = sigmoid_f(bt);
        float vj[VEC];
        in_load<Tin, VEC>(v + vec + c0, vj);
        __syncthreads();

        // 3. partial column sums over this thread's rows
        float yk[VEC], yq[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) yk[e] = yq[e] = 0.f;
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = rg + RG * m;
            const float ak = s_ak[i], aq = s_aq[i];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                yk[e] += s[m][e] * ak;
                yq[e] += s[m][e] * aq;
            }
        }
#pragma unroll
        for (int e = 0; e < VEC; e += 4) {
            *reinterpret_cast<float4*>(&s_part[0][rg][c0 + e]) =
                make_float4(yk[e], yk[e + 1], yk[e + 2], yk[e + 3]);
            *reinterpret_cast<float4*>(&s_part[1][rg][c0 + e]) =
                make_float4(yq[e], yq[e + 1], yq[e + 2], yq[e + 3]);
        }
        __syncthreads();

        // 4. full column sums, adding the row groups in order.  Where both
        // kernels use the same row groups (D < 128), one call over n_tok tokens
        // equals n_tok single steps bit for bit (fp32 states); for D = 128 the
        // single-token kernel's row groups (32 for fp32 states, 64 for bf16)
        // regroup the sum.
        float Yk[VEC], Yq[VEC];
        if constexpr (S::COL_SUMS) {
            // once per column: thread t sums one column of Y_k (t < D) or Y_q,
            // then every thread reads its own columns (per token, 1/RG of the
            // LDS reads of each thread summing its own columns, for one more
            // barrier: faster from two tokens up, and with 64 row groups)
            for (int idx = tid; idx < 2 * D; idx += NT) {
                const int which = idx >= D, col = idx - which * D;
                float acc = s_part[which][0][col];
#pragma unroll
                for (int r = 1; r < RG; ++r) acc += s_part[which][r][col];
                s_y[which][col] = acc;
            }
            __syncthreads();
#pragma unroll
            for (int e = 0; e < VEC; e += 4) {
                const float4 a = *reinterpret_cast<const float4*>(&s_y[0][c0 + e]);
                const float4 c = *reinterpret_cast<const float4*>(&s_y[1][c0 + e]);
                Yk[e] = a.x; Yk[e + 1] = a.y; Yk[e + 2] = a.z; Yk[e + 3] = a.w;
                Yq[e] = c.x; Yq[e + 1] = c.y; Yq[e + 2] = c.z; Yq[e + 3] = c.w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                Yk[e] = s_part[0][0][c0 + e];
                Yq[e] = s_part[1][0][c0 + e];
            }
            // the partial sums of the other row groups; a bounded unroll keeps
            // the LDS reads in flight (registers) in check for 16 row groups
            constexpr int RU = VEC == 4 ? RG : 4;
#pragma unroll RU
            for (int r = 1; r < RG; ++r)
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    Yk[e] += s_part[0][r][c0 + e];
                    Yq[e] += s_part[1][r][c0 + e];
                }
        }
        float qk = 0.f;
        if constexpr (NT % 64 == 0) {
#pragma unroll
            for (int w = 0; w < NWAVE; ++w) qk += s_qk[w];
        } else {
#pragma unroll
            for (int i = 0; i < D; ++i) qk += s_qkp[i];
        }
        float u[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) u[e] = bt * (vj[e] - Yk[e]);
        if (rg == 0) {
            float ov[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) ov[e] = Yq[e] + qk * u[e];
            if (zg) {  // output gate: o * sigmoid(z)
                float zv[VEC];
                in_load<Tin, VEC>(zg + vec + c0, zv);
#pragma unroll
                for (int e = 0; e < VEC; ++e) ov[e] *= sigmoid_f(zv[e]);
            }
            in_store<Tin, VEC>(o + vec + c0, ov);
        }

        // 5. decay + rank-1 write, in registers; optionally a copy per token
        TS* snap = token_states ? token_states + (size_t)row * (D * D) : nullptr;
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = rg + RG * m;
            const float a = s_a[i], kk = s_k[i];
#pragma unroll
            for (int e = 0; e < VEC; ++e) s[m][e] = a * s[m][e] + kk * u[e];
            if (snap) {
                if constexpr (MULTI)
                    StateIO<TS>::store(window(snap, SB), voff, MSTEP * m, s[m]);
                else
                    StateIO<TS>::store(snap + (size_t)i * D + c0, s[m]);
            }
        }
    }

    // 6. stream the state out
    if constexpr (MULTI) {
#pragma unroll
        for (int m = 0; m < RPT; ++m) StateIO<TS>::store(window(st, SB), voff, MSTEP * m, s[m]);
    } else {
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            StateIO<TS>::store(st + (size_t)(rg + RG * m) * D + c0, s[m]);
    }
}

template <int D, typename Tin, typename TS>
static hipError_t launch_decode_t(const void* q, const void* k, const void* v, Gate g,
                                  const float* beta, void* state, int64_t n_slots,
                                  const int32_t* slot_idx, int B, int n_tok, int H,
                                  void* token_states, const void* zg, void* o,
                                  hipStream_t stream) {
    const int64_t blocks = (int64_t)B * H;
    if (blocks == 0 || n_tok == 0) return hipSuccess;
    const bool proj = g.mode == GATE_PROJ;
    auto kern = n_tok > 1 ? (proj ? decode_kernel<D, Tin, TS, true, true>
                                  : decode_kernel<D, Tin, TS, true, false>)
                          : (proj ? decode_kernel<D, Tin, TS, false, true>
                                  : decode_kernel<D, Tin, TS, false, false>);
    constexpr int VEC = decode_vec<D, TS>();
    const int nt = n_tok > 1 ? DecodeShape<D, VEC, true>::NT : DecodeShape<D, VEC, false>::NT;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(nt),
                       0, stream, (const Tin*)q, (const Tin*)k, (const Tin*)v,
                       static_cast<const float*>(g.g), g.a_log, beta, (int)(g.mode == GATE_HEAD),
                       (TS*)state, n_slots, slot_idx, H, n_tok, (TS*)token_states,
                       (const Tin*)zg, (Tin*)o);
    return hipGetLastError();
}

template <int D, typename Tin>
static hipError_t launch_decode_s(const void* q, const void* k, const void* v, Gate g,
                                  const float* beta, void* state,
                                  kda_dtype state_dtype, int64_t n_slots,
                                  const int32_t* slot_idx, int B, int n_tok, int H,
                                  void* token_states, const void* zg, void* o,
                                  hipStream_t stream) {
    if (state_dtype == KDA_BF16)
        return launch_decode_t<D, Tin, bf16_t>(q, k, v, g, beta, state, n_slots, slot_idx,
                                               B, n_tok, H, token_states, zg, o, stream);
    return launch_decode_t<D, Tin, float>(q, k, v, g, beta, state, n_slots, slot_idx, B,
                                          n_tok, H, token_states, zg, o, stream);
}

hipError_t launch_decode(const void* q, const void* k, const void* v, Gate g,
                         const float* beta, kda_dtype dtype, void* state,
                         kda_dtype state_dtype, int64_t n_slots, const int32_t* slot_idx, int B,
                         int n_tok, int H, int d, void* token_states, const void* out_gate,
                         void* o, hipStream_t stream) {
#define KDA_DEC(D)                                                                           \
    if (d == D) {                                                                            \
        if (dtype == KDA_BF16)                                                               \
            return launch_decode_s<D, bf16_t>(q, k, v, g, beta, state, state_dtype,  \
                                              n_slots, slot_idx, B, n_tok, H, token_states,  \
                                              out_gate, o, stream);                          \
        return launch_decode_s<D, float>(q, k, v, g, beta, state, state_dtype, n_slots, \
                                         slot_idx, B, n_tok, H, token_states, out_gate, o,   \
                                         stream);                                            \
    }
    KDA_DEC(16)
    KDA_DEC(32)
    KDA_DEC(64)
    KDA_DEC(128)
#undef KDA_DEC
    return hipErrorInvalidValue;
}

}  // namespace kda
