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
#include "kda_internal.h"

namespace kda {

// 128-bit state access with the non-temporal (streaming) hint.
__device__ __forceinline__ float4 load_stream(const float* p) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store_stream(float* p, float4 r) {
    const f32x4 v = {r.x, r.y, r.z, r.w};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}

// ---------------------------------------------------------------- state init

__global__ void __launch_bounds__(256) state_fill_kernel(float4* __restrict__ dst,
                                                         const float4* __restrict__ src,
                                                         int64_t n4) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
        dst[i] = src ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
}

hipError_t launch_state_init(float* state, int64_t n_floats, const float* src,
                             hipStream_t stream) {
    if (n_floats == 0) return hipSuccess;
    const int64_t n4 = n_floats / 4;  // n_floats is a multiple of 16 (d >= 16)
    int64_t blocks = (n4 + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(state_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<float4*>(state), reinterpret_cast<const float4*>(src),
                       n4);
    return hipGetLastError();
}

// ---------------------------------------------------------------- decode

// Thread layout for one (sequence, head) state of D x D floats:
//   CG = D/4 column groups (4 consecutive value columns, one float4 each),
//   RG row groups; thread (rg, cg) owns rows rg, rg+RG, rg+2RG, ... (RPT rows).
// For D = 128: 256 threads, 16 rows each; the 64 lanes of a wave cover two
// adjacent 512-byte rows per load instruction (1 KiB contiguous).
template <int D>
struct DecodeShape {
    static constexpr int CG = D / 4;
    static constexpr int RG = (D / 4) < 8 ? (D / 4) : 8;
    static constexpr int NT = CG * RG;
    static constexpr int RPT = D / RG;
};

template <int D, typename Tin>
__global__ void __launch_bounds__(DecodeShape<D>::NT)
decode_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
              const float* __restrict__ g, const float* __restrict__ beta,
              int g_head, float* __restrict__ state, int64_t n_slots,
              const int32_t* __restrict__ slot_idx, int H, int n_tok,
              float* __restrict__ token_states, Tin* __restrict__ o) {
    using S = DecodeShape<D>;
    constexpr int NT = S::NT, CG = S::CG, RG = S::RG, RPT = S::RPT;
    constexpr int NWAVE = (NT + 63) / 64;

    __shared__ float s_ak[D];   // alpha * k
    __shared__ float s_aq[D];   // alpha * q
    __shared__ float s_a[D];    // alpha
    __shared__ float s_k[D];    // k
    __shared__ float s_qk[NWAVE];
    __shared__ float s_qkp[D];  // q_i * k_i (only summed directly when NT < 64)
    __shared__ float4 s_part[2][RG][CG];  // per-row-group partial column sums

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

    float* st = state + ((size_t)slot * H + h) * (size_t)(D * D);
    const int cg = tid % CG, rg = tid / CG;

    // 1. stream the state in: RPT independent 128-bit loads per thread
    float4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) s[m] = load_stream(st + (size_t)(rg + RG * m) * D + 4 * cg);

    // 2-5 once per token, the state staying in registers
    for (int j = 0; j < n_tok; ++j) {
        const int64_t row = token_row(j), vec = row * D;
        if (j > 0) __syncthreads();  // the previous token's reads of the LDS vectors are done

        // 2. gate vectors (small, cooperative)
        float qk_part = 0.f;
        for (int i = tid; i < D; i += NT) {
            const float a = __expf(g_head ? g[row] : g[vec + i]);
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
        const float bt = beta[row];
        float vj[4];
        In<Tin>::load4(v + vec + 4 * cg, vj);
        __syncthreads();

        // 3. partial column sums over this thread's rows
        float yk[4] = {0.f, 0.f, 0.f, 0.f}, yq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = rg + RG * m;
            const float ak = s_ak[i], aq = s_aq[i];
            yk[0] += s[m].x * ak; yk[1] += s[m].y * ak; yk[2] += s[m].z * ak; yk[3] += s[m].w * ak;
            yq[0] += s[m].x * aq; yq[1] += s[m].y * aq; yq[2] += s[m].z * aq; yq[3] += s[m].w * aq;
        }
        s_part[0][rg][cg] = make_float4(yk[0], yk[1], yk[2], yk[3]);
        s_part[1][rg][cg] = make_float4(yq[0], yq[1], yq[2], yq[3]);
        __syncthreads();

        // 4. full column sums, write value and output
        float4 Yk = s_part[0][0][cg], Yq = s_part[1][0][cg];
#pragma unroll
        for (int r = 1; r < RG; ++r) {
            const float4 a = s_part[0][r][cg], c = s_part[1][r][cg];
            Yk.x += a.x; Yk.y += a.y; Yk.z += a.z; Yk.w += a.w;
            Yq.x += c.x; Yq.y += c.y; Yq.z += c.z; Yq.w += c.w;
        }
        float qk = 0.f;
        if constexpr (NT % 64 == 0) {
#pragma unroll
            for (int w = 0; w < NWAVE; ++w) qk += s_qk[w];
        } else {
#pragma unroll
            for (int i = 0; i < D; ++i) qk += s_qkp[i];
        }
        float u[4];
        u[0] = bt * (vj[0] - Yk.x);
        u[1] = bt * (vj[1] - Yk.y);
        u[2] = bt * (vj[2] - Yk.z);
        u[3] = bt * (vj[3] - Yk.w);
        if (rg == 0) {
            float ov[4] = {Yq.x + qk * u[0], Yq.y + qk * u[1], Yq.z + qk * u[2], Yq.w + qk * u[3]};
            In<Tin>::store4(o + vec + 4 * cg, ov);
        }

        // 5. decay + rank-1 write, in registers; optionally a copy per token
        float* snap = token_states ? token_states + (size_t)row * (D * D) : nullptr;
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = rg + RG * m;
            const float a = s_a[i], kk = s_k[i];
            s[m].x = a * s[m].x + kk * u[0];
            s[m].y = a * s[m].y + kk * u[1];
            s[m].z = a * s[m].z + kk * u[2];
            s[m].w = a * s[m].w + kk * u[3];
            if (snap) store_stream(snap + (size_t)i * D + 4 * cg, s[m]);
        }
    }

    // 6. stream the state out
#pragma unroll
    for (int m = 0; m < RPT; ++m) store_stream(st + (size_t)(rg + RG * m) * D + 4 * cg, s[m]);
}

template <int D, typename Tin>
static hipError_t launch_decode_t(const void* q, const void* k, const void* v, const float* g,
                                  const float* beta, bool g_head, float* state, int64_t n_slots,
                                  const int32_t* slot_idx, int B, int n_tok, int H,
                                  float* token_states, void* o, hipStream_t stream) {
    const int64_t blocks = (int64_t)B * H;
    if (blocks == 0 || n_tok == 0) return hipSuccess;
    hipLaunchKernelGGL((decode_kernel<D, Tin>), dim3((unsigned)blocks),
                       dim3(DecodeShape<D>::NT), 0, stream, (const Tin*)q, (const Tin*)k,
                       (const Tin*)v, g, beta, (int)g_head, state, n_slots, slot_idx, H, n_tok,
                       token_states, (Tin*)o);
    return hipGetLastError();
}

hipError_t launch_decode(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, kda_dtype dtype, bool g_head, float* state,
                         int64_t n_slots,
                         const int32_t* slot_idx, int B, int n_tok, int H, int d,
                         float* token_states, void* o, hipStream_t stream) {
#define KDA_DEC(D)                                                                          \
    if (d == D) {                                                                           \
        if (dtype == KDA_BF16)                                                              \
            return launch_decode_t<D, bf16_t>(q, k, v, g, beta, g_head, state, n_slots, slot_idx, \
                                              B, n_tok, H, token_states, o, stream);        \
        return launch_decode_t<D, float>(q, k, v, g, beta, g_head, state, n_slots, slot_idx, B, \
                                         n_tok, H, token_states, o, stream);                 \
    }
    KDA_DEC(16)
    KDA_DEC(32)
    KDA_DEC(64)
    KDA_DEC(128)
#undef KDA_DEC
    return hipErrorInvalidValue;
}

}  // namespace kda
