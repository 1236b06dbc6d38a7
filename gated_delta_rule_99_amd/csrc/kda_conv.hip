// Width-4 causal depthwise convolution (+ optional per-head L2 normalisation)
// that q, k and v pass through before the KDA recurrence (page "Ling-3.1-flash: a
// 560B hybrid-attention MoE, counted from its safetensors headers", section "How
// KDA and MLA split the work"; the convolution tails it leaves behind are the
// "convolution tails" of section "Does 292 GiB fit on four Hopper GPUs?").
//
//   y_t[c] = sum_{j=0..3} w[c][j] x_{t-3+j}[c]     (w[c][3] multiplies x_t)
//   y_t[head] <- y_t[head] / sqrt(sum(y_t[head]^2) + eps)      (optional)
//
// Prefill: one wave per (run of RUN tokens, head); a lane owns two adjacent
// channels and slides a 4-tap window down the run, so every input row is read
// once; the head's sum of squares is a wave reduction (no LDS, no barrier).
// Heads wider than 128 channels use several lanes' pairs per lane.
#include "kda_internal.h"

namespace kda {

constexpr int RUN = 16;  // tokens per wave in the prefill convolution

template <typename Tin>
__device__ __forceinline__ void load2(const Tin* p, float& a, float& b);
template <>
__device__ __forceinline__ void load2<float>(const float* p, float& a, float& b) {
    const float2 v = *reinterpret_cast<const float2*>(p);
    a = v.x;
    b = v.y;
}
template <>
__device__ __forceinline__ void load2<bf16_t>(const bf16_t* p, float& a, float& b) {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(p);
    a = bf16_bits_to_f32(v & 0xffffu);
    b = bf16_bits_to_f32(v >> 16);
}
template <typename Tin>
__device__ __forceinline__ void store2(Tin* p, float a, float b);
template <>
__device__ __forceinline__ void store2<float>(float* p, float a, float b) {
    *reinterpret_cast<float2*>(p) = make_float2(a, b);
}
template <>
__device__ __forceinline__ void store2<bf16_t>(bf16_t* p, float a, float b) {
    *reinterpret_cast<uint32_t*>(p) =
        (uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

// Number of the sequence that token t belongs to (cu non-decreasing, t < cu[n]).
__device__ __forceinline__ int seq_of(const int32_t* cu, int n_seqs, int64_t t) {
    int lo = 0, hi = n_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)cu[mid] <= t) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// grid: (ceil(T / RUN), groups); block: 64 threads.  A group is one head of
// l2_head_dim channels, or 128 channels when there is no normalisation.  PAIRS
// channel pairs per lane (group width = 128 * PAIRS).
template <typename Tin, int PAIRS>
__global__ void __launch_bounds__(64)
conv_prefill_kernel(const Tin* __restrict__ x, const float* __restrict__ w,
                    const int32_t* __restrict__ cu, int n_seqs, int64_t T, int channels,
                    int group, int l2, float eps, const Tin* __restrict__ tail_in,
                    Tin* __restrict__ y) {
    const int lane = threadIdx.x;
    const int64_t t_begin = (int64_t)blockIdx.x * RUN;
    const int c_base = blockIdx.y * group;
    int64_t t_end = t_begin + RUN;
    if (t_end > T) t_end = T;

    int ci[PAIRS];
    bool act[PAIRS];
    float w0[PAIRS][2], w1[PAIRS][2], w2[PAIRS][2], w3[PAIRS][2];
#pragma unroll
    for (int p = 0; p < PAIRS; ++p) {
        const int off = 2 * (lane + 64 * p);
        act[p] = off < group;
        ci[p] = c_base + (act[p] ? off : 0);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const float4 ww = act[p] ? *reinterpret_cast<const float4*>(w + (size_t)(ci[p] + u) * 4)
                                     : make_float4(0.f, 0.f, 0.f, 0.f);
            w0[p][u] = ww.x; w1[p][u] = ww.y; w2[p][u] = ww.z; w3[p][u] = ww.w;
        }
    }

    int n = seq_of(cu, n_seqs, t_begin);
    int64_t s_start = cu[n], s_next = cu[n + 1];
    while (s_next <= t_begin && n + 1 < n_seqs) {  // skip empty sequences
        ++n;
        s_start = cu[n];
        s_next = cu[n + 1];
    }
    // window h1 = x_{t-3}, h2 = x_{t-2}, h3 = x_{t-1} for the first token
    float h1[PAIRS][2], h2[PAIRS][2], h3[PAIRS][2];
    auto hist = [&](int64_t t, int p, float& a, float& b) {
        // input at absolute token t (< the current token) of sequence n
        if (t >= s_start && t >= 0) {
            load2<Tin>(x + (size_t)t * channels + ci[p], a, b);
        } else if (tail_in) {
            int64_t m = 3 - (s_start - t);  // tail slot 0..2
            m = m < 0 ? 0 : (m > 2 ? 2 : m);
            load2<Tin>(tail_in + ((size_t)n * 3 + m) * channels + ci[p], a, b);
        } else {
            a = 0.f;
            b = 0.f;
        }
    };
#pragma unroll
    for (int p = 0; p < PAIRS; ++p) {
        if (act[p]) {
            hist(t_begin - 3, p, h1[p][0], h1[p][1]);
            hist(t_begin - 2, p, h2[p][0], h2[p][1]);
            hist(t_begin - 1, p, h3[p][0], h3[p][1]);
        } else {
            h1[p][0] = h1[p][1] = h2[p][0] = h2[p][1] = h3[p][0] = h3[p][1] = 0.f;
        }
    }

    for (int64_t t = t_begin; t < t_end; ++t) {
        if (t >= s_next) {  // a new sequence starts here: reload the window from its tail
            while (n + 1 < n_seqs && (int64_t)cu[n + 1] <= t) ++n;
            s_start = cu[n];
            s_next = cu[n + 1];
#pragma unroll
            for (int p = 0; p < PAIRS; ++p) {
                if (act[p]) {
                    hist(t - 3, p, h1[p][0], h1[p][1]);
                    hist(t - 2, p, h2[p][0], h2[p][1]);
                    hist(t - 1, p, h3[p][0], h3[p][1]);
                }
            }
        }
        float yv[PAIRS][2];
        float ss = 0.f;
#pragma unroll
        for (int p = 0; p < PAIRS; ++p) {
            float x0 = 0.f, x1 = 0.f;
            if (act[p]) load2<Tin>(x + (size_t)t * channels + ci[p], x0, x1);
            yv[p][0] = w0[p][0] * h1[p][0] + w1[p][0] * h2[p][0] + w2[p][0] * h3[p][0] +
                       w3[p][0] * x0;
            yv[p][1] = w0[p][1] * h1[p][1] + w1[p][1] * h2[p][1] + w2[p][1] * h3[p][1] +
                       w3[p][1] * x1;
            h1[p][0] = h2[p][0]; h1[p][1] = h2[p][1];
            h2[p][0] = h3[p][0]; h2[p][1] = h3[p][1];
            h3[p][0] = x0; h3[p][1] = x1;
            ss += yv[p][0] * yv[p][0] + yv[p][1] * yv[p][1];
        }
        float scale = 1.f;
        if (l2) scale = rsqrtf(wave_sum(ss) + eps);
#pragma unroll
        for (int p = 0; p < PAIRS; ++p)
            if (act[p])
                store2<Tin>(y + (size_t)t * channels + ci[p], yv[p][0] * scale, yv[p][1] * scale);
    }
}

// ---------------------------------------------------------------- prefill, wide
// The same convolution with one 16-byte access per lane and row: VC = 8 bf16 or
// 4 fp32 channels per lane, 256 lanes per workgroup.  A head of l2_head_dim
// channels is GL = l2_head_dim / VC consecutive lanes (a power of two up to a
// wave), so its sum of squares is a butterfly over those lanes.  Used when the
// shape allows it; the kernel above covers the rest.
template <typename Tin>
struct Vec16;
// 16 bytes with the non-temporal hint: x and y stream through once.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4_t load16_nt(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ void store16_nt(void* p, u32x4_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

template <>
struct Vec16<bf16_t> {
    static constexpr int VC = 8;
    static __device__ __forceinline__ void unpack(u32x4_t v, float (&x)[8]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = bf16_bits_to_f32(v[e] & 0xffffu);
            x[2 * e + 1] = bf16_bits_to_f32(v[e] >> 16);
        }
    }
    static __device__ __forceinline__ void load(const bf16_t* p, float (&x)[8]) {
        const uint4 v = *reinterpret_cast<const uint4*>(p);
        unpack(u32x4_t{v.x, v.y, v.z, v.w}, x);
    }
    static __device__ __forceinline__ void store(bf16_t* p, const float (&x)[8]) {
        u32x4_t u;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            u[e] = (uint32_t)f32_to_bf16_bits(x[2 * e]) |
                   ((uint32_t)f32_to_bf16_bits(x[2 * e + 1]) << 16);
        store16_nt(p, u);
    }
};
template <>
struct Vec16<float> {
    static constexpr int VC = 4;
    static __device__ __forceinline__ void unpack(u32x4_t v, float (&x)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(v[e]);
    }
    static __device__ __forceinline__ void load(const float* p, float (&x)[4]) {
        const float4 v = *reinterpret_cast<const float4*>(p);
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    }
    static __device__ __forceinline__ void store(float* p, const float (&x)[4]) {
        store16_nt(p, u32x4_t{__float_as_uint(x[0]), __float_as_uint(x[1]),
                              __float_as_uint(x[2]), __float_as_uint(x[3])});
    }
};

// x moved between lanes by a DPP pattern within each row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of gl lanes (gl a power of two, at most 64), every
// lane receiving its group's sum: quad swaps, then the half-row and row
// mirrors pair quads and half-rows; across rows, lane shuffles.
__device__ __forceinline__ float group_sum(float x, int gl) {
    if (gl >= 2) x += dpp_f<0xB1>(x);   // quad_perm [1, 0, 3, 2]
    if (gl >= 4) x += dpp_f<0x4E>(x);   // quad_perm [2, 3, 0, 1]
    if (gl >= 8) x += dpp_f<0x141>(x);  // row_half_mirror
    if (gl >= 16) x += dpp_f<0x140>(x); // row_mirror
    if (gl >= 32) x += __shfl_xor(x, 16);
    if (gl >= 64) x += __shfl_xor(x, 32);
    return x;
}

// grid: (ceil(T / run), ceil(channels / (256 VC))); block: 256 threads.
// gl: lanes per normalised head (0: no normalisation).  run: tokens per
// workgroup (longer runs re-read the 3-token history less often).
template <typename Tin>
__global__ void __launch_bounds__(256)
conv_prefill_wide_kernel(const Tin* __restrict__ x, const float* __restrict__ w,
                         const int32_t* __restrict__ cu, int n_seqs, int64_t T, int channels,
                         int gl, int run, float eps, const Tin* __restrict__ tail_in,
                         Tin* __restrict__ y) {
    constexpr int VC = Vec16<Tin>::VC;
    const int64_t t_begin = (int64_t)blockIdx.x * run;
    const int c = (blockIdx.y * 256 + threadIdx.x) * VC;
    const bool act = c < channels;
    const int ci = act ? c : 0;
    int64_t t_end = t_begin + run;
    if (t_end > T) t_end = T;

    float w0[VC], w1[VC], w2[VC], w3[VC];
#pragma unroll
    for (int u = 0; u < VC; ++u) {
        const float4 ww = act ? *reinterpret_cast<const float4*>(w + (size_t)(ci + u) * 4)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
        w0[u] = ww.x; w1[u] = ww.y; w2[u] = ww.z; w3[u] = ww.w;
    }
    int n = seq_of(cu, n_seqs, t_begin);
    int64_t s_start = cu[n], s_next = cu[n + 1];
    while (s_next <= t_begin && n + 1 < n_seqs) {  // skip empty sequences
        ++n;
        s_start = cu[n];
        s_next = cu[n + 1];
    }
    // input at absolute token t (< the current token) of sequence n
    auto hist = [&](int64_t t, float (&h)[VC]) {
        if (act && t >= s_start && t >= 0) {
            Vec16<Tin>::load(x + (size_t)t * channels + ci, h);
        } else if (act && tail_in) {
            int64_t m = 3 - (s_start - t);  // tail slot 0..2
            m = m < 0 ? 0 : (m > 2 ? 2 : m);
            Vec16<Tin>::load(tail_in + ((size_t)n * 3 + m) * channels + ci, h);
        } else {
#pragma unroll
            for (int u = 0; u < VC; ++u) h[u] = 0.f;
        }
    };
    float h1[VC], h2[VC], h3[VC];  // x_{t-3}, x_{t-2}, x_{t-1}
    hist(t_begin - 3, h1);
    hist(t_begin - 2, h2);
    hist(t_begin - 1, h3);
    // one token: conv, optional L2 norm, store y[t]
    auto step = [&](float (&xv)[VC], int64_t t) {
        float yv[VC];
        float ss = 0.f;
#pragma unroll
        for (int u = 0; u < VC; ++u) {
            yv[u] = w0[u] * h1[u] + w1[u] * h2[u] + w2[u] * h3[u] + w3[u] * xv[u];
            h1[u] = h2[u];
            h2[u] = h3[u];
            h3[u] = xv[u];
            ss += yv[u] * yv[u];
        }
        if (gl) {
            ss = group_sum(ss, gl);
            const float scale = rsqrtf(ss + eps);
#pragma unroll
            for (int u = 0; u < VC; ++u) yv[u] *= scale;
        }
        if (act) Vec16<Tin>::store(y + (size_t)t * channels + ci, yv);
    };
    // Blocks of TB tokens inside one sequence load their TB rows of x first
    // (non-temporal), then run the steps; a block that would cross the run's
    // end or a sequence start goes token by token.  The test is uniform over
    // the workgroup, so the group sums' lanes stay together.  Measured on
    // 3 x 32768 x 8192 bf16: 0.649 -> 0.615 ms (blocks of 8: 0.624; blocks
    // without the hints: 0.637).
    constexpr int TB = 4;
    int64_t t = t_begin;
    while (t < t_end) {
        if (t + TB <= t_end && t + TB <= s_next) {
            u32x4_t raw[TB];
#pragma unroll
            for (int j = 0; j < TB; ++j)
                raw[j] = act ? load16_nt(x + (size_t)(t + j) * channels + ci)
                             : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
            for (int j = 0; j < TB; ++j) {
                float xv[VC];
                Vec16<Tin>::unpack(raw[j], xv);
                step(xv, t + j);
            }
            t += TB;
            continue;
        }
        if (t >= s_next) {  // a new sequence starts here: reload the window from its tail
            while (n + 1 < n_seqs && (int64_t)cu[n + 1] <= t) ++n;
            s_start = cu[n];
            s_next = cu[n + 1];
            hist(t - 3, h1);
            hist(t - 2, h2);
            hist(t - 1, h3);
        }
        float xv[VC];
        if (act) Vec16<Tin>::load(x + (size_t)t * channels + ci, xv);
        else
#pragma unroll
            for (int u = 0; u < VC; ++u) xv[u] = 0.f;
        step(xv, t);
        ++t;
    }
}

// Tail update: one thread per (sequence, channel); reads the old tail in full
// before writing, so tail_out may equal tail_in.
template <typename Tin>
__global__ void __launch_bounds__(256)
conv_tail_kernel(const Tin* __restrict__ x, const int32_t* __restrict__ cu, int n_seqs,
                 int64_t T, int channels, const Tin* tail_in, Tin* tail_out) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)n_seqs * channels) return;
    const int n = (int)(idx / channels), c = (int)(idx % channels);
    int64_t b, e;
    seq_range(cu, n, T, b, e);
    float hv[3];
#pragma unroll
    for (int m = 0; m < 3; ++m)
        hv[m] = tail_in ? In<Tin>::load1(tail_in + ((size_t)n * 3 + m) * channels + c) : 0.f;
    const int64_t len = e - b;
    float nv[3];
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        // new slot m holds history position len + m (positions 0..2 are the old tail)
        const int64_t pos = len + m;
        nv[m] = pos >= 3 ? In<Tin>::load1(x + (size_t)(b + pos - 3) * channels + c) : hv[pos];
    }
#pragma unroll
    for (int m = 0; m < 3; ++m) In<Tin>::store1(tail_out + ((size_t)n * 3 + m) * channels + c, nv[m]);
}

template <typename Tin>
static hipError_t conv_prefill_t(const void* x, const float* w, const int32_t* cu, int n_seqs,
                                 int64_t T, int channels, int l2_head_dim, float eps,
                                 const void* tail_in, void* tail_out, void* y,
                                 hipStream_t stream) {
    constexpr int VC = Vec16<Tin>::VC;
    const int gl = l2_head_dim / VC;
    // 16-byte accesses: the entry point has checked every pointer for 16-byte
    // alignment, so rows are aligned when channels is a multiple of VC
    const bool wide = channels % VC == 0 &&
                      (l2_head_dim == 0 || (l2_head_dim % VC == 0 && gl <= 64 && !(gl & (gl - 1))));
    if (T > 0 && n_seqs > 0 && wide) {
        // the longest run (fewest history re-reads) that still gives >= 768
        // workgroups, three per CU; measured on 8192 channels of bf16 (L2 norm):
        // T = 32768 with runs of 16, 64, 128, 256 tokens took 0.30, 0.26, 0.255,
        // 0.38 ms; T = 24576 with runs of 64 and 128, 0.204 and 0.185 ms; T =
        // 8192 with runs of 32 and 64, 0.057 and 0.064 ms
        const int64_t cblocks = (channels + 256 * VC - 1) / (256 * VC);
        int run = 128;
        while (run > 16 && ((T + run - 1) / run) * cblocks < 768) run >>= 1;
        const int64_t runs = (T + run - 1) / run;
        const dim3 grid((unsigned)runs, (unsigned)cblocks);
        hipLaunchKernelGGL((conv_prefill_wide_kernel<Tin>), grid, dim3(256), 0, stream,
                           (const Tin*)x, w, cu, n_seqs, T, channels, gl, run, eps,
                           (const Tin*)tail_in, (Tin*)y);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    } else if (T > 0 && n_seqs > 0) {
        const int group = l2_head_dim > 0 ? l2_head_dim : (channels % 128 == 0 ? 128 : channels);
        const int pairs = (group + 127) / 128;
        const int64_t runs = (T + RUN - 1) / RUN;
        const dim3 grid((unsigned)runs, (unsigned)(channels / group));
        const int l2 = l2_head_dim > 0;
        if (pairs == 1)
            hipLaunchKernelGGL((conv_prefill_kernel<Tin, 1>), grid, dim3(64), 0, stream,
                               (const Tin*)x, w, cu, n_seqs, T, channels, group, l2, eps,
                               (const Tin*)tail_in, (Tin*)y);
        else if (pairs == 2)
            hipLaunchKernelGGL((conv_prefill_kernel<Tin, 2>), grid, dim3(64), 0, stream,
                               (const Tin*)x, w, cu, n_seqs, T, channels, group, l2, eps,
                               (const Tin*)tail_in, (Tin*)y);
        else
            return hipErrorInvalidValue;
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (tail_out && n_seqs > 0) {
        const int64_t total = (int64_t)n_seqs * channels;
        hipLaunchKernelGGL((conv_tail_kernel<Tin>), dim3((unsigned)((total + 255) / 256)),
                           dim3(256), 0, stream, (const Tin*)x, cu, n_seqs, T, channels,
                           (const Tin*)tail_in, (Tin*)tail_out);
        return hipGetLastError();
    }
    return hipSuccess;
}

hipError_t launch_short_conv_prefill(const void* x, const float* w, kda_dtype dtype,
                                     const int32_t* cu, int n_seqs, int64_t T, int channels,
                                     int l2_head_dim, float l2_eps, const void* tail_in,
                                     void* tail_out, void* y, hipStream_t stream) {
    if (dtype == KDA_BF16)
        return conv_prefill_t<bf16_t>(x, w, cu, n_seqs, T, channels, l2_head_dim, l2_eps,
                                      tail_in, tail_out, y, stream);
    return conv_prefill_t<float>(x, w, cu, n_seqs, T, channels, l2_head_dim, l2_eps, tail_in,
                                 tail_out, y, stream);
}

// ---------------------------------------------------------------- decode
// grid: (B, channels / group); block: 64 threads; PAIRS channel pairs per lane.
template <typename Tin, int PAIRS>
__global__ void __launch_bounds__(64)
conv_decode_kernel(const Tin* __restrict__ x, const float* __restrict__ w, Tin* tail,
                   int64_t n_slots, const int32_t* __restrict__ slot_idx, int channels,
                   int group, int l2, float eps, Tin* __restrict__ y) {
    const int lane = threadIdx.x;
    const int b = blockIdx.x;
    const int c_base = blockIdx.y * group;
    const int64_t slot = slot_idx ? (int64_t)slot_idx[b] : (int64_t)b;
    const bool ok = slot >= 0 && slot < n_slots;
    float yv[PAIRS][2];
    float ss = 0.f;
#pragma unroll
    for (int p = 0; p < PAIRS; ++p) {
        const int off = 2 * (lane + 64 * p);
        yv[p][0] = yv[p][1] = 0.f;
        if (off >= group || !ok) continue;
        const int c = c_base + off;
        float x0, x1, a0, a1, b0, b1, d0, d1;
        load2<Tin>(x + (size_t)b * channels + c, x0, x1);
        Tin* tp = tail + (size_t)slot * 3 * channels + c;
        load2<Tin>(tp, a0, a1);
        load2<Tin>(tp + channels, b0, b1);
        load2<Tin>(tp + 2 * (size_t)channels, d0, d1);
        const float4 wa = *reinterpret_cast<const float4*>(w + (size_t)c * 4);
        const float4 wb = *reinterpret_cast<const float4*>(w + (size_t)(c + 1) * 4);
        yv[p][0] = wa.x * a0 + wa.y * b0 + wa.z * d0 + wa.w * x0;
        yv[p][1] = wb.x * a1 + wb.y * b1 + wb.z * d1 + wb.w * x1;
        ss += yv[p][0] * yv[p][0] + yv[p][1] * yv[p][1];
        store2<Tin>(tp, b0, b1);
        store2<Tin>(tp + channels, d0, d1);
        store2<Tin>(tp + 2 * (size_t)channels, x0, x1);
    }
    float scale = 1.f;
    if (l2) scale = rsqrtf(wave_sum(ss) + eps);
    if (!ok) scale = __builtin_nanf("");
#pragma unroll
    for (int p = 0; p < PAIRS; ++p) {
        const int off = 2 * (lane + 64 * p);
        if (off < group)
            store2<Tin>(y + (size_t)b * channels + c_base + off, ok ? yv[p][0] * scale : scale,
                        ok ? yv[p][1] * scale : scale);
    }
}

template <typename Tin>
static hipError_t conv_decode_t(const void* x, const float* w, void* tail, int64_t n_slots,
                                const int32_t* slot_idx, int B, int channels, int l2_head_dim,
                                float eps, void* y, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    const int group = l2_head_dim > 0 ? l2_head_dim : (channels % 128 == 0 ? 128 : channels);
    const int pairs = (group + 127) / 128;
    const dim3 grid((unsigned)B, (unsigned)(channels / group));
    const int l2 = l2_head_dim > 0;
    if (pairs == 1)
        hipLaunchKernelGGL((conv_decode_kernel<Tin, 1>), grid, dim3(64), 0, stream,
                           (const Tin*)x, w, (Tin*)tail, n_slots, slot_idx, channels, group, l2,
                           eps, (Tin*)y);
    else if (pairs == 2)
        hipLaunchKernelGGL((conv_decode_kernel<Tin, 2>), grid, dim3(64), 0, stream,
                           (const Tin*)x, w, (Tin*)tail, n_slots, slot_idx, channels, group, l2,
                           eps, (Tin*)y);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_short_conv_decode(const void* x, const float* w, kda_dtype dtype, void* tail,
                                    int64_t n_slots, const int32_t* slot_idx, int B,
                                    int channels, int l2_head_dim, float l2_eps, void* y,
                                    hipStream_t stream) {
    if (dtype == KDA_BF16)
        return conv_decode_t<bf16_t>(x, w, tail, n_slots, slot_idx, B, channels, l2_head_dim,
                                     l2_eps, y, stream);
    return conv_decode_t<float>(x, w, tail, n_slots, slot_idx, B, channels, l2_head_dim, l2_eps,
                                y, stream);
}

}  // namespace kda
