// Internal declarations shared by the HIP sources of libkda.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

// ---------------------------------------------------------------- vector types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct bf16_t {
    uint16_t bits;
};

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}

// Load n consecutive input elements (fp32 or bf16) as fp32.
template <typename Tin>
struct In;

template <>
struct In<float> {
    static __device__ __forceinline__ void load4(const float* p, float (&x)[4]) {
        float4 v = *reinterpret_cast<const float4*>(p);
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    }
    static __device__ __forceinline__ float load1(const float* p) { return *p; }
    static __device__ __forceinline__ void store1(float* p, float x) { *p = x; }
    static __device__ __forceinline__ void store4(float* p, const float (&x)[4]) {
        *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
    }
};

template <>
struct In<bf16_t> {
    static __device__ __forceinline__ void load4(const bf16_t* p, float (&x)[4]) {
        uint2 v = *reinterpret_cast<const uint2*>(p);
        x[0] = bf16_bits_to_f32(v.x & 0xffffu);
        x[1] = bf16_bits_to_f32(v.x >> 16);
        x[2] = bf16_bits_to_f32(v.y & 0xffffu);
        x[3] = bf16_bits_to_f32(v.y >> 16);
    }
    static __device__ __forceinline__ float load1(const bf16_t* p) {
        return bf16_bits_to_f32(p->bits);
    }
    static __device__ __forceinline__ void store1(bf16_t* p, float x) {
        p->bits = f32_to_bf16_bits(x);
    }
    static __device__ __forceinline__ void store4(bf16_t* p, const float (&x)[4]) {
        uint2 v;
        v.x = (uint32_t)f32_to_bf16_bits(x[0]) | ((uint32_t)f32_to_bf16_bits(x[1]) << 16);
        v.y = (uint32_t)f32_to_bf16_bits(x[2]) | ((uint32_t)f32_to_bf16_bits(x[3]) << 16);
        *reinterpret_cast<uint2*>(p) = v;
    }
};

// Clamp a sequence's [begin, end) to [0, T) so that a device copy of
// cu_seqlens that disagrees with the validated host copy can never send an
// access outside the buffers.
__device__ __forceinline__ void seq_range(const int32_t* cu, int n, int64_t T, int64_t& b,
                                          int64_t& e) {
    int64_t lo = cu[n], hi = cu[n + 1];
    lo = lo < 0 ? 0 : (lo > T ? T : lo);
    hi = hi < lo ? lo : (hi > T ? T : hi);
    b = lo;
    e = hi;
}

// ---------------------------------------------------------------- snapshots
// Chunk-aligned state snapshots of a prefill: entry [n][j] of ptr
// ([n_seqs, capacity, H, D, D] fp32) is sequence n's state after its first
// (j + 1) * interval tokens.  ptr == nullptr: none taken.
struct Snapshots {
    float* ptr;
    int interval;  // tokens, a multiple of the chunk
    int capacity;  // snapshots per sequence in the buffer
};

// Head h's D x D state of snapshot j of sequence n, or nullptr when no snapshot
// is taken after `done` tokens of a sequence of `len` tokens.
__device__ __forceinline__ float* snapshot_at(const Snapshots& sn, int n, int h, int H, int D,
                                              int64_t done, int64_t len) {
    if (!sn.ptr || done > len || done % sn.interval) return nullptr;
    const int64_t j = done / sn.interval - 1;
    if (j < 0 || j >= sn.capacity) return nullptr;
    return sn.ptr + (((size_t)n * sn.capacity + j) * H + h) * (size_t)D * D;
}

// ---------------------------------------------------------------- decay inputs
// How a call gives the decay alpha = exp(g) and the write strength beta.
//   GATE_CH   g: [tokens, H, D] fp32 log decay per key channel; beta as given.
//   GATE_HEAD g: [tokens, H] fp32, one log decay per head; beta as given.
//   GATE_PROJ g: [tokens, H, D] decay projection f in the q/k/v dtype, with
//             one log rate a_log[h] per head: g = -exp(a_log[h]) softplus(f);
//             beta holds logits: beta = sigmoid(beta).
enum GateMode : int { GATE_CH = 0, GATE_HEAD = 1, GATE_PROJ = 2 };
struct Gate {
    const void* g;
    const float* a_log;  // [H], GATE_PROJ only
    int mode;
};

// log2 of the decay from the projection: -A softplus(f) / ln 2, with
// softplus(f) = max(f, 0) + ln(1 + e^{-|f|}).
__device__ __forceinline__ float proj_log2_decay(float f, float A) {
    const float LOG2E_ = 1.4426950408889634f;
    const float sp2 = fmaxf(f, 0.f) * LOG2E_ +
                      __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-fabsf(f) * LOG2E_));
    return -A * sp2;
}
__device__ __forceinline__ float sigmoid_f(float x) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
}

// Window of global memory as a buffer resource: loads past num_bytes read zero,
// stores past it are dropped.  The base is wave-uniform (scalar registers), so
// lanes address it with 32-bit offsets instead of 64-bit pointers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t window(const void* base, int num_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, num_bytes,
                                             0x00020000);
}
// Cache-policy operand of buffer loads and stores: non-temporal (streamed once).
constexpr int BUF_NT = 2;

// The calling thread's error text (what kda_last_error_detail returns).
void set_error_detail(const char* fmt, ...);

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; arguments are already checked.
// out_gate, where taken: the output gate's projection z in o's layout and dtype,
// or NULL; with it every output is multiplied by sigmoid(z) before it is stored.
// n_elems elements of state_dtype: zeros (src NULL) or src converted.
hipError_t launch_state_init(void* state, kda_dtype state_dtype, int64_t n_elems, const void* src,
                             kda_dtype src_dtype, hipStream_t stream);

// n_tok consecutive tokens per sequence; token_states may be NULL; state and
// token_states hold state_dtype elements.
// out_gate (o's layout and dtype) or NULL: o is multiplied by sigmoid(out_gate).
hipError_t launch_decode(const void* q, const void* k, const void* v, Gate gate,
                         const float* beta, kda_dtype dtype, void* state,
                         kda_dtype state_dtype, int64_t n_slots, const int32_t* slot_idx, int B,
                         int n_tok, int H, int d, void* token_states, const void* out_gate,
                         void* o, hipStream_t stream);

hipError_t launch_prefill_vector(const void* q, const void* k, const void* v, Gate gate,
                                 const float* beta, kda_dtype dtype, const int32_t* cu,
                                 int n_seqs, int64_t T, int H, int d, int chunk,
                                 const float* s0, float* s_final, const void* out_gate, void* o,
                                 Snapshots snap, hipStream_t stream);

// bf16, d = 128, chunk = 64, one fused kernel (no workspace).
hipError_t launch_prefill_fused(const void* q, const void* k, const void* v, Gate gate,
                                const float* beta, const int32_t* cu, int n_seqs,
                                int64_t T, int H, const float* s0, float* s_final,
                                const void* out_gate, void* o, Snapshots snap, hipStream_t stream);

// bf16, d = 128, chunk = 64, two kernels through a caller workspace of
// prefill_split_workspace_bytes(n_seqs, H) bytes; cu_host: the validated host
// copy of cu_seqlens (for the window plan).
size_t prefill_split_workspace_bytes(int n_seqs, int H);
// The least workspace the two-kernel path runs on: one tile per sequence and
// head (windows of one chunk where nothing more fits).
size_t prefill_split_workspace_bytes_least(int n_seqs, int H);

// The library's static device scratch (kda_noalloc.hip): its size, and its
// address on the device that `stream` runs on (looked up once per device).
size_t static_scratch_bytes();
hipError_t static_scratch(hipStream_t stream, void** out);
size_t prefill_split_workspace_bytes_batch(const int32_t* cu_host, int n_seqs, int H);
hipError_t launch_prefill_split(const void* q, const void* k, const void* v, Gate gate,
                                const float* beta, const int32_t* cu, const int32_t* cu_host,
                                int n_seqs, int64_t T, int H, const float* s0, float* s_final,
                                const void* out_gate, void* o, Snapshots snap, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

hipError_t launch_short_conv_prefill(const void* x, const float* w, kda_dtype dtype,
                                     const int32_t* cu, int n_seqs, int64_t T, int channels,
                                     int l2_head_dim, float l2_eps, const void* tail_in,
                                     void* tail_out, void* y, hipStream_t stream);

// bytes (a multiple of 16) from src to dst, both 16-byte aligned, not overlapping.
hipError_t launch_device_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);

hipError_t launch_short_conv_decode(const void* x, const float* w, kda_dtype dtype,
                                    void* tail, int64_t n_slots, const int32_t* slot_idx, int B,
                                    int channels, int l2_head_dim, float l2_eps, void* y,
                                    hipStream_t stream);

}  // namespace kda
