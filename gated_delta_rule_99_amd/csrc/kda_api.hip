// C ABI of libkda.so: host-side argument checks and kernel dispatch.
// Every check runs before anything is enqueued; a failed check returns a status
// and leaves the stream untouched.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "kda_internal.h"

namespace {

thread_local char g_detail[512];

kda_status fail(kda_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
    va_end(ap);
    return s;
}

kda_status hip_status(hipError_t err, const char* what) {
    if (err == hipSuccess) return KDA_OK;
    return fail(KDA_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(err), (int)err);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }  // NULL counts as aligned

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

bool supported_d(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// A dispatch counts its work-items in 32 bits: workgroups x threads per
// workgroup must stay below 2^32 along the grid's first dimension.
bool dispatch_fits(int64_t workgroups, int threads) {
    return workgroups <= (int64_t)0xffffffffll / threads;
}

// Shapes that run on the matrix cores.
bool mfma_shape(kda_dtype dtype, int dk, int dv, int chunk) {
    return dtype == KDA_BF16 && dk == 128 && dv == 128 && chunk == 64;
}

size_t elem_size(kda_dtype dt) { return dt == KDA_BF16 ? 2 : 4; }

// Gate layout and a_log checks shared by the recurrence entry points.
kda_status check_gate(const char* fn, kda_gate gate, const float* a_log) {
    if (gate != KDA_GATE_CHANNEL && gate != KDA_GATE_HEAD && gate != KDA_GATE_PROJ)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown gate layout %d", fn, (int)gate);
    if (gate == KDA_GATE_PROJ && (!a_log || ((uintptr_t)a_log & 3u)))
        return fail(KDA_ERR_INVALID_ARGUMENT,
                    "%s: KDA_GATE_PROJ needs a_log, non-NULL and 4-byte aligned", fn);
    if (gate != KDA_GATE_PROJ && a_log)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: a_log is only taken with KDA_GATE_PROJ", fn);
    return KDA_OK;
}

// Bytes of g for `tokens` tokens: fp32 per channel or per head, or the
// projection in the q/k/v dtype.
size_t gate_bytes(kda_gate gate, size_t tokens, int H, int dk, kda_dtype dtype) {
    if (gate == KDA_GATE_HEAD) return tokens * H * 4;
    return tokens * H * dk * (gate == KDA_GATE_PROJ ? elem_size(dtype) : 4);
}

kda::Gate make_gate(const void* g, const float* a_log, kda_gate gate) {
    return kda::Gate{g, a_log,
                     gate == KDA_GATE_HEAD   ? kda::GATE_HEAD
                     : gate == KDA_GATE_PROJ ? kda::GATE_PROJ
                                             : kda::GATE_CH};
}

// Common head-shape checks.  Returns KDA_OK or an error with detail set.
kda_status check_heads(const char* fn, int H, int dk, int dv) {
    if (H <= 0 || dk <= 0 || dv <= 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: H, dk, dv must be positive (got %d, %d, %d)",
                    fn, H, dk, dv);
    if (dk != dv)
        return fail(KDA_ERR_UNSUPPORTED, "%s: dk != dv (%d, %d) is not implemented", fn, dk, dv);
    if (!supported_d(dk))
        return fail(KDA_ERR_UNSUPPORTED, "%s: head dim %d not in {16, 32, 64, 128}", fn, dk);
    return KDA_OK;
}

kda_status check_cu(const char* fn, const int32_t* cu_host, int n_seqs, int64_t* T_out) {
    if (n_seqs < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: n_seqs < 0", fn);
    if (!cu_host) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: cu_seqlens_host is NULL", fn);
    if (cu_host[0] != 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: cu_seqlens[0] = %d, expected 0", fn,
                    cu_host[0]);
    for (int n = 0; n < n_seqs; ++n)
        if (cu_host[n + 1] < cu_host[n])
            return fail(KDA_ERR_INVALID_ARGUMENT,
                        "%s: cu_seqlens decreases at %d (%d -> %d)", fn, n, cu_host[n],
                        cu_host[n + 1]);
    *T_out = cu_host[n_seqs];
    return KDA_OK;
}

}  // namespace

namespace kda {
void set_error_detail(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
    va_end(ap);
}
}  // namespace kda

extern "C" {

const char* kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
        case KDA_ERR_HIP: return "KDA_ERR_HIP";
        case KDA_ERR_WORKSPACE_TOO_SMALL: return "KDA_ERR_WORKSPACE_TOO_SMALL";
    }
    return "KDA_ERR_UNKNOWN";
}

const char* kda_last_error_detail(void) { return g_detail; }

size_t kda_state_bytes(int H, int dk, int dv, kda_dtype state_dtype) {
    if (H <= 0 || dk <= 0 || dv <= 0) return 0;
    if (state_dtype != KDA_F32 && state_dtype != KDA_BF16) return 0;
    return elem_size(state_dtype) * (size_t)H * (size_t)dk * (size_t)dv;
}

kda_status kda_state_init(void* state, kda_dtype state_dtype, int64_t n_slots, int H, int dk,
                          int dv, const void* src, kda_dtype src_dtype, hipStream_t stream) {
    const char* fn = "kda_state_init";
    g_detail[0] = 0;
    if (state_dtype != KDA_F32 && state_dtype != KDA_BF16)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown state dtype %d", fn, (int)state_dtype);
    if (src && src_dtype != KDA_F32 && src_dtype != KDA_BF16)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown src dtype %d", fn, (int)src_dtype);
    if (kda_status s = check_heads(fn, H, dk, dv)) return s;
    if (n_slots < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: n_slots < 0", fn);
    if (n_slots == 0) return KDA_OK;
    if (!state || !aligned16(state) || (src && !aligned16(src)))
        return fail(KDA_ERR_INVALID_ARGUMENT,
                    "%s: state/src must be non-NULL and 16-byte aligned", fn);
    const size_t bytes = (size_t)n_slots * kda_state_bytes(H, dk, dv, state_dtype);
    const size_t src_bytes = src ? (size_t)n_slots * kda_state_bytes(H, dk, dv, src_dtype) : 0;
    if (src && overlaps(state, bytes, src, src_bytes))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: src overlaps state", fn);
    return hip_status(kda::launch_state_init(state, state_dtype,
                                             (int64_t)n_slots * H * dk * dv, src, src_dtype,
                                             stream),
                      "kda_state_init launch");
}

// The body of kda_prefill_chunked and kda_prefill_chunked_noalloc.  ws_floor:
// the smallest workspace accepted for the matrix-core shapes: the size
// kda_prefill_workspace_bytes returns (kda_prefill_chunked), or the least the
// two-kernel path can run on, one tile per sequence and head (the static
// scratch of kda_prefill_chunked_noalloc; windows are then shorter).
static kda_status prefill_entry(const char* fn, const void* q, const void* k, const void* v,
                                const void* g, const float* beta, kda_dtype dtype, kda_gate gate,
                                const float* a_log, const int32_t* cu_seqlens_dev,
                                const int32_t* cu_seqlens_host, int n_seqs, int H, int dk, int dv,
                                int chunk, const float* initial_state, float* final_state,
                                const void* out_gate, void* o, float* snapshots,
                                int snap_interval, int snap_capacity, void* workspace,
                                size_t workspace_bytes, bool floor_one_tile, hipStream_t stream) {
    g_detail[0] = 0;
    if (dtype != KDA_F32 && dtype != KDA_BF16)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", fn, (int)dtype);
    if (kda_status s = check_gate(fn, gate, a_log)) return s;
    if (kda_status s = check_heads(fn, H, dk, dv)) return s;
    if (chunk != 16 && chunk != 32 && chunk != 64)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: chunk %d not in {16, 32, 64}", fn, chunk);
    int64_t T = 0;
    if (kda_status s = check_cu(fn, cu_seqlens_host, n_seqs, &T)) return s;
    if (n_seqs == 0) return KDA_OK;
    if (!cu_seqlens_dev) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: cu_seqlens_dev is NULL", fn);
    const int d = dk;
    const int64_t blocks = (int64_t)n_seqs * H * (d == 128 ? 4 : (d < 32 ? 1 : d / 32));
    // prefill kernels take at most 1024 threads per workgroup
    if (!dispatch_fits(blocks, 1024))
        return fail(KDA_ERR_UNSUPPORTED,
                    "%s: %lld workgroups exceed 4194303 (32-bit dispatch size)", fn,
                    (long long)blocks);
    const size_t es = elem_size(dtype);
    const size_t n_qk = (size_t)T * H * d, n_bt = (size_t)T * H;
    const size_t gb = gate_bytes(gate, (size_t)T, H, d, dtype);
    const size_t ab = a_log ? (size_t)H * 4 : 0;
    const size_t sbytes = (size_t)n_seqs * kda_state_bytes(H, dk, dv, KDA_F32);
    if (T > 0) {
        if (!q || !k || !v || !g || !beta || !o)
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: q, k, v, g, beta and o are required", fn);
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(o) ||
            ((uintptr_t)beta & 3u))
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: misaligned tensor pointer", fn);
        if (!aligned16(out_gate))
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: misaligned out_gate", fn);
        if (overlaps(o, n_qk * es, q, n_qk * es) || overlaps(o, n_qk * es, k, n_qk * es) ||
            overlaps(o, n_qk * es, v, n_qk * es) || overlaps(o, n_qk * es, g, gb) ||
            overlaps(o, n_qk * es, beta, n_bt * 4) || overlaps(o, n_qk * es, a_log, ab) ||
            overlaps(o, n_qk * es, final_state, sbytes) ||
            overlaps(o, n_qk * es, initial_state, sbytes) ||
            overlaps(o, n_qk * es, out_gate, n_qk * es))
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: o overlaps another argument", fn);
        if (final_state && overlaps(final_state, sbytes, out_gate, n_qk * es))
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: final_state overlaps out_gate", fn);
    } else {
        out_gate = nullptr;
    }
    if ((initial_state && !aligned16(initial_state)) || (final_state && !aligned16(final_state)))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: misaligned state pointer", fn);
    if (initial_state && final_state && initial_state != final_state &&
        overlaps(initial_state, sbytes, final_state, sbytes))
        return fail(KDA_ERR_INVALID_ARGUMENT,
                    "%s: initial_state and final_state overlap without being equal", fn);
    if (final_state && T > 0 &&
        (overlaps(final_state, sbytes, q, n_qk * es) || overlaps(final_state, sbytes, k, n_qk * es) ||
         overlaps(final_state, sbytes, v, n_qk * es) || overlaps(final_state, sbytes, g, gb) ||
         overlaps(final_state, sbytes, a_log, ab)))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: final_state overlaps an input", fn);

    // snapshots: [n_seqs, snap_capacity, H, dk, dv] fp32
    if (snapshots) {
        if (snap_interval <= 0 || snap_interval % chunk)
            return fail(KDA_ERR_INVALID_ARGUMENT,
                        "%s: snap_interval %d must be a positive multiple of chunk %d", fn,
                        snap_interval, chunk);
        if (snap_capacity < 0)
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: snap_capacity < 0", fn);
        if (!aligned16(snapshots))
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: misaligned snapshots", fn);
        const size_t snb = (size_t)n_seqs * snap_capacity * kda_state_bytes(H, dk, dv, KDA_F32);
        if (overlaps(snapshots, snb, q, n_qk * es) || overlaps(snapshots, snb, k, n_qk * es) ||
            overlaps(snapshots, snb, v, n_qk * es) || overlaps(snapshots, snb, g, gb) ||
            overlaps(snapshots, snb, a_log, ab) ||
            overlaps(snapshots, snb, beta, n_bt * 4) || overlaps(snapshots, snb, o, n_qk * es) ||
            overlaps(snapshots, snb, initial_state, sbytes) ||
            overlaps(snapshots, snb, final_state, sbytes) ||
            overlaps(snapshots, snb, out_gate, n_qk * es) ||
            overlaps(snapshots, snb, workspace, workspace ? workspace_bytes : 0))
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: snapshots overlap another argument", fn);
        if (snap_capacity == 0) snapshots = nullptr;
    }
    const kda::Snapshots snap{snapshots, snapshots ? snap_interval : 0, snap_capacity};

    const bool mfma = mfma_shape(dtype, dk, dv, chunk);
    const size_t ws_need = !mfma          ? 0
                           : floor_one_tile ? kda::prefill_split_workspace_bytes_least(n_seqs, H)
                                            : kda::prefill_split_workspace_bytes(n_seqs, H);
    if (mfma && workspace) {
        if (workspace_bytes < ws_need)
            return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace of %zu bytes, %zu needed", fn,
                        workspace_bytes, ws_need);
        if (!aligned16(workspace))
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: misaligned workspace", fn);
        if (overlaps(workspace, workspace_bytes, q, n_qk * es) || overlaps(workspace, workspace_bytes, k, n_qk * es) ||
            overlaps(workspace, workspace_bytes, v, n_qk * es) || overlaps(workspace, workspace_bytes, g, gb) ||
            overlaps(workspace, workspace_bytes, a_log, ab) ||
            overlaps(workspace, workspace_bytes, beta, n_bt * 4) || overlaps(workspace, workspace_bytes, o, n_qk * es) ||
            overlaps(workspace, workspace_bytes, initial_state, sbytes) ||
            overlaps(workspace, workspace_bytes, final_state, sbytes) ||
            overlaps(workspace, workspace_bytes, out_gate, n_qk * es))
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: workspace overlaps another argument", fn);
    }

    const kda::Gate gt = make_gate(g, a_log, gate);
    hipError_t err;
    if (mfma && workspace) {
        err = kda::launch_prefill_split(q, k, v, gt, beta, cu_seqlens_dev, cu_seqlens_host,
                                        n_seqs, T, H, initial_state, final_state, out_gate, o,
                                        snap, workspace, workspace_bytes, stream);
    } else if (mfma)
        err = kda::launch_prefill_fused(q, k, v, gt, beta, cu_seqlens_dev, n_seqs, T, H,
                                        initial_state, final_state, out_gate, o, snap, stream);
    else
        err = kda::launch_prefill_vector(q, k, v, gt, beta, dtype, cu_seqlens_dev, n_seqs, T, H,
                                         d, chunk, initial_state, final_state, out_gate, o, snap,
                                         stream);
    return hip_status(err, "kda_prefill_chunked launch");
}

kda_status kda_prefill_chunked(const void* q, const void* k, const void* v, const void* g,
                               const float* beta, kda_dtype dtype, kda_gate gate,
                               const float* a_log, const int32_t* cu_seqlens_dev,
                               const int32_t* cu_seqlens_host, int n_seqs, int H, int dk, int dv,
                               int chunk, const float* initial_state, float* final_state,
                               const void* out_gate, void* o, float* snapshots, int snap_interval,
                               int snap_capacity, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
    return prefill_entry("kda_prefill_chunked", q, k, v, g, beta, dtype, gate, a_log,
                         cu_seqlens_dev, cu_seqlens_host, n_seqs, H, dk, dv, chunk, initial_state,
                         final_state, out_gate, o, snapshots, snap_interval, snap_capacity,
                         workspace, workspace_bytes, false, stream);
}

kda_status kda_prefill_chunked_noalloc(const void* q, const void* k, const void* v,
                                       const void* g, const float* beta, kda_dtype dtype,
                                       kda_gate gate, const float* a_log,
                                       const int32_t* cu_seqlens_dev,
                                       const int32_t* cu_seqlens_host, int n_seqs, int H, int dk,
                                       int dv, int chunk, const float* initial_state,
                                       float* final_state, const void* out_gate, void* o,
                                       float* snapshots, int snap_interval, int snap_capacity,
                                       hipStream_t stream) {
    const char* fn = "kda_prefill_chunked_noalloc";
    g_detail[0] = 0;
    // matrix-core shapes run on the static scratch: at least one tile per
    // sequence and head must fit in it
    const bool needs_scratch = n_seqs > 0 && H > 0 && mfma_shape(dtype, dk, dv, chunk);
    void* ws = nullptr;
    size_t ws_bytes = 0;
    if (needs_scratch) {
        const size_t least = kda::prefill_split_workspace_bytes_least(n_seqs, H);
        if (least > kda::static_scratch_bytes())
            return fail(KDA_ERR_WORKSPACE_TOO_SMALL,
                        "%s: %d sequences x %d heads need %zu bytes of scratch, the library's "
                        "static scratch holds %zu", fn, n_seqs, H, least,
                        kda::static_scratch_bytes());
        if (kda_status s = hip_status(kda::static_scratch(stream, &ws), "static scratch lookup"))
            return s;
        ws_bytes = kda::static_scratch_bytes();
    }
    return prefill_entry(fn, q, k, v, g, beta, dtype, gate, a_log, cu_seqlens_dev,
                         cu_seqlens_host, n_seqs, H, dk, dv, chunk, initial_state, final_state,
                         out_gate, o, snapshots, snap_interval, snap_capacity, ws, ws_bytes, true,
                         stream);
}

size_t kda_prefill_workspace_bytes_batch(const int32_t* cu_seqlens_host, int n_seqs, int H,
                                         int dk, int dv, int chunk, kda_dtype dtype) {
    if (n_seqs <= 0 || H <= 0 || !mfma_shape(dtype, dk, dv, chunk)) return 0;
    // a query: an invalid table gets the minimum, and no error detail is set
    bool valid = cu_seqlens_host && cu_seqlens_host[0] == 0;
    for (int n = 0; valid && n < n_seqs; ++n) valid = cu_seqlens_host[n + 1] >= cu_seqlens_host[n];
    if (!valid) return kda::prefill_split_workspace_bytes(n_seqs, H);
    return kda::prefill_split_workspace_bytes_batch(cu_seqlens_host, n_seqs, H);
}

size_t kda_prefill_workspace_bytes(int n_seqs, int H, int dk, int dv, int chunk,
                                   kda_dtype dtype) {
    if (n_seqs <= 0 || H <= 0 || !mfma_shape(dtype, dk, dv, chunk)) return 0;
    return kda::prefill_split_workspace_bytes(n_seqs, H);
}

// Shared by kda_decode_step (n_tok = 1, no snapshots) and kda_decode_tokens.
static kda_status decode_common(const char* fn, const void* q, const void* k, const void* v,
                                const void* g, const float* beta, kda_dtype dtype, kda_gate gate,
                                const float* a_log, void* state, kda_dtype state_dtype,
                                int64_t n_slots,
                                const int32_t* slot_idx, int B, int n_tok, int H, int dk, int dv,
                                const void* out_gate, void* o, void* token_states,
                                hipStream_t stream) {
    g_detail[0] = 0;
    if (dtype != KDA_F32 && dtype != KDA_BF16)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", fn, (int)dtype);
    if (state_dtype != KDA_F32 && state_dtype != KDA_BF16)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown state dtype %d", fn, (int)state_dtype);
    if (kda_status s = check_gate(fn, gate, a_log)) return s;
    if (kda_status s = check_heads(fn, H, dk, dv)) return s;
    if (B < 0 || n_slots < 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: B and n_slots must be >= 0", fn);
    if (n_tok < 1 || n_tok > 64)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: n_tok = %d, expected 1..64", fn, n_tok);
    if (B == 0) return KDA_OK;
    if (!slot_idx && n_slots < B)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: n_slots (%lld) < B (%d) without slot_idx", fn,
                    (long long)n_slots, B);
    // every decode shape spends at most 1024 work-items on one (sequence, head)
    if (!dispatch_fits((int64_t)B * H, 1024))
        return fail(KDA_ERR_UNSUPPORTED, "%s: B * H = %lld exceeds 4194303 (32-bit dispatch size)",
                    fn, (long long)B * H);
    if (!q || !k || !v || !g || !beta || !o || !state)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: q, k, v, g, beta, state and o are required",
                    fn);
    const size_t es = elem_size(dtype);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(o) ||
        !aligned16(state) || ((uintptr_t)beta & 3u) || ((uintptr_t)slot_idx & 3u) ||
        !aligned16(token_states) || !aligned16(out_gate))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: misaligned tensor pointer", fn);
    const size_t nv = (size_t)B * n_tok * H * dk, nb = (size_t)B * n_tok * H * 4;
    const size_t gb = gate_bytes(gate, (size_t)B * n_tok, H, dk, dtype);
    const size_t ab = a_log ? (size_t)H * 4 : 0;
    const size_t sbytes = (size_t)n_slots * kda_state_bytes(H, dk, dv, state_dtype);
    const size_t tbytes = (size_t)B * n_tok * kda_state_bytes(H, dk, dv, state_dtype);
    if (overlaps(o, nv * es, q, nv * es) || overlaps(o, nv * es, k, nv * es) ||
        overlaps(o, nv * es, v, nv * es) || overlaps(o, nv * es, g, gb) ||
        overlaps(o, nv * es, a_log, ab) ||
        overlaps(o, nv * es, state, sbytes) || overlaps(state, sbytes, q, nv * es) ||
        overlaps(state, sbytes, k, nv * es) || overlaps(state, sbytes, v, nv * es) ||
        overlaps(state, sbytes, g, gb) || overlaps(state, sbytes, beta, nb) ||
        overlaps(state, sbytes, a_log, ab) || overlaps(o, nv * es, out_gate, nv * es) ||
        overlaps(state, sbytes, out_gate, nv * es))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: state or o overlaps another argument", fn);
    if (token_states &&
        (overlaps(token_states, tbytes, state, sbytes) || overlaps(token_states, tbytes, o, nv * es) ||
         overlaps(token_states, tbytes, q, nv * es) || overlaps(token_states, tbytes, k, nv * es) ||
         overlaps(token_states, tbytes, v, nv * es) || overlaps(token_states, tbytes, g, gb) ||
         overlaps(token_states, tbytes, beta, nb) || overlaps(token_states, tbytes, a_log, ab) ||
         overlaps(token_states, tbytes, out_gate, nv * es)))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: token_states overlaps another argument", fn);
    return hip_status(kda::launch_decode(q, k, v, make_gate(g, a_log, gate), beta, dtype, state,
                                         state_dtype, n_slots, slot_idx, B, n_tok, H, dk,
                                         token_states, out_gate, o, stream),
                      "decode launch");
}

kda_status kda_decode_step(const void* q, const void* k, const void* v, const void* g,
                           const float* beta, kda_dtype dtype, kda_gate gate,
                           const float* a_log, void* state,
                           kda_dtype state_dtype, int64_t n_slots, const int32_t* slot_idx,
                           int B, int H, int dk, int dv, const void* out_gate, void* o,
                           hipStream_t stream) {
    return decode_common("kda_decode_step", q, k, v, g, beta, dtype, gate, a_log, state,
                         state_dtype, n_slots, slot_idx, B, 1, H, dk, dv, out_gate, o, nullptr,
                         stream);
}

kda_status kda_decode_tokens(const void* q, const void* k, const void* v, const void* g,
                             const float* beta, kda_dtype dtype, kda_gate gate,
                             const float* a_log, void* state,
                             kda_dtype state_dtype, int64_t n_slots, const int32_t* slot_idx,
                             int B, int n_tok, int H, int dk, int dv, const void* out_gate,
                             void* o, void* token_states, hipStream_t stream) {
    return decode_common("kda_decode_tokens", q, k, v, g, beta, dtype, gate, a_log, state,
                         state_dtype, n_slots, slot_idx, B, n_tok, H, dk, dv, out_gate, o,
                         token_states, stream);
}

static kda_status check_conv_common(const char* fn, const float* w, kda_dtype dtype,
                                    int channels, int l2_head_dim, float l2_eps) {
    if (dtype != KDA_F32 && dtype != KDA_BF16)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", fn, (int)dtype);
    if (channels <= 0 || channels % 2)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: channels must be positive and even", fn);
    if (!w || !aligned16(w))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: w must be non-NULL and 16-byte aligned", fn);
    if (l2_head_dim < 0 || (l2_head_dim > 0 && (channels % l2_head_dim || l2_head_dim % 2)))
        return fail(KDA_ERR_INVALID_ARGUMENT,
                    "%s: l2_head_dim must be 0 or an even divisor of channels", fn);
    if (l2_head_dim > 256)
        return fail(KDA_ERR_UNSUPPORTED, "%s: l2_head_dim > 256", fn);
    if (l2_head_dim == 0 && channels % 128 && channels > 256)
        return fail(KDA_ERR_UNSUPPORTED,
                    "%s: without normalisation, channels must be a multiple of 128 or <= 256",
                    fn);
    if (!(l2_eps >= 0.f))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: l2_eps must be >= 0", fn);
    return KDA_OK;
}

kda_status kda_short_conv_prefill(const void* x, const float* w, kda_dtype dtype,
                                  const int32_t* cu_seqlens_dev,
                                  const int32_t* cu_seqlens_host, int n_seqs, int channels,
                                  int l2_head_dim, float l2_eps, const void* conv_tail_in,
                                  void* conv_tail_out, void* y, hipStream_t stream) {
    const char* fn = "kda_short_conv_prefill";
    g_detail[0] = 0;
    if (kda_status s = check_conv_common(fn, w, dtype, channels, l2_head_dim, l2_eps)) return s;
    int64_t T = 0;
    if (kda_status s = check_cu(fn, cu_seqlens_host, n_seqs, &T)) return s;
    if (n_seqs == 0) return KDA_OK;
    if (!cu_seqlens_dev) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: cu_seqlens_dev is NULL", fn);
    // runs of at least 16 tokens per workgroup of 256 threads; the tail pass
    // takes one thread per (sequence, channel)
    if (!dispatch_fits((T + 15) / 16, 256) || !dispatch_fits((int64_t)n_seqs * channels + 255, 1))
        return fail(KDA_ERR_UNSUPPORTED,
                    "%s: T = %lld tokens of %d channels exceed the 32-bit dispatch size", fn,
                    (long long)T, channels);
    const size_t es = elem_size(dtype);
    const size_t nx = (size_t)T * channels * es, nt = (size_t)n_seqs * 3 * channels * es;
    if (T > 0) {
        if (!x || !y) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: x and y are required", fn);
        if (!aligned16(x) || !aligned16(y))
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: misaligned x or y", fn);
        if (overlaps(x, nx, y, nx) || overlaps(y, nx, conv_tail_in, nt) ||
            overlaps(y, nx, conv_tail_out, nt) || overlaps(x, nx, conv_tail_out, nt))
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s: y or conv_tail_out overlaps an input", fn);
    }
    if ((conv_tail_in && !aligned16(conv_tail_in)) || (conv_tail_out && !aligned16(conv_tail_out)))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: misaligned conv tail", fn);
    if (conv_tail_in && conv_tail_out && conv_tail_in != conv_tail_out &&
        overlaps(conv_tail_in, nt, conv_tail_out, nt))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: conv tails overlap without being equal", fn);
    return hip_status(kda::launch_short_conv_prefill(x, w, dtype, cu_seqlens_dev, n_seqs, T,
                                                     channels, l2_head_dim, l2_eps,
                                                     conv_tail_in, conv_tail_out, y, stream),
                      "kda_short_conv_prefill launch");
}

kda_status kda_short_conv_decode(const void* x, const float* w, kda_dtype dtype,
                                 void* conv_tail, int64_t n_slots, const int32_t* slot_idx,
                                 int B, int channels, int l2_head_dim, float l2_eps, void* y,
                                 hipStream_t stream) {
    const char* fn = "kda_short_conv_decode";
    g_detail[0] = 0;
    if (kda_status s = check_conv_common(fn, w, dtype, channels, l2_head_dim, l2_eps)) return s;
    if (B < 0 || n_slots < 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: B and n_slots must be >= 0", fn);
    if (B == 0) return KDA_OK;
    if (!slot_idx && n_slots < B)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: n_slots < B without slot_idx", fn);
    if (!dispatch_fits(B, 64))  // one 64-thread workgroup per sequence and head group
        return fail(KDA_ERR_UNSUPPORTED, "%s: B = %d exceeds 67108863 (32-bit dispatch size)",
                    fn, B);
    if (!x || !y || !conv_tail)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: x, y and conv_tail are required", fn);
    if (!aligned16(x) || !aligned16(y) || !aligned16(conv_tail) || ((uintptr_t)slot_idx & 3u))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: misaligned pointer", fn);
    const size_t es = elem_size(dtype);
    const size_t nx = (size_t)B * channels * es, nt = (size_t)n_slots * 3 * channels * es;
    if (overlaps(x, nx, y, nx) || overlaps(y, nx, conv_tail, nt) || overlaps(x, nx, conv_tail, nt))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: x, y and conv_tail must not overlap", fn);
    return hip_status(kda::launch_short_conv_decode(x, w, dtype, conv_tail, n_slots, slot_idx, B,
                                                    channels, l2_head_dim, l2_eps, y, stream),
                      "kda_short_conv_decode launch");
}

kda_status kda_device_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
    const char* fn = "kda_device_copy";
    g_detail[0] = 0;
    if (bytes == 0) return KDA_OK;
    if (!dst || !src) return fail(KDA_ERR_INVALID_ARGUMENT, "%s: dst and src are required", fn);
    if (!aligned16(dst) || !aligned16(src) || bytes % 16)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: pointers and size must be 16-byte aligned", fn);
    if (overlaps(dst, bytes, src, bytes))
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: dst and src overlap", fn);
    return hip_status(kda::launch_device_copy(dst, src, bytes, stream), "kda_device_copy launch");
}

}  // extern "C"
