/*
 * kda.h -- C ABI of libkda.so, the MI355X (gfx950) implementation of the Kimi
 * Delta Attention (KDA) gated delta-rule token mixer.
 *
 * The operation (page "Ling-3.1-flash: a 560B hybrid-attention MoE, counted
 * from its safetensors headers", section "How KDA and MLA split the work"):
 * every head keeps a d_k x d_v state S, decayed per key channel by
 * alpha_t = exp(g_t) and written with a per-head scalar strength beta_t,
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = S_t^T q_t,
 *
 * with q, k, v first passed through a width-4 causal depthwise convolution.
 * The state is fixed-size per sequence and 128 x 128 fp32 per head in the layer
 * those pages describe (page "Ling-3.1-flash and the 7:1 hybrid: how much KV
 * cache does a 560B model need at 1M tokens?", section "How big is the cache
 * per token, exactly?").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor arguments are device pointers to contiguous row-major memory,
 *   16-byte aligned, owned by the caller.  The library never allocates device
 *   memory and keeps no per-call state: scratch memory, where a path uses
 *   some, is a workspace argument that the caller provides.
 * - Layouts: q, k, g  [tokens, H, d_k];  v, o  [tokens, H, d_v];
 *   beta [tokens, H];  state [slots, H, d_k, d_v] (d_v contiguous: row i of a
 *   head's state belongs to key channel i).
 * - q, k, v and o share one dtype (KDA_F32 or KDA_BF16).  g (the log of the
 *   decay, alpha = exp(g)) and beta are always fp32; the state is fp32, except
 *   that decode and state init also take states stored in bf16 (their
 *   state_dtype argument; arithmetic stays fp32).  g is per key
 *   channel ([..., H, d_k], KDA_GATE_CHANNEL) or per head ([..., H],
 *   KDA_GATE_HEAD, alpha broadcast over the channels).  No query scale is
 *   applied: a caller that wants one scales q.
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the
 *   call returns at once.  Arguments are checked on the host before anything is
 *   enqueued: a failed check returns a non-zero status and enqueues nothing.
 *   Device-side errors surface at the caller's next synchronisation, as for any
 *   HIP kernel.
 * - Thread safety: calls may come from several host threads; the only shared
 *   state is a thread-local error text.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enumerations are int-sized in C.  Compiled as C++ they get int as their
 * fixed underlying type, so that any int a caller passes (an out-of-range code
 * included, which the entry points reject) is a valid value of the parameter's
 * type rather than undefined behaviour. */
#ifdef __cplusplus
#define KDA_ENUM_BASE : int
#else
#define KDA_ENUM_BASE
#endif

typedef enum kda_status KDA_ENUM_BASE {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad size, bad cu_seqlens */
    KDA_ERR_UNSUPPORTED = 2,      /* valid but not implemented (e.g. d_k != d_v), or
                                     a launch beyond the 32-bit dispatch size (2^32
                                     work-items): decode with B * H > 4194303, prefill
                                     with n_seqs * H * (4 for d = 128, d / 32 from 32,
                                     else 1) > 4194303, a convolution over T >= 2^28
                                     tokens or of B > 67108863 sequences */
    KDA_ERR_HIP = 3,              /* a HIP runtime call failed; see kda_last_error_detail */
    KDA_ERR_WORKSPACE_TOO_SMALL = 4 /* a workspace below the size its query returns */
} kda_status;

typedef enum kda_dtype KDA_ENUM_BASE {
    KDA_F32 = 0,
    KDA_BF16 = 1
} kda_dtype;

/* Layout of the log decay g.  KDA decays every key channel separately; its
 * special case with one decay per head and token is Gated DeltaNet, which
 * page "Ling-3.1-flash and the 7:1 hybrid: how much KV cache does a 560B model
 * need at 1M tokens?" (section "Why would a model keep only 9 full-attention
 * layers?") names as the layer KDA extends with finer-grained gating. */
typedef enum kda_gate KDA_ENUM_BASE {
    KDA_GATE_CHANNEL = 0, /* g [tokens, H, d_k] fp32: alpha_t per key channel (KDA) */
    KDA_GATE_HEAD = 1,    /* g [tokens, H] fp32: one alpha_t per head, all channels */
    KDA_GATE_PROJ = 2     /* gate prologue fused in: see below */
} kda_gate;

/* KDA_GATE_PROJ takes the decay and write strength before their activations,
 * as the layer's projections produce them.  Page "Ling-3.1-flash: a 560B
 * hybrid-attention MoE, counted from its safetensors headers" (section "How KDA
 * and MLA split the work") names the tensors behind them, f_proj and A_log for
 * the per-channel decay and b_proj for the per-head write strength, but not the
 * formula; the library applies
 *     g_t    = -exp(a_log[h]) * softplus(f_t)     (log alpha_t, per key channel)
 *     beta_t = sigmoid(b_t)
 * with softplus(x) = log(1 + exp(x)).  Then:
 *   g     : f, [tokens, H, d_k] in the q/k/v dtype (half the bytes of an fp32
 *           g for bf16 inputs);
 *   a_log : [H] fp32, one log rate per head (a positive rate exp(a_log));
 *   beta  : the logits b, [tokens, H] fp32.
 * With the other gate layouts a_log must be NULL. */

/* Text for a status code (static storage). */
const char* kda_status_string(kda_status s);

/* Human-readable detail of the last failure on the calling thread ("" if none).
 * Valid until the next call into the library from that thread. */
const char* kda_last_error_detail(void);

/* Bytes of one sequence's state for one layer: H * d_k * d_v elements of
 * state_dtype (4 bytes for KDA_F32, 2 for KDA_BF16).  4 194 304 for H = 64,
 * d_k = d_v = 128 in fp32; 0 for non-positive sizes or an unknown dtype. */
size_t kda_state_bytes(int H, int dk, int dv, kda_dtype state_dtype);

/*
 * kda_state_init -- set n_slots sequence states to zero (src == NULL) or to a
 * copy of src, converted to state_dtype.  This is the state the recurrence
 * starts from (S_0); it also converts a prefill's fp32 final states into the
 * bf16 states of the bf16-state decode, and back.
 *   state     : [n_slots, H, dk, dv] state_dtype, written.
 *   src       : [n_slots, H, dk, dv] src_dtype or NULL; must not overlap state.
 * fp32 -> bf16 rounds to nearest even; bf16 -> fp32 is exact.  Uses a
 * fill/copy kernel (no memset node), so it may be captured in a graph.
 */
kda_status kda_state_init(void* state, kda_dtype state_dtype, int64_t n_slots, int H, int dk,
                          int dv, const void* src, kda_dtype src_dtype, hipStream_t stream);

/*
 * kda_prefill_chunked -- run the recurrence over n_seqs packed sequences,
 * chunk tokens at a time (the chunked/WY form, exact up to rounding).
 *
 *   q, k            : [T, H, dk] dtype       v, o : [T, H, dv] dtype
 *   g               : [T, H, dk] fp32 (log decay; alpha = exp(g)), [T, H] fp32
 *                     with gate = KDA_GATE_HEAD, or the decay projection
 *                     [T, H, dk] in dtype with gate = KDA_GATE_PROJ.  Range:
 *                     any finite g <= 0 (alpha in (0, 1]), however strong the
 *                     decay over a chunk: the kernels reference the scaled
 *                     operands to a clamped per-channel point and switch a
 *                     chunk that decays below 2^-160 (about -111 in natural
 *                     log; -80 in the fp32 vector kernel) on any channel to
 *                     pairwise decay factors, so no factor overflows.  Tested
 *                     down to about -540 per chunk.  g > 0 (alpha > 1) lies
 *                     outside the method and may overflow.
 *   a_log           : [H] fp32 with KDA_GATE_PROJ, else NULL
 *   beta            : [T, H] fp32 (logits with KDA_GATE_PROJ)
 *   cu_seqlens_dev  : [n_seqs + 1] int32 on the device
 *   cu_seqlens_host : the same values in host memory (validated: cu[0] = 0,
 *                     non-decreasing; T = cu[n_seqs]).  The kernels clamp
 *                     every index to [0, T), so a device copy that disagrees
 *                     with the host copy gives wrong results, never an access
 *                     outside the buffers.
 *   chunk           : 16, 32 or 64 tokens; the result does not depend on it
 *                     beyond rounding.
 *   initial_state   : [n_seqs, H, dk, dv] fp32, or NULL for zeros.
 *   final_state     : [n_seqs, H, dk, dv] fp32, or NULL (not written).  May be
 *                     the same pointer as initial_state (in-place update).
 *   out_gate        : [T, H, dv] dtype, or NULL.  The output gate: when given,
 *                     every output is o_t * sigmoid(out_gate_t), elementwise
 *                     per (token, head, value channel), rounded to dtype once.
 *                     Page "Ling-3.1-flash: a 560B hybrid-attention MoE,
 *                     counted from its safetensors headers" (section "How KDA
 *                     and MLA split the work") lists a full-rank gate
 *                     projection (4096 -> 8192, one value per head and value
 *                     channel) before the output projection, without naming
 *                     its activation; the sigmoid is the one the same section
 *                     gives the gated MLA's output gate.  No normalisation
 *                     comes before it (the pages name none).  Must not overlap
 *                     o or final_state.
 *   o               : [T, H, dv] dtype, written; must not overlap any input.
 *   snapshots       : [n_seqs, snap_capacity, H, dk, dv] fp32, or NULL.  Entry
 *                     [n, j] receives sequence n's state after its first
 *                     (j + 1) * snap_interval tokens, for every j below
 *                     snap_capacity with (j + 1) * snap_interval <= its
 *                     length; other entries are left untouched.  These are the
 *                     chunk-aligned states a prefix cache keeps for recurrent
 *                     layers (page "Ling-3.1-flash and the 7:1 hybrid: how much
 *                     KV cache does a 560B model need at 1M tokens?", section
 *                     "How should I decide whether a hybrid fits my workload?":
 *                     the serving engine manages the linear state like
 *                     recurrent-model state, block-aligned, and prefix caching
 *                     behaves differently for it).  Must not overlap any other
 *                     argument.
 *   snap_interval   : tokens between snapshots, a positive multiple of chunk
 *                     (ignored when snapshots is NULL).
 *   snap_capacity   : snapshots per sequence that the buffer holds (>= 0).
 *   workspace       : device scratch of workspace_bytes >=
 *                     kda_prefill_workspace_bytes(...) bytes (more gives longer
 *                     windows; see kda_prefill_workspace_bytes_batch), 16-byte aligned,
 *                     owned by the caller, not overlapping any other argument;
 *                     or NULL.  Its contents on entry do not matter and on
 *                     return are unspecified.  Calls that share one workspace
 *                     must be ordered (same stream, or synchronised).
 * Supported: dk == dv in {16, 32, 64, 128}.  bf16 inputs with dk = dv = 128 and
 * chunk = 64 run on the matrix cores (bf16 operands, fp32 accumulation, fp32
 * state): with a workspace, a chunk-parallel kernel first forms every chunk's
 * state-independent operands (decay-scaled keys and queries, the inverse
 * (I + N)^{-1}, the causal query-key products) and a second kernel runs the
 * sequential state pass over them; with workspace == NULL one fused kernel does
 * both (slower: its per-chunk work is repeated for every quarter of the value
 * dimension).  Every other case runs the fp32 vector kernel and ignores the
 * workspace.  T = 0 or n_seqs = 0 is valid: final states of empty sequences
 * equal their initial states.
 * Errors: KDA_ERR_WORKSPACE_TOO_SMALL for a non-NULL workspace smaller than
 * kda_prefill_workspace_bytes; KDA_ERR_INVALID_ARGUMENT for a misaligned one
 * or one that overlaps another argument.
 */
kda_status kda_prefill_chunked(const void* q, const void* k, const void* v,
                               const void* g, const float* beta, kda_dtype dtype, kda_gate gate,
                               const float* a_log,
                               const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host,
                               int n_seqs, int H, int dk, int dv, int chunk,
                               const float* initial_state, float* final_state,
                               const void* out_gate, void* o,
                               float* snapshots, int snap_interval, int snap_capacity,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kda_prefill_chunked_noalloc -- kda_prefill_chunked for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Arguments, results and errors are those of
 * kda_prefill_chunked, without the workspace: the matrix-core shapes (bf16,
 * dk = dv = 128, chunk 64) run the two-kernel path on a static scratch array
 * of 128 MiB that the library keeps in every GPU's memory it runs on until the
 * process ends; the other shapes need no scratch.  The call allocates no
 * device memory (no hipMalloc, hipFree or memset), so it may be captured in a
 * graph.  The two-kernel path runs on any workspace that holds the state
 * carry and one operand tile per sequence and head (123 648 bytes per sequence
 * and head, plus 256 per 64 sequences), in windows as long as the rest of the
 * scratch allows (up to 32 chunks: at H = 64, the full length for one
 * sequence, one chunk for 16); a batch that needs more than the scratch returns
 * KDA_ERR_WORKSPACE_TOO_SMALL: at H = 64, more than 16 sequences per call.  The first call on a device looks the array's address up
 * (KDA_ERR_HIP if that fails).  All calls on one GPU share its array, which
 * keeps the last call's contents: calls that overlap on one GPU (unordered
 * streams) race on it and must be serialised by the caller.
 */
kda_status kda_prefill_chunked_noalloc(const void* q, const void* k, const void* v,
                                       const void* g, const float* beta, kda_dtype dtype,
                                       kda_gate gate, const float* a_log,
                                       const int32_t* cu_seqlens_dev,
                                       const int32_t* cu_seqlens_host, int n_seqs, int H, int dk,
                                       int dv, int chunk, const float* initial_state,
                                       float* final_state, const void* out_gate, void* o,
                                       float* snapshots, int snap_interval, int snap_capacity,
                                       hipStream_t stream);

/*
 * kda_prefill_workspace_bytes -- size of the workspace that lets
 * kda_prefill_chunked use its two-kernel matrix-core path for this shape; 0 when
 * the shape runs a path that needs none.  Depends only on n_seqs and H for the
 * matrix-core shapes: a state carry (64 KiB per sequence and head), a table of
 * the sequences ranked by length (4 bytes per sequence, rounded up to 256),
 * and the per-chunk operand tiles (58 112 bytes per chunk and head) of one
 * window: 192 MiB, or 32 chunks of every sequence if that is less, and at least
 * one chunk of every sequence.  The sequences still running at a window's
 * start share its tiles, so windows grow as shorter sequences end (up to 32
 * chunks).
 */
size_t kda_prefill_workspace_bytes(int n_seqs, int H, int dk, int dv, int chunk,
                                   kda_dtype dtype);

/*
 * kda_prefill_workspace_bytes_batch -- the workspace that runs this batch
 * (cu_seqlens_host: [n_seqs + 1] int32 in host memory, as for
 * kda_prefill_chunked) in its longest windows: min(32, longest sequence's
 * chunks) chunks of every sequence, as long as those tiles stay within 4 GiB;
 * never less than kda_prefill_workspace_bytes.  kda_prefill_chunked gives the
 * tiles whatever a workspace holds beyond the state carry and rank table, so a
 * larger workspace means longer windows: at H = 64, batches of 16-128
 * sequences ran 1.4-2x faster than with the minimum.  Returns
 * kda_prefill_workspace_bytes for an invalid cu_seqlens_host and 0 where that
 * does.
 */
size_t kda_prefill_workspace_bytes_batch(const int32_t* cu_seqlens_host, int n_seqs, int H,
                                         int dk, int dv, int chunk, kda_dtype dtype);

/*
 * kda_decode_step -- advance B sequences by one token each, in place.
 *
 *   q, k     : [B, H, dk] dtype        v, o : [B, H, dv] dtype
 *   g        : [B, H, dk] fp32 ([B, H] fp32 with KDA_GATE_HEAD; the decay
 *              projection [B, H, dk] in dtype with KDA_GATE_PROJ)
 *   a_log    : [H] fp32 with KDA_GATE_PROJ, else NULL
 *   beta     : [B, H] fp32 (logits with KDA_GATE_PROJ)
 *   state    : [n_slots, H, dk, dv] state_dtype, read and written in place.
 *   state_dtype : KDA_F32, or KDA_BF16 for half the state bytes: the state is
 *              widened to fp32 when read, stepped in fp32, and rounded to the
 *              nearest bf16 (ties to even) once per call when written.  Page
 *              "Ling-3.1-flash and the 7:1 hybrid: how much KV cache does a
 *              560B model need at 1M tokens?" (section "How fast did the
 *              community react?") warns that linear-attention state is
 *              sensitive to precision; the rounding error accumulates over
 *              steps.
 *   slot_idx : [B] int32 on the device giving each sequence's state slot, or
 *              NULL for slot b = b (then n_slots >= B).  Slots must be
 *              distinct.  A slot outside [0, n_slots) is not touched and that
 *              sequence's output is set to NaN.
 *   out_gate : [B, H, dv] dtype or NULL: the output gate, o * sigmoid(out_gate),
 *              as in kda_prefill_chunked.
 * Supported: dk == dv in {16, 32, 64, 128}.  Each state is read once and
 * written once (fused form of one recurrence step).
 */
kda_status kda_decode_step(const void* q, const void* k, const void* v, const void* g,
                           const float* beta, kda_dtype dtype, kda_gate gate,
                           const float* a_log, void* state,
                           kda_dtype state_dtype, int64_t n_slots, const int32_t* slot_idx,
                           int B, int H, int dk, int dv, const void* out_gate, void* o,
                           hipStream_t stream);

/*
 * kda_decode_tokens -- advance B sequences by n_tok consecutive tokens each, in
 * place: the recurrence above applied to tokens 0, 1, ..., n_tok - 1 of every
 * sequence in order, with each state read once and written once.  This is the
 * verification step of speculative decoding: the serving recipe on page
 * "Ling-3.1-flash and the 7:1 hybrid: how much KV cache does a 560B model need
 * at 1M tokens?" (section "What does that mean for serving?") drafts three
 * tokens per step with the model's multi-token-prediction layer, and page
 * "Ling-3.1-flash: a 560B hybrid-attention MoE, counted from its safetensors
 * headers" (section "The serving numbers are not one experiment") reports an
 * average of about 2-2.6 accepted tokens per step.  The verifier advances every
 * sequence by the drafted tokens at once.
 *
 *   q, k         : [B, n_tok, H, dk] dtype    v, o : [B, n_tok, H, dv] dtype
 *   g            : [B, n_tok, H, dk] fp32 ([B, n_tok, H] fp32 with
 *                  KDA_GATE_HEAD; the decay projection [B, n_tok, H, dk] in
 *                  dtype with KDA_GATE_PROJ)
 *   a_log        : [H] fp32 with KDA_GATE_PROJ, else NULL
 *   beta         : [B, n_tok, H] fp32 (logits with KDA_GATE_PROJ)
 *   state        : [n_slots, H, dk, dv] state_dtype, read and written in
 *                  place; on return it holds the state after the last token.
 *   state_dtype  : as in kda_decode_step (a bf16 state is rounded once, after
 *                  the last token).
 *   slot_idx     : as in kda_decode_step.
 *   out_gate     : [B, n_tok, H, dv] dtype or NULL: the output gate, as in
 *                  kda_prefill_chunked.
 *   token_states : [B, n_tok, H, dk, dv] state_dtype, or NULL.  When given, entry
 *                  [b, j] receives sequence b's state after token j, so that
 *                  a caller that accepts only the first m drafts can restore
 *                  the state after token m - 1 (kda_state_init copies it).
 *                  Must not overlap any other argument.
 * n_tok in 1..64; n_tok = 1 without token_states is exactly kda_decode_step.
 * Out-of-range slots leave every state untouched and set all n_tok outputs of
 * that sequence to NaN.
 */
kda_status kda_decode_tokens(const void* q, const void* k, const void* v, const void* g,
                             const float* beta, kda_dtype dtype, kda_gate gate,
                             const float* a_log, void* state,
                             kda_dtype state_dtype, int64_t n_slots, const int32_t* slot_idx,
                             int B, int n_tok, int H, int dk, int dv, const void* out_gate,
                             void* o, void* token_states, hipStream_t stream);

/*
 * kda_short_conv_prefill -- width-4 causal depthwise convolution over packed
 * sequences, optionally followed by a per-head L2 normalisation (the front end
 * that q, k and v pass through before the recurrence):
 *
 *     y_t[c] = sum_{j=0..3} w[c][j] * x_{t-3+j}[c]      (w[c][3]: current token)
 *     y_t[head] <- y_t[head] / sqrt(sum y_t[head]^2 + l2_eps)   if l2_head_dim > 0
 *
 *   x, y            : [T, channels] dtype (one stream, e.g. the 8192 q channels)
 *   w               : [channels, 4] fp32
 *   cu_seqlens_dev/host : as in kda_prefill_chunked
 *   conv_tail_in    : [n_seqs, 3, channels] dtype: inputs x_{-3}, x_{-2}, x_{-1}
 *                     before each sequence, or NULL for zero history.
 *   conv_tail_out   : [n_seqs, 3, channels] dtype, or NULL: receives the last
 *                     three inputs of each sequence (history included for
 *                     sequences shorter than three).  May equal conv_tail_in.
 *   l2_head_dim     : 0 (no normalisation) or a divisor of channels, at most
 *                     256 and a multiple of 2.
 * Math is fp32; y is rounded to dtype.  y must not overlap x.
 */
kda_status kda_short_conv_prefill(const void* x, const float* w, kda_dtype dtype,
                                  const int32_t* cu_seqlens_dev,
                                  const int32_t* cu_seqlens_host, int n_seqs, int channels,
                                  int l2_head_dim, float l2_eps, const void* conv_tail_in,
                                  void* conv_tail_out, void* y, hipStream_t stream);

/*
 * kda_short_conv_decode -- the same convolution for one token per sequence,
 * shifting each sequence's tail in place.
 *   x, y      : [B, channels] dtype
 *   conv_tail : [n_slots, 3, channels] dtype, read and written in place.
 *   slot_idx  : [B] int32 device array or NULL (slot b = b; then n_slots >= B).
 *               Out-of-range slots are skipped and their y set to NaN.
 */
kda_status kda_short_conv_decode(const void* x, const float* w, kda_dtype dtype,
                                 void* conv_tail, int64_t n_slots, const int32_t* slot_idx,
                                 int B, int channels, int l2_head_dim, float l2_eps, void* y,
                                 hipStream_t stream);

/*
 * kda_device_copy -- the streaming-bandwidth reference for the kernels above
 * (not part of the recurrence): copies `bytes` from src to dst on the device
 * with 16-byte non-temporal loads and stores, four independent pieces per lane
 * in flight.  Its achieved rate is the practical ceiling that the HBM-bound
 * kernels are compared with, and its byte counters calibrate profiler traffic
 * readings.
 *   dst, src : device buffers, 16-byte aligned, not overlapping.
 *   bytes    : a multiple of 16; 0 does nothing.
 * Errors: KDA_ERR_INVALID_ARGUMENT for a NULL pointer with bytes > 0, a
 * misaligned pointer or size, or overlapping buffers; KDA_ERR_HIP if the
 * launch fails.
 */
kda_status kda_device_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
