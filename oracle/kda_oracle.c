/*
 * KDA oracle -- a plain, slow, sequential CPU reference for the Kimi Delta
 * Attention (KDA) gated delta-rule token mixer and its short-conv front end.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load or call this library.  The HIP
 * library never links it, and it shares no source, header, table or helper with
 * the HIP code.  Inputs reach it as plain arrays produced by the seeded input
 * generators; nothing it consumes comes from the GPU path.
 *
 * What it computes (page "Ling-3.1-flash: a 560B hybrid-attention MoE, counted
 * from its safetensors headers", section "How KDA and MLA split the work"):
 * each head keeps a d_k x d_v state S; per token the state is decayed channel
 * by channel with alpha_t = exp(g_t) (one factor per key channel), then the new
 * key-value association is written with a per-head scalar strength beta_t.  The
 * display equation of that section was lost from the page text; the update used
 * here is the gated delta rule that the prose describes,
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = S_t^T q_t,
 *
 * written out in its rank-1 form (identical up to rounding order):
 *
 *     S'  = Diag(alpha_t) S_{t-1}                    decay rows (key channels)
 *     u_t = beta_t (v_t - S'^T k_t)                   delta-rule write value
 *     S_t = S' + k_t u_t^T                            rank-1 write
 *     o_t = S_t^T q_t                                 read after the write
 *
 * The state is per head, fixed-size and carried token by token (page "Ling-3.1-
 * flash and the 7:1 hybrid: how much KV cache does a 560B model need at 1M
 * tokens?", section "Why would a model keep only 9 full-attention layers?"), and
 * 128 x 128 fp32 per head in the layer the pages describe (same page, section
 * "How big is the cache per token, exactly?").
 *
 * q, k and v pass through a width-4 causal depthwise convolution before the
 * recurrence (section "How KDA and MLA split the work" again); that convolution
 * and a per-head L2 normalisation are provided below as separate steps.
 *
 * Two precisions of the recurrence are built from one macro: *_f64 (double
 * state and arithmetic, the parity reference) and *_f32 (float state and
 * arithmetic, the plain sequential fp32 recurrence).  OpenMP spreads independent
 * (sequence, head) pairs over threads; tokens are always processed in order.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC kda_oracle.c -o libkda_oracle.so -lm
 * (The pin tests also compile patched copies of this file, each with one
 * planted mistake, to show that every such mistake fails a pin; the file itself
 * holds no switch for them.)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Return codes. */
#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_NO_MEM 2

static int check_cu(const int32_t* cu, int n_seqs) {
    if (!cu || n_seqs < 0) return 0;
    if (cu[0] != 0) return 0;
    for (int n = 0; n < n_seqs; ++n)
        if (cu[n + 1] < cu[n]) return 0;
    return 1;
}

/*
 * Recurrence over packed sequences.
 *   q, k, g : [T, H, dk]     v, o : [T, H, dv]     beta : [T, H]
 *   cu_seqlens : [n_seqs + 1], cu_seqlens[0] = 0, non-decreasing, T = cu[n_seqs]
 *   S0      : [n_seqs, H, dk, dv] or NULL (zero initial state)
 *   S_final : [n_seqs, H, dk, dv] or NULL (not written)
 * Each sequence starts from its own initial state; nothing crosses a sequence
 * boundary.  n_threads <= 0 uses the OpenMP default.
 */
#define DEFINE_RECURRENCE(SUFFIX, REAL, EXPF)                                              \
int kda_oracle_recurrence_##SUFFIX(const REAL* q, const REAL* k, const REAL* v,            \
                                   const REAL* g, const REAL* beta,                        \
                                   const int32_t* cu_seqlens, int n_seqs, int H,           \
                                   int dk, int dv, const REAL* S0, REAL* o,                \
                                   REAL* S_final, int n_threads) {                         \
    if (!q || !k || !v || !g || !beta || !o || H <= 0 || dk <= 0 || dv <= 0)               \
        return ORACLE_BAD_ARG;                                                             \
    if (!check_cu(cu_seqlens, n_seqs)) return ORACLE_BAD_ARG;                              \
    const int64_t n_pairs = (int64_t)n_seqs * H;                                           \
    int status = ORACLE_OK;                                                                \
    int nt = n_threads > 0 ? n_threads : 0;                                                \
    _Pragma("omp parallel num_threads(nt > 0 ? nt : omp_get_max_threads())")              \
    {                                                                                      \
        REAL* S = (REAL*)malloc(sizeof(REAL) * (size_t)dk * dv);                           \
        REAL* alpha = (REAL*)malloc(sizeof(REAL) * (size_t)dk);                            \
        REAL* y = (REAL*)malloc(sizeof(REAL) * (size_t)dv);                                \
        REAL* u = (REAL*)malloc(sizeof(REAL) * (size_t)dv);                                \
        if (!S || !alpha || !y || !u) {                                                    \
            _Pragma("omp atomic write") status = ORACLE_NO_MEM;                            \
        } else {                                                                           \
            _Pragma("omp for schedule(dynamic, 1)")                                        \
            for (int64_t pair = 0; pair < n_pairs; ++pair) {                               \
                const int n = (int)(pair / H), h = (int)(pair % H);                        \
                const size_t sidx = ((size_t)n * H + h) * (size_t)dk * dv;                 \
                if (S0) memcpy(S, S0 + sidx, sizeof(REAL) * (size_t)dk * dv);              \
                else memset(S, 0, sizeof(REAL) * (size_t)dk * dv);                         \
                for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {              \
                    const REAL* qt = q + ((size_t)t * H + h) * dk;                         \
                    const REAL* kt = k + ((size_t)t * H + h) * dk;                         \
                    const REAL* gt = g + ((size_t)t * H + h) * dk;                         \
                    const REAL* vt = v + ((size_t)t * H + h) * dv;                         \
                    const REAL bt = beta[(size_t)t * H + h];                               \
                    REAL* ot = o + ((size_t)t * H + h) * dv;                               \
                    /* alpha_t = exp(g_t), one factor per key channel */                   \
                    for (int i = 0; i < dk; ++i) alpha[i] = (REAL)EXPF(gt[i]);             \
                    /* S' = Diag(alpha_t) S_{t-1}: row i (key channel i) scaled */         \
                    for (int i = 0; i < dk; ++i)                                           \
                        for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= alpha[i];    \
                    /* y = S'^T k_t */                                                     \
                    for (int j = 0; j < dv; ++j) y[j] = 0;                                 \
                    for (int i = 0; i < dk; ++i)                                           \
                        for (int j = 0; j < dv; ++j) y[j] += S[(size_t)i * dv + j] * kt[i];\
                    /* u_t = beta_t (v_t - y) */                                           \
                    for (int j = 0; j < dv; ++j) u[j] = bt * (vt[j] - y[j]);               \
                    /* S_t = S' + k_t u_t^T */                                             \
                    for (int i = 0; i < dk; ++i)                                           \
                        for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += kt[i] * u[j];\
                    /* o_t = S_t^T q_t */                                                  \
                    for (int j = 0; j < dv; ++j) ot[j] = 0;                                \
                    for (int i = 0; i < dk; ++i)                                           \
                        for (int j = 0; j < dv; ++j) ot[j] += S[(size_t)i * dv + j] * qt[i];\
                }                                                                          \
                if (S_final) memcpy(S_final + sidx, S, sizeof(REAL) * (size_t)dk * dv);    \
            }                                                                              \
        }                                                                                  \
        free(S); free(alpha); free(y); free(u);                                            \
    }                                                                                      \
    return status;                                                                         \
}

DEFINE_RECURRENCE(f64, double, exp)
DEFINE_RECURRENCE(f32, float, expf)

/*
 * Causal depthwise convolution of width 4 over packed sequences (the short
 * convolution that q, k and v pass through before the recurrence):
 *
 *     y_t[c] = sum_{j=0..3} w[c][j] * x_{t-3+j}[c]
 *
 * so w[c][3] multiplies the current token.  x_{t'} for t' before the sequence
 * start comes from tail_in[n] (tail_in[n][0] = x_{-3}, [1] = x_{-2},
 * [2] = x_{-1}), or is zero when tail_in is NULL.  No bias, no activation.
 *   x, y     : [T, Cch]
 *   w        : [Cch, 4]
 *   tail_in  : [n_seqs, 3, Cch] or NULL
 *   tail_out : [n_seqs, 3, Cch] or NULL; receives the last three inputs of each
 *              sequence, history included when a sequence is shorter than 3.
 */
int kda_oracle_short_conv_f64(const double* x, const double* w, const int32_t* cu_seqlens,
                              int n_seqs, int Cch, const double* tail_in, double* y,
                              double* tail_out) {
    if (!x || !w || !y || Cch <= 0) return ORACLE_BAD_ARG;
    if (!check_cu(cu_seqlens, n_seqs)) return ORACLE_BAD_ARG;
    int status = ORACLE_OK;
#pragma omp parallel for schedule(static)
    for (int c = 0; c < Cch; ++c) {
        for (int n = 0; n < n_seqs; ++n) {
            const int64_t t0 = cu_seqlens[n], t1 = cu_seqlens[n + 1];
            const int64_t len = t1 - t0;
            /* hist[m] = x_{m-3} relative to the sequence start, m = 0..len+2 */
            double* hist = (double*)malloc(sizeof(double) * (size_t)(len + 3));
            if (!hist) {
#pragma omp atomic write
                status = ORACLE_NO_MEM;
                continue;
            }
            for (int m = 0; m < 3; ++m)
                hist[m] = tail_in ? tail_in[((size_t)n * 3 + m) * Cch + c] : 0.0;
            for (int64_t t = 0; t < len; ++t) hist[t + 3] = x[(size_t)(t0 + t) * Cch + c];
            for (int64_t t = 0; t < len; ++t) {
                double acc = 0.0;
                for (int j = 0; j < 4; ++j) acc += w[(size_t)c * 4 + j] * hist[t + j];
                y[(size_t)(t0 + t) * Cch + c] = acc;
            }
            if (tail_out)
                for (int m = 0; m < 3; ++m)
                    tail_out[((size_t)n * 3 + m) * Cch + c] = hist[len + m];
            free(hist);
        }
    }
    return status;
}

/*
 * Per-head L2 normalisation in place: each run of head_dim channels in each row
 * of x [rows, width] becomes x / sqrt(sum x^2 + eps).
 */
int kda_oracle_l2norm_heads_f64(double* x, int64_t rows, int width, int head_dim, double eps) {
    if (!x || rows < 0 || width <= 0 || head_dim <= 0 || width % head_dim) return ORACLE_BAD_ARG;
    const int heads = width / head_dim;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int h = 0; h < heads; ++h) {
            double* p = x + (size_t)r * width + (size_t)h * head_dim;
            double ss = 0.0;
            for (int i = 0; i < head_dim; ++i) ss += p[i] * p[i];
            const double inv = 1.0 / sqrt(ss + eps);
            for (int i = 0; i < head_dim; ++i) p[i] *= inv;
        }
    }
    return ORACLE_OK;
}
