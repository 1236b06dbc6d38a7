/*
 * Host sanitizer run of the CPU oracle (test infrastructure).  Built by
 * tests/test_oracle_sanitize.py with AddressSanitizer and
 * UndefinedBehaviorSanitizer, with the oracle's source compiled into the same
 * binary.  Every oracle entry point is driven over ragged packed sequences
 * (empty ones and ones shorter than the convolution's history included),
 * d_k != d_v, both precisions, with and without initial states and tails, and
 * over its argument-error paths.  A few properties that the definition fixes
 * are checked on the way, so that a run that only avoids crashing still fails:
 * beta = 0 and g = 0 leave the state unchanged bit for bit, the fp32 build
 * stays near the fp64 one, the conv tail of a short sequence carries the older
 * history forward, and L2-normalised heads have unit norm.
 * Prints "OK" and exits 0 when everything holds.
 */
#include "../oracle/kda_oracle.c"

#include <stdio.h>

static uint64_t lcg_state = 12345u;
static double uniform(void) {  /* in [-1, 1) */
    lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(lcg_state >> 11) / 4503599627370496.0 - 1.0;
}

#define CHECK(cond, msg)                                        \
    do {                                                        \
        if (!(cond)) {                                          \
            fprintf(stderr, "FAIL: %s (line %d)\n", msg, __LINE__); \
            return 1;                                           \
        }                                                       \
    } while (0)

static int recurrence_cases(void) {
    enum { NS = 4, H = 3, DK = 16, DV = 8 };
    const int32_t cu[NS + 1] = {0, 5, 5, 22, 23};
    const int T = cu[NS];
    const size_t nk = (size_t)T * H * DK, nv = (size_t)T * H * DV, nb = (size_t)T * H;
    const size_t ns = (size_t)NS * H * DK * DV;
    double *q = malloc(nk * 8), *k = malloc(nk * 8), *g = malloc(nk * 8), *v = malloc(nv * 8);
    double *beta = malloc(nb * 8), *o = malloc(nv * 8), *S0 = malloc(ns * 8), *S = malloc(ns * 8);
    float *qf = malloc(nk * 4), *kf = malloc(nk * 4), *gf = malloc(nk * 4), *vf = malloc(nv * 4);
    float *bf = malloc(nb * 4), *of = malloc(nv * 4), *S0f = malloc(ns * 4), *Sf = malloc(ns * 4);
    for (size_t i = 0; i < nk; ++i) {
        q[i] = uniform() * 0.25; k[i] = uniform() * 0.25; g[i] = -0.2 * (uniform() + 1.0);
        qf[i] = (float)q[i]; kf[i] = (float)k[i]; gf[i] = (float)g[i];
    }
    for (size_t i = 0; i < nv; ++i) { v[i] = uniform(); vf[i] = (float)v[i]; }
    for (size_t i = 0; i < nb; ++i) { beta[i] = 0.5 * (uniform() + 1.0); bf[i] = (float)beta[i]; }
    for (size_t i = 0; i < ns; ++i) { S0[i] = 0.1 * uniform(); S0f[i] = (float)S0[i]; }

    CHECK(kda_oracle_recurrence_f64(q, k, v, g, beta, cu, NS, H, DK, DV, S0, o, S, 2) == ORACLE_OK,
          "f64 recurrence");
    CHECK(kda_oracle_recurrence_f32(qf, kf, vf, gf, bf, cu, NS, H, DK, DV, S0f, of, Sf, 2) ==
              ORACLE_OK, "f32 recurrence");
    double num = 0, den = 0;
    for (size_t i = 0; i < ns; ++i) { num += (Sf[i] - S[i]) * (Sf[i] - S[i]); den += S[i] * S[i]; }
    CHECK(den > 0 && sqrt(num / den) < 1e-5, "fp32 state near fp64");
    /* the empty sequence 1 keeps its initial state */
    for (size_t i = (size_t)1 * H * DK * DV; i < (size_t)2 * H * DK * DV; ++i)
        CHECK(S[i] == S0[i], "empty sequence keeps its state");
    /* no initial state, no final state */
    CHECK(kda_oracle_recurrence_f64(q, k, v, g, beta, cu, NS, H, DK, DV, NULL, o, NULL, 1) ==
              ORACLE_OK, "f64 recurrence without states");

    /* beta = 0, g = 0: the state is unchanged bit for bit and o_t = S0^T q_t */
    for (size_t i = 0; i < nk; ++i) g[i] = 0.0;
    for (size_t i = 0; i < nb; ++i) beta[i] = 0.0;
    CHECK(kda_oracle_recurrence_f64(q, k, v, g, beta, cu, NS, H, DK, DV, S0, o, S, 3) == ORACLE_OK,
          "identity run");
    for (size_t i = 0; i < ns; ++i) CHECK(S[i] == S0[i], "identity keeps the state");
    {
        const int t = 7, h = 2, n = 2;  /* token 7 lies in sequence 2 */
        for (int j = 0; j < DV; ++j) {
            double ref = 0;
            for (int i = 0; i < DK; ++i)
                ref += S0[(((size_t)n * H + h) * DK + i) * DV + j] * q[((size_t)t * H + h) * DK + i];
            CHECK(fabs(o[((size_t)t * H + h) * DV + j] - ref) <= 1e-12, "identity read");
        }
    }

    /* argument errors */
    const int32_t bad0[NS + 1] = {1, 5, 5, 22, 23}, bad1[NS + 1] = {0, 5, 4, 22, 23};
    CHECK(kda_oracle_recurrence_f64(NULL, k, v, g, beta, cu, NS, H, DK, DV, NULL, o, NULL, 1) ==
              ORACLE_BAD_ARG, "null q");
    CHECK(kda_oracle_recurrence_f64(q, k, v, g, beta, bad0, NS, H, DK, DV, NULL, o, NULL, 1) ==
              ORACLE_BAD_ARG, "cu[0] != 0");
    CHECK(kda_oracle_recurrence_f64(q, k, v, g, beta, bad1, NS, H, DK, DV, NULL, o, NULL, 1) ==
              ORACLE_BAD_ARG, "decreasing cu");
    CHECK(kda_oracle_recurrence_f64(q, k, v, g, beta, cu, -1, H, DK, DV, NULL, o, NULL, 1) ==
              ORACLE_BAD_ARG, "negative n_seqs");
    CHECK(kda_oracle_recurrence_f32(qf, kf, vf, gf, bf, cu, NS, 0, DK, DV, NULL, of, NULL, 1) ==
              ORACLE_BAD_ARG, "zero heads");
    {
        const int32_t none[1] = {0};
        CHECK(kda_oracle_recurrence_f64(q, k, v, g, beta, none, 0, H, DK, DV, NULL, o, NULL, 1) ==
                  ORACLE_OK, "no sequences");
    }
    free(q); free(k); free(g); free(v); free(beta); free(o); free(S0); free(S);
    free(qf); free(kf); free(gf); free(vf); free(bf); free(of); free(S0f); free(Sf);
    return 0;
}

static int conv_cases(void) {
    enum { NS = 3, CCH = 6 };
    const int32_t cu[NS + 1] = {0, 2, 2, 9};  /* lengths 2, 0, 7 */
    const int T = cu[NS];
    double *x = malloc((size_t)T * CCH * 8), *y = malloc((size_t)T * CCH * 8);
    double *w = malloc((size_t)CCH * 4 * 8), *tin = malloc((size_t)NS * 3 * CCH * 8);
    double *tout = malloc((size_t)NS * 3 * CCH * 8);
    for (int i = 0; i < T * CCH; ++i) x[i] = uniform();
    for (int i = 0; i < CCH * 4; ++i) w[i] = uniform();
    for (int i = 0; i < NS * 3 * CCH; ++i) tin[i] = uniform();
    CHECK(kda_oracle_short_conv_f64(x, w, cu, NS, CCH, tin, y, tout) == ORACLE_OK, "conv");
    for (int c = 0; c < CCH; ++c) {
        /* sequence 0 (2 tokens): its tail is x_{-1} of the old tail, then x_0, x_1 */
        CHECK(tout[(0 * 3 + 0) * CCH + c] == tin[(0 * 3 + 2) * CCH + c], "short tail, oldest");
        CHECK(tout[(0 * 3 + 1) * CCH + c] == x[0 * CCH + c], "short tail, x_0");
        CHECK(tout[(0 * 3 + 2) * CCH + c] == x[1 * CCH + c], "short tail, x_1");
        /* the empty sequence 1 passes its tail through */
        for (int m = 0; m < 3; ++m)
            CHECK(tout[(1 * 3 + m) * CCH + c] == tin[(1 * 3 + m) * CCH + c], "empty tail");
        /* first output of sequence 2 reads the three tail values and x_2 */
        double ref = 0;
        for (int j = 0; j < 3; ++j) ref += w[c * 4 + j] * tin[(2 * 3 + j) * CCH + c];
        ref += w[c * 4 + 3] * x[2 * CCH + c];
        CHECK(fabs(y[2 * CCH + c] - ref) <= 1e-12, "conv reads the tail");
    }
    CHECK(kda_oracle_short_conv_f64(x, w, cu, NS, CCH, NULL, y, NULL) == ORACLE_OK, "conv, no tail");
    CHECK(kda_oracle_short_conv_f64(NULL, w, cu, NS, CCH, NULL, y, NULL) == ORACLE_BAD_ARG,
          "conv, null x");
    free(x); free(y); free(w); free(tin); free(tout);
    return 0;
}

static int l2_cases(void) {
    enum { ROWS = 5, WIDTH = 32, HD = 16 };
    double* x = malloc((size_t)ROWS * WIDTH * 8);
    for (int i = 0; i < ROWS * WIDTH; ++i) x[i] = uniform();
    CHECK(kda_oracle_l2norm_heads_f64(x, ROWS, WIDTH, HD, 0.0) == ORACLE_OK, "l2norm");
    for (int r = 0; r < ROWS; ++r)
        for (int h = 0; h < WIDTH / HD; ++h) {
            double ss = 0;
            for (int e = 0; e < HD; ++e) ss += x[r * WIDTH + h * HD + e] * x[r * WIDTH + h * HD + e];
            CHECK(fabs(ss - 1.0) < 1e-12, "unit norm");
        }
    CHECK(kda_oracle_l2norm_heads_f64(x, ROWS, WIDTH, 12, 0.0) == ORACLE_BAD_ARG, "width % head");
    free(x);
    return 0;
}

int main(void) {
    if (recurrence_cases() || conv_cases() || l2_cases()) return 1;
    printf("OK\n");
    return 0;
}
