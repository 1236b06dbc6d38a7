// KDA chunked prefill, fp32 vector-ALU kernel (any d in {16, 32, 64, 128}, chunk in
// {16, 32, 64}, fp32 or bf16 inputs).  Used for fp32 inputs and for the shapes
// the MFMA kernel does not cover.
//
// The recurrence (page "Ling-3.1-flash: a 560B hybrid-attention MoE, counted from
// its safetensors headers", section "How KDA and MLA split the work"):
//   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
//   o_t = S_t^T q_t,   alpha_t = exp(g_t).
// Chunked form over a chunk of C tokens with incoming state S (exact algebra):
//   b_t = sum_{s<=t} g_s (cumulative log decay inside the chunk, per channel)
//   Kt = K * e^{b},  Kh = K * e^{-b},  Qt = Q * e^{b},  Gam = e^{b_{C-1}}
//   N  = strict_lower(diag(beta) Kt Kh^T)
//   U  = (I + N)^{-1} diag(beta) (V - Kt S)            forward substitution
//   O  = Qt S + lower(Qt Kh^T) U
//   S <- Gam * S + (Kh * Gam)^T U                       (Kh * Gam = K e^{b_C - b})
// (Kt Kh^T)[t][s] = K_t K_s e^{b_t - b_s}.  Where some channel's b_C drops below
// -VEC_SLOW, Kh would overflow: that chunk forms every factor from b directly
// (e^{b_t - b_s}, e^{b_t}, e^{b_C - b_t}, all at most 1), which holds for any
// decay.
// Tokens past the end of a sequence are treated as k = q = v = 0, g = 0,
// beta = 0, which leaves the state unchanged.
//
// One workgroup per (sequence, head, slice of DVS value columns); value columns
// of the state evolve independently, so slices need no communication.
#include "kda_internal.h"

namespace kda {

constexpr float VEC_SLOW = 80.f;  // e^80 stays well inside fp32

template <int D, int C>
struct VecShape {
    static constexpr int DVS = D < 32 ? D : 32;    // value columns per workgroup
    static constexpr int NS = D / DVS;             // slices per head
    static constexpr int LD = D + 1;               // padded row of [C][D] tiles
    static constexpr int NT = 256;
    // LDS floats: Kt, Kh, Qt [C][LD]; NP [C][C]; U [C][DVS]; S [D][DVS]; Gam [D]; Beta [C];
    // the chunk's pairwise flag
    static constexpr int FLOATS = 3 * C * LD + C * C + C * DVS + D * DVS + D + C + 1;
    static constexpr size_t BYTES = sizeof(float) * FLOATS;
};

template <int D, int C, typename Tin>
__global__ void __launch_bounds__(256)
prefill_vector_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k,
                      const Tin* __restrict__ v, Gate gate,
                      const float* __restrict__ beta, const int32_t* __restrict__ cu,
                      int64_t T, int H, const float* __restrict__ s0,
                      float* __restrict__ s_final, const Tin* __restrict__ zg,
                      Tin* __restrict__ o, Snapshots snap) {
    using SH = VecShape<D, C>;
    constexpr int DVS = SH::DVS, NS = SH::NS, LD = SH::LD, NT = SH::NT;
    extern __shared__ float smem[];
    float* sKt = smem;
    float* sKh = sKt + C * LD;
    float* sQt = sKh + C * LD;
    float* sNP = sQt + C * LD;
    float* sU = sNP + C * C;
    float* sS = sU + C * DVS;
    float* sGam = sS + D * DVS;
    float* sBeta = sGam + D;
    int* sSlow = reinterpret_cast<int*>(sBeta + C);

    const int tid = threadIdx.x;
    const int slice = blockIdx.x % NS;
    const int pair = blockIdx.x / NS;  // n * H + h
    const int n = pair / H, h = pair - n * H;
    const int j0 = slice * DVS;
    int64_t tb, te;
    seq_range(cu, n, T, tb, te);

    const size_t sidx = (size_t)pair * D * D;
    for (int e = tid; e < D * DVS; e += NT) {
        const int i = e / DVS, j = e % DVS;
        sS[e] = s0 ? s0[sidx + (size_t)i * D + j0 + j] : 0.f;
    }

    const size_t rowk = (size_t)H * D;  // stride between tokens in q/k/g/v/o
    const float* g = static_cast<const float*>(gate.g);
    const float rate = gate.mode == GATE_PROJ ? __expf(gate.a_log[h]) : 0.f;
    for (int64_t c0 = tb; c0 < te; c0 += C) {
        const int L = (int)((te - c0) < C ? (te - c0) : C);
        __syncthreads();  // previous chunk done with every buffer
        if (tid == 0) *sSlow = 0;
        // raw k -> sKt, g -> sKh, q -> sQt (zeros past the end)
        for (int e = tid; e < C * D; e += NT) {
            const int t = e / D, i = e % D;
            float kv = 0.f, gv = 0.f, qv = 0.f;
            if (t < L) {
                const size_t off = (size_t)(c0 + t) * rowk + (size_t)h * D + i;
                kv = In<Tin>::load1(k + off);
                gv = gate.mode == GATE_HEAD ? g[(size_t)(c0 + t) * H + h]
                     : gate.mode == GATE_PROJ
                         ? 0.6931471805599453f *
                               proj_log2_decay(In<Tin>::load1(static_cast<const Tin*>(gate.g) + off),
                                               rate)
                         : g[off];
                qv = In<Tin>::load1(q + off);
            }
            sKt[t * LD + i] = kv;
            sKh[t * LD + i] = gv;
            sQt[t * LD + i] = qv;
        }
        for (int t = tid; t < C; t += NT)
            sBeta[t] = t >= L                    ? 0.f
                       : gate.mode == GATE_PROJ ? sigmoid_f(beta[(size_t)(c0 + t) * H + h])
                                                : beta[(size_t)(c0 + t) * H + h];
        __syncthreads();
        // cumulative log decay per channel into sKh (raw k stays in sKt, q in sQt)
        if (tid < D) {
            const int i = tid;
            float b = 0.f;
            for (int t = 0; t < C; ++t) {
                b += sKh[t * LD + i];
                sKh[t * LD + i] = b;
            }
            sGam[i] = __expf(b);
            if (b < -VEC_SLOW) *sSlow = 1;  // every writer stores the same value
        }
        __syncthreads();
        // A chunk in which some channel decays below e^-VEC_SLOW takes the
        // pairwise form: e^{-b} would overflow, so every factor is formed as
        // e^{b_t - b_s}, e^{b_t} or e^{b_C - b_t} (all at most 1) where it is
        // used, from raw k, q and b.  Otherwise, the scaled tiles.
        const bool slow = *sSlow != 0;
        if (!slow && tid < D) {
            const int i = tid;
            for (int t = 0; t < C; ++t) {
                const float kr = sKt[t * LD + i], b = sKh[t * LD + i];
                const float e = __expf(b), ei = __expf(-b);
                sKt[t * LD + i] = kr * e;
                sKh[t * LD + i] = kr * ei;
                sQt[t * LD + i] *= e;
            }
        }
        __syncthreads();
        // N = strict_lower(diag(beta) Kt Kh^T)
        for (int e = tid; e < C * C; e += NT) {
            const int t = e / C, s = e % C;
            float acc = 0.f;
            if (s < t) {
                if (!slow)
                    for (int i = 0; i < D; ++i) acc += sKt[t * LD + i] * sKh[s * LD + i];
                else
                    for (int i = 0; i < D; ++i)
                        acc += sKt[t * LD + i] * sKt[s * LD + i] *
                               __expf(sKh[t * LD + i] - sKh[s * LD + i]);
                acc *= sBeta[t];
            }
            sNP[e] = acc;
        }
        // R = diag(beta) (V - Kt S)
        for (int e = tid; e < C * DVS; e += NT) {
            const int t = e / DVS, j = e % DVS;
            float acc = 0.f;
            if (!slow)
                for (int i = 0; i < D; ++i) acc += sKt[t * LD + i] * sS[i * DVS + j];
            else
                for (int i = 0; i < D; ++i)
                    acc += sKt[t * LD + i] * __expf(sKh[t * LD + i]) * sS[i * DVS + j];
            const float vv =
                t < L ? In<Tin>::load1(v + (size_t)(c0 + t) * rowk + (size_t)h * D + j0 + j) : 0.f;
            sU[e] = sBeta[t] * (vv - acc);
        }
        __syncthreads();
        // U = (I + N)^{-1} R by forward substitution, one value column per thread
        if (tid < DVS) {
            const int j = tid;
            for (int t = 1; t < C; ++t) {
                float x = sU[t * DVS + j];
                for (int s = 0; s < t; ++s) x -= sNP[t * C + s] * sU[s * DVS + j];
                sU[t * DVS + j] = x;
            }
        }
        __syncthreads();
        // P = lower(Qt Kh^T), reusing the N buffer
        for (int e = tid; e < C * C; e += NT) {
            const int t = e / C, s = e % C;
            float acc = 0.f;
            if (s <= t) {
                if (!slow)
                    for (int i = 0; i < D; ++i) acc += sQt[t * LD + i] * sKh[s * LD + i];
                else
                    for (int i = 0; i < D; ++i)
                        acc += sQt[t * LD + i] * sKt[s * LD + i] *
                               __expf(sKh[t * LD + i] - sKh[s * LD + i]);
            }
            sNP[e] = acc;
        }
        __syncthreads();
        // O = Qt S + P U
        for (int e = tid; e < C * DVS; e += NT) {
            const int t = e / DVS, j = e % DVS;
            if (t >= L) continue;
            float acc = 0.f;
            if (!slow)
                for (int i = 0; i < D; ++i) acc += sQt[t * LD + i] * sS[i * DVS + j];
            else
                for (int i = 0; i < D; ++i)
                    acc += sQt[t * LD + i] * __expf(sKh[t * LD + i]) * sS[i * DVS + j];
            for (int s = 0; s <= t; ++s) acc += sNP[t * C + s] * sU[s * DVS + j];
            const size_t oat = (size_t)(c0 + t) * rowk + (size_t)h * D + j0 + j;
            if (zg) acc *= sigmoid_f(In<Tin>::load1(zg + oat));  // output gate
            In<Tin>::store1(o + oat, acc);
        }
        __syncthreads();
        // S <- Gam * S + (K e^{b_C - b})^T U (and the snapshot when one falls here)
        float* snp = snapshot_at(snap, n, h, H, D, c0 + L - tb, te - tb);
        for (int e = tid; e < D * DVS; e += NT) {
            const int i = e / DVS, j = e % DVS;
            const float gm = sGam[i];
            float acc = 0.f;
            if (!slow) {
                for (int t = 0; t < C; ++t) acc += (sKh[t * LD + i] * gm) * sU[t * DVS + j];
            } else {
                const float bC = sKh[(C - 1) * LD + i];
                for (int t = 0; t < C; ++t)
                    acc += sKt[t * LD + i] * __expf(bC - sKh[t * LD + i]) * sU[t * DVS + j];
            }
            sS[e] = gm * sS[e] + acc;
            if (snp) snp[(size_t)i * D + j0 + j] = sS[e];
        }
    }
    __syncthreads();
    if (s_final) {
        for (int e = tid; e < D * DVS; e += NT) {
            const int i = e / DVS, j = e % DVS;
            s_final[sidx + (size_t)i * D + j0 + j] = sS[e];
        }
    }
}

template <int D, int C, typename Tin>
static hipError_t launch_vec_t(const void* q, const void* k, const void* v, Gate g,
                               const float* beta, const int32_t* cu, int n_seqs,
                               int64_t T, int H, const float* s0, float* s_final,
                               const void* zg, void* o, Snapshots snap, hipStream_t stream) {
    using SH = VecShape<D, C>;
    const int64_t blocks = (int64_t)n_seqs * H * SH::NS;
    if (blocks == 0) return hipSuccess;
    auto kern = prefill_vector_kernel<D, C, Tin>;
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         (int)SH::BYTES);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(SH::NT), SH::BYTES, stream,
                       (const Tin*)q, (const Tin*)k, (const Tin*)v, g, beta, cu, T, H,
                       s0, s_final, (const Tin*)zg, (Tin*)o, snap);
    return hipGetLastError();
}

template <int D, typename Tin>
static hipError_t launch_vec_c(int chunk, const void* q, const void* k, const void* v,
                               Gate g, const float* beta, const int32_t* cu,
                               int n_seqs, int64_t T, int H, const float* s0, float* s_final,
                               const void* zg, void* o, Snapshots snap, hipStream_t stream) {
    switch (chunk) {
        case 16: return launch_vec_t<D, 16, Tin>(q, k, v, g, beta, cu, n_seqs, T, H, s0, s_final, zg, o, snap, stream);
        case 32: return launch_vec_t<D, 32, Tin>(q, k, v, g, beta, cu, n_seqs, T, H, s0, s_final, zg, o, snap, stream);
        case 64: return launch_vec_t<D, 64, Tin>(q, k, v, g, beta, cu, n_seqs, T, H, s0, s_final, zg, o, snap, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_prefill_vector(const void* q, const void* k, const void* v, Gate g,
                                 const float* beta, kda_dtype dtype, const int32_t* cu,
                                 int n_seqs, int64_t T, int H, int d, int chunk,
                                 const float* s0, float* s_final, const void* out_gate, void* o,
                                 Snapshots snap, hipStream_t stream) {
#define KDA_VEC(D)                                                                            \
    if (d == D) {                                                                             \
        if (dtype == KDA_BF16)                                                                \
            return launch_vec_c<D, bf16_t>(chunk, q, k, v, g, beta, cu, n_seqs, T, H, \
                                           s0, s_final, out_gate, o, snap, stream);           \
        return launch_vec_c<D, float>(chunk, q, k, v, g, beta, cu, n_seqs, T, H, s0,  \
                                      s_final, out_gate, o, snap, stream);                    \
    }
    KDA_VEC(16)
    KDA_VEC(32)
    KDA_VEC(64)
    KDA_VEC(128)
#undef KDA_VEC
    return hipErrorInvalidValue;
}

}  // namespace kda
