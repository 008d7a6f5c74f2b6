// k_gemm.hip — weight-streaming skinny GEMM for the verify pass (M = draft nodes, 1..64 rows
// per launch) on gfx950 MFMA.
//
// At batch 1 the verify pass reads every target weight for a handful of tokens, so it is bound
// by HBM, not by arithmetic [SpecPilot digest, airadar.tv — summary paragraph]. The kernel is
// built around the weight stream:
//   * Y^T = W . X^T on v_mfma_f32_16x16x32_bf16: the weight W [N][Kd] is the A operand, so each
//     lane loads its A fragment (8 consecutive bf16 of one weight row = one 128-bit load) straight
//     from HBM into registers; no LDS round trip for data used exactly once.
//   * The activations X [M][Kd] (tiny, cache resident) are the B operand, loaded with the same
//     K-permutation as W, so any K order inside a 32-step is consistent between A and B.
//   * A workgroup (4 waves) owns 16*NT weight rows and one K range; its waves interleave over
//     32-wide K steps so that at any moment the 4 waves read 4 adjacent 64-byte pieces of each
//     row. The 4 waves' sums are added in LDS in a fixed order (w0+w1+w2+w3), and K splits go to
//     separate partial buffers that the consumer adds in split order: results do not depend on
//     timing.
// MFMA lane layout (16x16x32): lane l supplies A row l%16, K elements 8*(l/16)..+7, and B
// column l%16, the same K elements; it receives D rows 4*(l/16)..+3 of column l%16.
#include "kernels.hpp"

namespace sv {

template <int NT, int MT>
struct Acc {
    floatx4 v[NT][MT];
};

// Main loop shared by both epilogues: accumulates this wave's K steps into acc.
template <int NT, int MT, int U>
__device__ __forceinline__ void skinny_mainloop(const bf16 *__restrict__ X, int ldx, int M,
                                                const bf16 *__restrict__ W, int N, int Kd, int n0,
                                                int s_begin, int s_end, Acc<NT, MT> &acc) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
    const bf16 *wp[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        int n = min(n0 + 16 * t + r16, N - 1);
        wp[t] = W + (int64_t)n * Kd + grp * 8;
    }
    const bf16 *xp[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        int m = min(16 * mt + r16, M - 1);
        xp[mt] = X + (int64_t)m * ldx + grp * 8;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc.v[t][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

    int s = s_begin + wave;
    for (; s + 4 * (U - 1) < s_end; s += 4 * U) {
        bf16x8 a[U][NT], b[U][MT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = (s + 4 * u) << 5;
#pragma unroll
            for (int t = 0; t < NT; ++t) a[u][t] = *(const bf16x8 *)(wp[t] + k);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) b[u][mt] = *(const bf16x8 *)(xp[mt] + k);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc.v[t][mt] = mfma16x16x32(a[u][t], b[u][mt], acc.v[t][mt]);
    }
    for (; s < s_end; s += 4) {
        const int k = s << 5;
        bf16x8 a[NT], b[MT];
#pragma unroll
        for (int t = 0; t < NT; ++t) a[t] = *(const bf16x8 *)(wp[t] + k);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) b[mt] = *(const bf16x8 *)(xp[mt] + k);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc.v[t][mt] = mfma16x16x32(a[t], b[mt], acc.v[t][mt]);
    }
}

// Adds the four waves' accumulators in LDS (w0 + w1 + w2 + w3); the total lands in wave 0.
template <int NT, int MT>
__device__ __forceinline__ void reduce_waves(Acc<NT, MT> &acc, floatx4 *red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (wave > 0) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) red[((wave - 1) * NT * MT + t * MT + mt) * 64 + lane] = acc.v[t][mt];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int w = 0; w < 3; ++w)
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    floatx4 o = red[(w * NT * MT + t * MT + mt) * 64 + lane];
                    acc.v[t][mt] += o;
                }
    }
}

template <int NT, int MT>
__global__ __launch_bounds__(256) void gemm_partials_kernel(const bf16 *__restrict__ X, int ldx,
                                                            int M, int m_total, int m0,
                                                            const bf16 *__restrict__ W, int N,
                                                            int Kd, int n_groups, int ksteps,
                                                            float *__restrict__ P) {
    extern __shared__ floatx4 red[];
    const int ng = blockIdx.x % n_groups;
    const int split = blockIdx.x / n_groups;
    const int n0 = ng * 16 * NT;
    const int s_begin = split * ksteps;
    const int s_end = min(s_begin + ksteps, Kd >> 5);
    constexpr int U = (NT * MT >= 8) ? 2 : 4;
    Acc<NT, MT> acc;
    skinny_mainloop<NT, MT, U>(X, ldx, M, W, N, Kd, n0, s_begin, s_end, acc);
    reduce_waves<NT, MT>(acc, red);
    if ((threadIdx.x >> 6) != 0) return;
    const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int n = n0 + 16 * t + 4 * grp;
        if (n0 + 16 * t >= N) continue;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = 16 * mt + r16;
            if (m < M) *(floatx4 *)(P + ((int64_t)split * m_total + m0 + m) * N + n) = acc.v[t][mt];
        }
    }
}

template <int NT, int MT>
__global__ __launch_bounds__(256) void gemm_argmax_kernel(const bf16 *__restrict__ X, int ldx,
                                                          int M, int m_total, int m0,
                                                          const bf16 *__restrict__ W, int N,
                                                          int Kd, int n_groups,
                                                          float *__restrict__ logits,
                                                          float *__restrict__ amax_val,
                                                          int *__restrict__ amax_idx) {
    extern __shared__ floatx4 red[];
    const int ng = blockIdx.x;
    const int n0 = ng * 16 * NT;
    constexpr int U = (NT * MT >= 8) ? 2 : 4;
    Acc<NT, MT> acc;
    skinny_mainloop<NT, MT, U>(X, ldx, M, W, N, Kd, n0, 0, Kd >> 5, acc);
    reduce_waves<NT, MT>(acc, red);
    if ((threadIdx.x >> 6) != 0) return;
    const int lane = threadIdx.x & 63, r16 = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = 16 * mt + r16;
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int n = n0 + 16 * t + 4 * grp;
            if (n0 + 16 * t >= N) continue;
            if (logits != nullptr && m < M) *(floatx4 *)(logits + (int64_t)(m0 + m) * N + n) = acc.v[t][mt];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (better(acc.v[t][mt][j], n + j, bv, bi)) { bv = acc.v[t][mt][j]; bi = n + j; }
        }
        // the 4 lanes holding column m: lane, lane ^ 16, lane ^ 32, lane ^ 48
#pragma unroll
        for (int o = 16; o < 64; o <<= 1) {
            float ov = __shfl_xor(bv, o, 64);
            int oi = __shfl_xor(bi, o, 64);
            if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
        }
        if (grp == 0 && m < M) {
            amax_val[(int64_t)ng * m_total + m0 + m] = bv;
            amax_idx[(int64_t)ng * m_total + m0 + m] = bi;
        }
    }
}

static int mt_for(int m) { return m <= 16 ? 1 : (m <= 32 ? 2 : 4); }

int gemm_groups(const GemmShape &g) {
    const int rows = 16 * g.nt;
    return (g.N + rows - 1) / rows;
}

template <int NT, int MT>
static hipError_t launch_partials(const GemmShape &g, int m0, int mc, const bf16 *X,
                                  const bf16 *W, float *P, hipStream_t st) {
    const int ng = gemm_groups(g);
    const int steps = g.Kd >> 5;
    const int ks = (steps + g.splits - 1) / g.splits;
    const size_t lds = sizeof(floatx4) * 3 * NT * MT * 64;
    hipLaunchKernelGGL((gemm_partials_kernel<NT, MT>), dim3(ng * g.splits), dim3(256), lds, st,
                       X + (int64_t)m0 * g.ldx, g.ldx, mc, g.M, m0, W, g.N, g.Kd, ng, ks, P);
    return hipGetLastError();
}

template <int NT, int MT>
static hipError_t launch_argmax(const GemmShape &g, int m0, int mc, const bf16 *X, const bf16 *W,
                                float *logits, float *av, int *ai, hipStream_t st) {
    const int ng = gemm_groups(g);
    const size_t lds = sizeof(floatx4) * 3 * NT * MT * 64;
    hipLaunchKernelGGL((gemm_argmax_kernel<NT, MT>), dim3(ng), dim3(256), lds, st,
                       X + (int64_t)m0 * g.ldx, g.ldx, mc, g.M, m0, W, g.N, g.Kd, ng, logits, av, ai);
    return hipGetLastError();
}

#define SV_DISPATCH(NTV, MTV, CALL)                                 \
    do {                                                            \
        if ((NTV) == 4) {                                           \
            if ((MTV) == 1) { CALL(4, 1); }                         \
            else if ((MTV) == 2) { CALL(4, 2); }                    \
            else { CALL(4, 4); }                                    \
        } else {                                                    \
            if ((MTV) == 1) { CALL(2, 1); }                         \
            else if ((MTV) == 2) { CALL(2, 2); }                    \
            else { CALL(2, 4); }                                    \
        }                                                           \
    } while (0)

hipError_t gemm_partials(const GemmShape &g, const bf16 *X, const bf16 *W, float *P, hipStream_t st) {
    for (int m0 = 0; m0 < g.M; m0 += 64) {
        const int mc = g.M - m0 < 64 ? g.M - m0 : 64;
        hipError_t e = hipSuccess;
#define SV_CALL(A, B) e = launch_partials<A, B>(g, m0, mc, X, W, P, st)
        SV_DISPATCH(g.nt, mt_for(mc), SV_CALL);
#undef SV_CALL
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t gemm_argmax(const GemmShape &g, const bf16 *X, const bf16 *W, float *logits,
                       float *amax_val, int *amax_idx, hipStream_t st) {
    for (int m0 = 0; m0 < g.M; m0 += 64) {
        const int mc = g.M - m0 < 64 ? g.M - m0 : 64;
        hipError_t e = hipSuccess;
#define SV_CALL(A, B) e = launch_argmax<A, B>(g, m0, mc, X, W, logits, amax_val, amax_idx, st)
        SV_DISPATCH(g.nt, mt_for(mc), SV_CALL);
#undef SV_CALL
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace sv
