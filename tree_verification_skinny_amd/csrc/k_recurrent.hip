// k_recurrent.hip — tree verification for the recurrent layers of a hybrid target, and the
// state commit after acceptance.
//
// The SpecPilot digest [airadar.tv — "Reasons"] and news piece [wireai.ir — key innovations]
// name tree verification for targets that mix recurrent layers in, without the recurrence.
// The reading here is a scalar-gated linear recurrence per head (gated linear attention, the
// form of Mamba-2's state-space layer): with a state S [dk][dv],
//     S <- a S + k v^T,  a = exp(g),  o = S^T q  per token,
// and in a draft tree every node continues its parent's state, the root the committed one.
//
// Forking the state per node would write K copies of dk x dv values. Instead the pass uses the
// closed form of the recurrence along a root path: with c_i the sum of the log-gates on node
// i's path (root to i, inclusive) and anc(i) that path as a 64-bit mask,
//     o_i = exp(c_i) q_i^T S0 + sum_{j in anc(i)} exp(c_i - c_j) (q_i . k_j) v_j,
// so the committed state is read once per (request, head) and never copied; the tree enters
// only through the mask and the path sums, exactly as the attention layers see it. The commit
// rebuilds the accepted node's state in place:
//     S <- exp(c_best) S0 + sum_{t on the path} exp(c_best - c_t) k_t v_t^T.
// Path sums are taken in float64 (at most 64 terms); everything else is fp32.
#include "kernels.hpp"

namespace sv {

namespace {

constexpr int kRecMaxK = 64;

// 8 bf16 -> 8 floats in LDS
__device__ __forceinline__ void put8(float *dst, bf16x8 v) {
    float4 a = make_float4(to_f(v[0]), to_f(v[1]), to_f(v[2]), to_f(v[3]));
    float4 b = make_float4(to_f(v[4]), to_f(v[5]), to_f(v[6]), to_f(v[7]));
    *reinterpret_cast<float4 *>(dst) = a;
    *reinterpret_cast<float4 *>(dst + 4) = b;
}

}  // namespace

// One workgroup (256 threads) per (request, head): wg = b * H + h. Rows of q, k, v are
// [B][K][H][D] bf16; the state [B][H][D][D] fp32; out [B][K][H][D] fp32.
template <int D>
__global__ __launch_bounds__(256) void rec_tree_kernel(
    const float *__restrict__ state, const bf16 *__restrict__ q, const bf16 *__restrict__ k,
    const bf16 *__restrict__ v, const float *__restrict__ log_gate,
    const int32_t *__restrict__ tree_parent, int K, int H, float *__restrict__ out,
    int32_t *__restrict__ status) {
    constexpr int QP = D + 4;            // padded LDS row of q and k (floats)
    constexpr int NG = 256 / D;          // node groups in the output phase
    constexpr int NPT = kRecMaxK / NG;   // nodes per thread there, at most
    __shared__ __attribute__((aligned(16))) float qs[kRecMaxK * QP];
    __shared__ __attribute__((aligned(16))) float ks[kRecMaxK * QP];
    __shared__ __attribute__((aligned(16))) float vs[kRecMaxK * D];
    __shared__ float w[kRecMaxK * kRecMaxK];
    __shared__ double csum[kRecMaxK];
    __shared__ uint64_t anc[kRecMaxK];
    __shared__ float gl[kRecMaxK];
    __shared__ int bad_s;

    const int wg = blockIdx.x;
    const int b = wg / H, h = wg % H;
    const int t = threadIdx.x, lane = t & 63;

    // ---- the tree: parent links, ancestor masks (pointer jumping), path sums of log-gates ----
    if (t < 64) {
        int p = lane - 1;
        if (tree_parent != nullptr && lane < K) p = tree_parent[(int64_t)b * K + lane];
        const bool ok = lane >= K || (lane == 0 ? p == -1 : (p >= 0 && p < lane));
        const bool bad = __any(!ok);
        if (lane < K) gl[lane] = log_gate[((int64_t)b * K + lane) * H + h];
        if (lane == 0) bad_s = bad ? 1 : 0;
        if (!bad) {
            // invariant: m holds the path from lane up to (not including) ptr
            uint64_t m = lane < K ? (1ull << lane) : 0ull;
            int ptr = lane < K ? p : -1;
#pragma unroll
            for (int round = 0; round < 6; ++round) {
                const int src = ptr < 0 ? 0 : ptr;
                const uint32_t lo = __shfl((uint32_t)m, src, 64);
                const uint32_t hi = __shfl((uint32_t)(m >> 32), src, 64);
                const int pp = __shfl(ptr, src, 64);
                if (ptr >= 0) {
                    m |= ((uint64_t)hi << 32) | lo;
                    ptr = pp;
                }
            }
            if (lane < K) anc[lane] = m;
        }
    }
    __syncthreads();
    const bool bad = bad_s != 0;
    if (h == 0 && t == 0) status[b] = bad ? 1 : 0;
    if (bad) {
        for (int e = t; e < K * D; e += 256) {
            const int i = e / D, c = e % D;
            out[(((int64_t)b * K + i) * H + h) * D + c] = 0.f;
        }
        return;
    }
    if (t < K) {
        const uint64_t m = anc[t];
        double s = 0.0;
        for (int j = 0; j < K; ++j)
            if ((m >> j) & 1ull) s += (double)gl[j];
        csum[t] = s;
    }

    // ---- q, k, v rows into LDS as fp32 -----------------------------------------------------
    {
        constexpr int TPR = D / 8;       // threads per row (16 bytes each)
        for (int e = t; e < 3 * K * TPR; e += 256) {
            const int which = e / (K * TPR), rem = e % (K * TPR);
            const int i = rem / TPR, col = (rem % TPR) * 8;
            const int64_t off = (((int64_t)b * K + i) * H + h) * D + col;
            const bf16 *src = which == 0 ? q : (which == 1 ? k : v);
            const bf16x8 x = *reinterpret_cast<const bf16x8 *>(src + off);
            float *dst = which == 0 ? &qs[i * QP + col] : (which == 1 ? &ks[i * QP + col] : &vs[i * D + col]);
            put8(dst, x);
        }
    }
    __syncthreads();

    // ---- weights w_ij = exp(c_i - c_j) (q_i . k_j) for j on i's path, else 0 ---------------
    {
        const int j = lane, i0 = t >> 6;
        float s[kRecMaxK / 4];
#pragma unroll
        for (int m = 0; m < kRecMaxK / 4; ++m) s[m] = 0.f;
        for (int r = 0; r < D; r += 4) {
            const float4 kv = *reinterpret_cast<const float4 *>(&ks[j * QP + r]);
#pragma unroll
            for (int m = 0; m < kRecMaxK / 4; ++m) {
                if (i0 + 4 * m < K) {
                    const float4 qv = *reinterpret_cast<const float4 *>(&qs[(i0 + 4 * m) * QP + r]);
                    s[m] = __builtin_fmaf(qv.x, kv.x, s[m]);
                    s[m] = __builtin_fmaf(qv.y, kv.y, s[m]);
                    s[m] = __builtin_fmaf(qv.z, kv.z, s[m]);
                    s[m] = __builtin_fmaf(qv.w, kv.w, s[m]);
                }
            }
        }
        if (j < K) {
            const double cj = csum[j];
#pragma unroll
            for (int m = 0; m < kRecMaxK / 4; ++m) {
                const int i = i0 + 4 * m;
                if (i < K) {
                    const bool on = (anc[i] >> j) & 1ull;
                    w[i * kRecMaxK + j] = on ? expf((float)(csum[i] - cj)) * s[m] : 0.f;
                }
            }
        }
    }
    __syncthreads();

    // ---- o_i[c] = exp(c_i) (q_i^T S0)[c] + sum_j w_ij v_j[c] ---------------------------------
    {
        const int c = t % D, ig = t / D;   // ig uniform over a wave
        const float *S0 = state + ((int64_t)b * H + h) * D * D;
        float acc[NPT];
#pragma unroll
        for (int m = 0; m < NPT; ++m) acc[m] = 0.f;
        for (int r0 = 0; r0 < D; r0 += 16) {
            float sv[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) sv[u] = S0[(int64_t)(r0 + u) * D + c];
#pragma unroll
            for (int u4 = 0; u4 < 4; ++u4) {
#pragma unroll
                for (int m = 0; m < NPT; ++m) {
                    const int i = ig + NG * m;
                    if (i < K) {
                        const float4 qv = *reinterpret_cast<const float4 *>(&qs[i * QP + r0 + 4 * u4]);
                        acc[m] = __builtin_fmaf(qv.x, sv[4 * u4 + 0], acc[m]);
                        acc[m] = __builtin_fmaf(qv.y, sv[4 * u4 + 1], acc[m]);
                        acc[m] = __builtin_fmaf(qv.z, sv[4 * u4 + 2], acc[m]);
                        acc[m] = __builtin_fmaf(qv.w, sv[4 * u4 + 3], acc[m]);
                    }
                }
            }
        }
#pragma unroll
        for (int m = 0; m < NPT; ++m) {
            const int i = ig + NG * m;
            if (i < K) {
                float o = expf((float)csum[i]) * acc[m];
                for (int j = 0; j < K; ++j) o = __builtin_fmaf(w[i * kRecMaxK + j], vs[j * D + c], o);
                out[(((int64_t)b * K + i) * H + h) * D + c] = o;
            }
        }
    }
}

// The accepted node's state, in place: one workgroup (256 threads) per (request, head).
// Requests with accepted_len < 0 (failed) keep their state.
template <int D>
__global__ __launch_bounds__(256) void rec_commit_kernel(
    float *__restrict__ state, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ log_gate, const int32_t *__restrict__ accepted_len,
    const int32_t *__restrict__ accepted_path, int K, int H) {
    constexpr int NG = 256 / D;
    __shared__ __attribute__((aligned(16))) float kk[kRecMaxK * D];   // e_t k_t, path order
    __shared__ __attribute__((aligned(16))) float vv[kRecMaxK * D];
    __shared__ float e_s[kRecMaxK + 1];
    __shared__ int node[kRecMaxK];
    __shared__ int bad_s;

    const int wg = blockIdx.x;
    const int b = wg / H, h = wg % H;
    const int t = threadIdx.x;
    const int a = accepted_len[b];
    if (a < 0) return;                   // uniform: a failed request keeps its state
    const int n = a + 1 <= K ? a + 1 : K;
    if (t < 64) {
        const int p = t < n ? accepted_path[(int64_t)b * K + t] : 0;
        const bool bad = __any(t < n && (p < 0 || p >= K));
        if (t < n) node[t] = p;
        if (t == 0) bad_s = (a + 1 > K || bad) ? 1 : 0;
    }
    __syncthreads();
    if (bad_s) return;                   // not a path this pass could have produced
    if (t <= n) {
        // t < n: decay from node t (exclusive) to the accepted node; t == n: from S0
        double s = 0.0;
        for (int u = (t < n ? t + 1 : 0); u < n; ++u)
            s += (double)log_gate[((int64_t)b * K + node[u]) * H + h];
        e_s[t] = expf((float)s);
    }
    __syncthreads();
    {
        constexpr int TPR = D / 8;
        for (int e = t; e < 2 * n * TPR; e += 256) {
            const int which = e / (n * TPR), rem = e % (n * TPR);
            const int tt = rem / TPR, col = (rem % TPR) * 8;
            const int64_t off = (((int64_t)b * K + node[tt]) * H + h) * D + col;
            const bf16x8 x = *reinterpret_cast<const bf16x8 *>((which == 0 ? k : v) + off);
            if (which == 0) {
                const float et = e_s[tt];
#pragma unroll
                for (int u = 0; u < 8; ++u) kk[tt * D + col + u] = et * to_f(x[u]);
            } else {
                put8(&vv[tt * D + col], x);
            }
        }
    }
    __syncthreads();
    const int c = t % D, rg = t / D;
    const float e0 = e_s[n];
    float *S = state + ((int64_t)b * H + h) * D * D;
    constexpr int RB = 8;                // rows in flight per thread
    for (int r0 = rg; r0 < D; r0 += NG * RB) {
        float sv[RB];
#pragma unroll
        for (int u = 0; u < RB; ++u) sv[u] = S[(int64_t)(r0 + NG * u) * D + c];
#pragma unroll
        for (int u = 0; u < RB; ++u) {
            const int r = r0 + NG * u;
            float x = e0 * sv[u];
            for (int tt = 0; tt < n; ++tt) x = __builtin_fmaf(kk[tt * D + r], vv[tt * D + c], x);
            S[(int64_t)r * D + c] = x;
        }
    }
}

hipError_t rec_tree(const float *state, const bf16 *q, const bf16 *k, const bf16 *v,
                    const float *log_gate, const int32_t *tree_parent, int B, int K, int H, int D,
                    float *out, int32_t *status, hipStream_t st) {
    const dim3 grid((unsigned)(B * H));
    if (D == 128)
        hipLaunchKernelGGL(rec_tree_kernel<128>, grid, dim3(256), 0, st, state, q, k, v, log_gate,
                           tree_parent, K, H, out, status);
    else
        hipLaunchKernelGGL(rec_tree_kernel<64>, grid, dim3(256), 0, st, state, q, k, v, log_gate,
                           tree_parent, K, H, out, status);
    return hipGetLastError();
}

hipError_t rec_commit(float *state, const bf16 *k, const bf16 *v, const float *log_gate,
                      const int32_t *accepted_len, const int32_t *accepted_path, int B, int K, int H,
                      int D, hipStream_t st) {
    const dim3 grid((unsigned)(B * H));
    if (D == 128)
        hipLaunchKernelGGL(rec_commit_kernel<128>, grid, dim3(256), 0, st, state, k, v, log_gate,
                           accepted_len, accepted_path, K, H);
    else
        hipLaunchKernelGGL(rec_commit_kernel<64>, grid, dim3(256), 0, st, state, k, v, log_gate,
                           accepted_len, accepted_path, K, H);
    return hipGetLastError();
}

}  // namespace sv
