// k_rec_commit.hip — the state commit of a hybrid target's recurrent layers after acceptance.
//
// Tree verification for targets that mix recurrent layers in is named by the SpecPilot digest
// [airadar.tv — "Reasons"]; the recurrence read here is per head S <- exp(g) S + k v^T. Once the
// accepted root path is known, the committed state becomes the accepted node's:
//     S <- exp(c_best) S0 + sum_{t on the path} exp(c_best - c_t) k_t v_t^T,
// with c the running sum of the log-gates along the path (float64), a rank-n update written in
// place on the vector units.
#include "kernels.hpp"

namespace sv {

// The accepted node's state, in place: two workgroups (256 threads) per (request, head), each
// taking half the value columns. The state is stored transposed (S^T [dv][dk]); a thread owns
// entry r of rows c = cg, cg + NG, ... of S^T: S^T[c][r] = e_0 S0^T[c][r] + sum_t (e_t k_t[r])
// v_t[c], path order, with the rows of the first 16 path tokens staged in LDS and e_t k_t[r] of
// the first 8 held in registers (deeper tokens, rare, are read from memory). Held to 64
// registers, eight workgroups fit a compute unit and the grid of a 32 x 32-head batch runs in
// one round. Requests with accepted_len < 0 (failed) keep their state.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8))) void rec_commit_kernel(
    float *__restrict__ state, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ log_gate, const int32_t *__restrict__ accepted_len,
    const int32_t *__restrict__ accepted_path, int K, int H) {
    constexpr int NG = 256 / D;
    constexpr int RT = D / NG / 2;       // rows of S^T per thread (each workgroup takes half)
    constexpr int VS = 16;               // path tokens whose rows are staged in LDS
    constexpr int VR = 8;                // of those, tokens whose keys sit in registers
    __shared__ __attribute__((aligned(16))) bf16 kb[VS * D];   // k_t of the first VS path tokens
    __shared__ __attribute__((aligned(16))) bf16 vb[VS * D];   // v_t of the first VS path tokens
    __shared__ float e_s[kRecMaxK + 1];
    __shared__ float gp[kRecMaxK];        // log-gates of the path's nodes
    __shared__ int node[kRecMaxK];
    __shared__ int bad_s;

    const int wg = blockIdx.x >> 1, half = blockIdx.x & 1;
    const int b = wg / H, h = wg % H;
    const int t = threadIdx.x;
    const int a = accepted_len[b];
    if (a < 0) return;                   // uniform: a failed request keeps its state
    // this thread's entries of its rows, in flight while the path is set up
    const int r = t % D, cg = (D / 2) * half + t / D;   // cg is wave-uniform
    float *S = state + ((int64_t)b * H + h) * D * D;
    float sv[RT];
#pragma unroll
    for (int u = 0; u < RT; ++u) sv[u] = S[(int64_t)(cg + NG * u) * D + r];
    const int n = a + 1 <= K ? a + 1 : K;
    if (t < 64) {
        const int p = t < n ? accepted_path[(int64_t)b * K + t] : 0;
        const bool bad = __any(t < n && (p < 0 || p >= K));
        if (t < n) {
            node[t] = p;
            if (!bad) gp[t] = log_gate[((int64_t)b * K + p) * H + h];
        }
        if (t == 0) bad_s = (a + 1 > K || bad) ? 1 : 0;
    }
    __syncthreads();
    if (bad_s) return;                   // not a path this pass could have produced
    if (t <= n) {
        // t < n: decay from node t (exclusive) to the accepted node; t == n: from S0
        double s = 0.0;
        for (int u = (t < n ? t + 1 : 0); u < n; ++u) s += (double)gp[u];
        e_s[t] = expf((float)s);
    }
    {
        constexpr int TPR = D / 8;
        constexpr int NIT = 2 * VS * TPR / 256;
        bf16x8 x[NIT];
#pragma unroll
        for (int u = 0; u < NIT; ++u) {
            const int e = t + 256 * u;
            const int which = e / (VS * TPR), rem = e % (VS * TPR);
            const int tt = rem / TPR, col = (rem % TPR) * 8;
            if (tt < n)
                x[u] = *reinterpret_cast<const bf16x8 *>((which == 0 ? k : v) +
                                                         (((int64_t)b * K + node[tt]) * H + h) * D + col);
        }
#pragma unroll
        for (int u = 0; u < NIT; ++u) {
            const int e = t + 256 * u;
            const int which = e / (VS * TPR), rem = e % (VS * TPR);
            const int tt = rem / TPR, col = (rem % TPR) * 8;
            if (tt < n) *reinterpret_cast<bf16x8 *>(&(which == 0 ? kb : vb)[tt * D + col]) = x[u];
        }
    }
    __syncthreads();
    const float e0 = e_s[n];
    float kr[VR];
#pragma unroll
    for (int tt = 0; tt < VR; ++tt) kr[tt] = tt < n ? e_s[tt] * to_f(kb[tt * D + r]) : 0.f;
#pragma unroll
    for (int u = 0; u < RT; ++u) {
        const int c = cg + NG * u;
        float x = e0 * sv[u];
#pragma unroll
        for (int tt = 0; tt < VR; ++tt)
            if (tt < n) x = __builtin_fmaf(kr[tt], to_f(vb[tt * D + c]), x);
        for (int tt = VR; tt < n && tt < VS; ++tt)
            x = __builtin_fmaf(e_s[tt] * to_f(kb[tt * D + r]), to_f(vb[tt * D + c]), x);
        for (int tt = VS; tt < n; ++tt) {   // deeper paths (rare): rows straight from memory
            const int64_t row = (((int64_t)b * K + node[tt]) * H + h) * D;
            x = __builtin_fmaf(e_s[tt] * to_f(k[row + r]), to_f(v[row + c]), x);
        }
        S[(int64_t)c * D + r] = x;
    }
}

hipError_t rec_commit(float *state, const bf16 *k, const bf16 *v, const float *log_gate,
                      const int32_t *accepted_len, const int32_t *accepted_path, int B, int K, int H,
                      int D, hipStream_t st) {
    const dim3 grid((unsigned)(2 * B * H));   // two workgroups per state: halves of its rows
    if (D == 128)
        hipLaunchKernelGGL(rec_commit_kernel<128>, grid, dim3(256), 0, st, state, k, v, log_gate,
                           accepted_len, accepted_path, K, H);
    else
        hipLaunchKernelGGL(rec_commit_kernel<64>, grid, dim3(256), 0, st, state, k, v, log_gate,
                           accepted_len, accepted_path, K, H);
    return hipGetLastError();
}

}  // namespace sv
