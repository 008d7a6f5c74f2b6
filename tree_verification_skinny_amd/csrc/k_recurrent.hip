// k_recurrent.hip — tree verification for the recurrent layers of a hybrid target (the state
// commit after acceptance is in k_rec_commit.hip).
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
// only through the mask and the path sums, exactly as the attention layers see it. Path sums are
// taken in float64 (at most 64 terms); everything else accumulates in fp32.
#include "kernels.hpp"

namespace sv {

// x = hi + mid + lo with three bf16 parts, each the rounded remainder of the previous (the
// remainders are exact in fp32): the sum carries 24 significant bits, so products with bf16
// operands on the bf16 matrix core keep fp32 accuracy.
__device__ __forceinline__ void split3(const float (&x)[8], bf16x8 &hi, bf16x8 &mid, bf16x8 &lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const bf16 a = to_bf(x[e]);
        const float r1 = x[e] - to_f(a);
        const bf16 m = to_bf(r1);
        hi[e] = a;
        mid[e] = m;
        lo[e] = to_bf(r1 - to_f(m));
    }
}

// One workgroup (4 waves) per (request, head): wg = b * H + h. Rows of q, k, v are
// [B][K][H][D] bf16; the state is stored transposed, S^T [B][H][dv][dk] fp32 (element [c][r]
// holds S[r][c]); out [B][K][H][D] fp32. On the matrix core
// (v_mfma_f32_16x16x32_bf16; a lane's A fragment is row l % 16, columns 8 (l / 16) .. + 7 of a
// 16 x 32 tile, its B fragment rows 8 (l / 16) .. + 7 of column l % 16, its result rows
// 4 (l / 16) .. + 3 of column l % 16):
//   scores  S = Q K^T, wave w taking node tile w against the key tiles at or before it;
//   weights W_ij = exp(c_i - c_j) S_ij on i's path, else 0, in LDS;
//   output  O = diag(exp(c)) (Q S0) + W V, wave w taking columns 32 w .. 32 w + 31 (16 w ..
//           at D = 64) for every node tile, with S0 and W split into three bf16 parts and V
//           staged transposed in LDS.
template <int D>
__global__ __launch_bounds__(256) void rec_tree_kernel(
    const float *__restrict__ state, const bf16 *__restrict__ q, const bf16 *__restrict__ k,
    const bf16 *__restrict__ v, const float *__restrict__ log_gate,
    const int32_t *__restrict__ tree_parent, int K, int H, float *__restrict__ out,
    int32_t *__restrict__ status) {
    constexpr int RS = D / 32;           // 32-wide steps over the state's rows
    constexpr int CPW = D / 64;          // 16-column tiles per wave
    constexpr int WP = kRecMaxK + 4;     // padded LDS row of W (floats)
    constexpr int VP = kRecMaxK + 8;     // padded LDS row of V^T (bf16)
    // key rows (bf16, padded) until the scores are done, then W (fp32, row pitch WP)
    __shared__ __attribute__((aligned(16))) float kw[kRecMaxK * WP];
    bf16 *ks = reinterpret_cast<bf16 *>(kw);
    float *wl = kw;
    static_assert(kRecMaxK * (D + 8) * 2 <= kRecMaxK * WP * 4, "key rows fit the W area");
    __shared__ __attribute__((aligned(16))) bf16 vt[D * VP];
    __shared__ __attribute__((aligned(16))) bf16 qs[kRecMaxK * (D + 8)];   // query rows, padded
    __shared__ double csum[kRecMaxK];
    __shared__ uint64_t anc[kRecMaxK];
    __shared__ int bad_s;

    const int wg = blockIdx.x;
    const int b = wg / H, h = wg % H;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int r16 = lane & 15, grp = lane >> 4;
    const int NT = (K + 15) >> 4;        // node tiles
    auto row_ptr = [&](const bf16 *base, int i) { return base + (((int64_t)b * K + i) * H + h) * D; };

    // Loads go out in the order they are needed (a wave waits for its loads in issue order):
    // the tree's links and gates, the value, key and query rows (staged in LDS before the first
    // barrier), the state fragments.
    int p_in = lane - 1;
    float g_in = 0.f;
    if (t < 64 && lane < K) {
        if (tree_parent != nullptr) p_in = tree_parent[(int64_t)b * K + lane];
        g_in = log_gate[((int64_t)b * K + lane) * H + h];
    }
    constexpr int TPR = D / 8;
    constexpr int NIT = kRecMaxK * TPR / 256;
    bf16x8 vx[NIT], kx[NIT], qx[NIT];
#pragma unroll
    for (int u = 0; u < NIT; ++u) {
        const int e = t + 256 * u, j = e / TPR, col = (e % TPR) * 8;
        vx[u] = j < K ? *reinterpret_cast<const bf16x8 *>(row_ptr(v, j) + col) : bf16x8{};
    }
#pragma unroll
    for (int u = 0; u < NIT; ++u) {
        const int e = t + 256 * u, j = e / TPR, col = (e % TPR) * 8;
        kx[u] = j < K ? *reinterpret_cast<const bf16x8 *>(row_ptr(k, j) + col) : bf16x8{};
    }
#pragma unroll
    for (int u = 0; u < NIT; ++u) {
        const int e = t + 256 * u, j = e / TPR, col = (e % TPR) * 8;
        qx[u] = j < K ? *reinterpret_cast<const bf16x8 *>(row_ptr(q, j) + col) : bf16x8{};
    }

    // this wave's state fragments: column 16 ct + r16, rows 32 rs + 8 grp .. + 7, which the
    // transposed layout keeps contiguous (two 16-byte loads per fragment)
    const float *S0T = state + ((int64_t)b * H + h) * D * D;
    float sf[CPW][RS][8];
#pragma unroll
    for (int u = 0; u < CPW; ++u)
#pragma unroll
        for (int rs = 0; rs < RS; ++rs) {
            const float *src = S0T + (int64_t)(16 * (wave * CPW + u) + r16) * D + 32 * rs + 8 * grp;
            const float4 a = *reinterpret_cast<const float4 *>(src);
            const float4 c4 = *reinterpret_cast<const float4 *>(src + 4);
            sf[u][rs][0] = a.x; sf[u][rs][1] = a.y; sf[u][rs][2] = a.z; sf[u][rs][3] = a.w;
            sf[u][rs][4] = c4.x; sf[u][rs][5] = c4.y; sf[u][rs][6] = c4.z; sf[u][rs][7] = c4.w;
        }

    // ---- the tree: parent links, ancestor masks and path sums of log-gates (pointer jumping) --
    if (t < 64) {
        const int p = p_in;
        const bool ok = lane >= K || (lane == 0 ? p == -1 : (p >= 0 && p < lane));
        const bool bad = __any(!ok);
        if (lane == 0) bad_s = bad ? 1 : 0;
        if (!bad) {
            // invariant: m holds the path from lane up to (not including) ptr, cs the sum of
            // its log-gates (float64)
            uint64_t m = lane < K ? (1ull << lane) : 0ull;
            double cs = lane < K ? (double)g_in : 0.0;
            int ptr = lane < K ? p : -1;
#pragma unroll
            for (int round = 0; round < 6; ++round) {
                const int src = ptr < 0 ? 0 : ptr;
                const uint32_t lo = __shfl((uint32_t)m, src, 64);
                const uint32_t hi = __shfl((uint32_t)(m >> 32), src, 64);
                const double cp = __shfl(cs, src, 64);
                const int pp = __shfl(ptr, src, 64);
                if (ptr >= 0) {
                    m |= ((uint64_t)hi << 32) | lo;
                    cs += cp;
                    ptr = pp;
                }
            }
            if (lane < K) {
                anc[lane] = m;
                csum[lane] = cs;
            }
        }
    }
    // V^T, key and query rows staged
#pragma unroll
    for (int u = 0; u < NIT; ++u) {
        const int e = t + 256 * u, j = e / TPR, col = (e % TPR) * 8;
#pragma unroll
        for (int z = 0; z < 8; ++z) vt[(col + z) * VP + j] = vx[u][z];
        *reinterpret_cast<bf16x8 *>(&ks[j * (D + 8) + col]) = kx[u];
        *reinterpret_cast<bf16x8 *>(&qs[j * (D + 8) + col]) = qx[u];
    }
    __syncthreads();
    const bool bad = bad_s != 0;
    if (h == 0 && t == 0) status[b] = bad ? 1 : 0;
    if (bad) {
        for (int e = t; e < K * D; e += 256)
            out[(((int64_t)b * K + e / D) * H + h) * D + e % D] = 0.f;
        return;
    }

    // query fragment (node tile it, 32-wide step rs) from LDS; rows past K are zero
    auto qfrag = [&](int it, int rs) __attribute__((always_inline)) {
        return *reinterpret_cast<const bf16x8 *>(&qs[(16 * it + r16) * (D + 8) + 32 * rs + 8 * grp]);
    };

    // ---- W: wave w scores node tile w against key tiles 0..w ---------------------------------
    floatx4 sc[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) sc[jt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        if (it != wave || it >= NT) continue;   // wave-uniform: this wave's node tile only
#pragma unroll
        for (int jt = 0; jt <= it; ++jt) {
            const int j = 16 * jt + r16;
#pragma unroll
            for (int rs = 0; rs < RS; ++rs)
                sc[jt] = mfma16x16x32(qfrag(it, rs), *reinterpret_cast<const bf16x8 *>(&ks[j * (D + 8) + 32 * rs + 8 * grp]), sc[jt]);
        }
    }
    __syncthreads();                     // every wave is done with the key rows
    // W rows of this wave's node tile, all 64 key columns (zero off the path and past the tile)
    if (wave < NT) {
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            const int j = 16 * jt + r16;
            const double cj = j < K ? csum[j] : 0.0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * wave + 4 * grp + e;
                float wv = 0.f;
                if (jt <= wave && i < K && j < K && ((anc[i] >> j) & 1ull))
                    wv = expf((float)(csum[i] - cj)) * sc[jt][e];
                wl[i * WP + j] = wv;
            }
        }
    }
    __syncthreads();

    // ---- O = diag(exp(c)) (Q S0) + W V ------------------------------------------------------
    floatx4 o[CPW][4];
#pragma unroll
    for (int u = 0; u < CPW; ++u)
#pragma unroll
        for (int it = 0; it < 4; ++it) o[u][it] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < CPW; ++u)
#pragma unroll
        for (int rs = 0; rs < RS; ++rs) {
            bf16x8 hi, mid, lo;
            split3(sf[u][rs], hi, mid, lo);
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                if (it < NT) {
                    const bf16x8 qv = qfrag(it, rs);
                    o[u][it] = mfma16x16x32(qv, hi, o[u][it]);
                    o[u][it] = mfma16x16x32(qv, mid, o[u][it]);
                    o[u][it] = mfma16x16x32(qv, lo, o[u][it]);
                }
            }
        }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        if (it < NT) {
            float ec[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * it + 4 * grp + e;
                ec[e] = i < K ? expf((float)csum[i]) : 0.f;
            }
#pragma unroll
            for (int u = 0; u < CPW; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e) o[u][it][e] *= ec[e];
            // key steps that can hold an ancestor of the tile's nodes: j <= 16 it + 15
            for (int js = 0; js <= (16 * it + 15) / 32 && 32 * js < K; ++js) {
                float wv[8];
                const float4 w0 = *reinterpret_cast<const float4 *>(&wl[(16 * it + r16) * WP + 32 * js + 8 * grp]);
                const float4 w1 = *reinterpret_cast<const float4 *>(&wl[(16 * it + r16) * WP + 32 * js + 8 * grp + 4]);
                wv[0] = w0.x; wv[1] = w0.y; wv[2] = w0.z; wv[3] = w0.w;
                wv[4] = w1.x; wv[5] = w1.y; wv[6] = w1.z; wv[7] = w1.w;
                bf16x8 hi, mid, lo;
                split3(wv, hi, mid, lo);
#pragma unroll
                for (int u = 0; u < CPW; ++u) {
                    const int cc = 16 * (wave * CPW + u) + r16;
                    const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(&vt[cc * VP + 32 * js + 8 * grp]);
                    o[u][it] = mfma16x16x32(hi, vf, o[u][it]);
                    o[u][it] = mfma16x16x32(mid, vf, o[u][it]);
                    o[u][it] = mfma16x16x32(lo, vf, o[u][it]);
                }
            }
            if constexpr (CPW == 2) {
                // the wave's 32 columns of a row as one 128-byte line: lane r16 stores columns
                // 2 r16 and 2 r16 + 1, gathered from its row group's lanes
                const int s0 = 16 * grp + ((2 * r16) & 15), s1 = s0 + 1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float a0 = __shfl(o[0][it][e], s0, 64), a1 = __shfl(o[0][it][e], s1, 64);
                    const float b0 = __shfl(o[1][it][e], s0, 64), b1 = __shfl(o[1][it][e], s1, 64);
                    const int i = 16 * it + 4 * grp + e;
                    if (i < K)
                        *reinterpret_cast<float2 *>(&out[(((int64_t)b * K + i) * H + h) * D + 32 * wave + 2 * r16]) =
                            r16 < 8 ? make_float2(a0, a1) : make_float2(b0, b1);
                }
            } else {
#pragma unroll
                for (int u = 0; u < CPW; ++u) {
                    const int cc = 16 * (wave * CPW + u) + r16;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 16 * it + 4 * grp + e;
                        if (i < K) out[(((int64_t)b * K + i) * H + h) * D + cc] = o[u][it][e];
                    }
                }
            }
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

// ---- a recurrent layer inside the verify pass ------------------------------------------------
// The layer's projection leaves split-K partials P [splits][M][N] of [q | k | v | a] (N columns:
// q, k, v heads of D, then one gate input per head, then padding). One workgroup per (row,
// head), thread j takes dim j: the splits added in order, q, k, v rounded to bf16 ([M][H][D]),
// and the head's log-gate g = -softplus(bf16(a)) in fp32 (-a above a = 20), [M][H].
template <int SP>
__global__ void reduce_rec_kernel(const float *__restrict__ P, int splits, int M, int N, int H, int D,
                                  bf16 *__restrict__ q, bf16 *__restrict__ k, bf16 *__restrict__ v,
                                  float *__restrict__ g) {
    const int m = blockIdx.x, h = blockIdx.y, j = threadIdx.x;
    const int64_t pstride = (int64_t)M * N;
    const float *pr = P + (int64_t)m * N;
    const int cq = h * D + j, ck = H * D + cq, cv = 2 * H * D + cq, ca = 3 * H * D + h;
    float sq = 0.f, sk = 0.f, sv = 0.f, sa = 0.f;
    for (int s0 = 0; s0 < splits; s0 += SP) {
        float vq[SP], vk[SP], vv[SP], va[SP];
#pragma unroll
        for (int t = 0; t < SP; ++t) {
            const int s = s0 + t < splits ? s0 + t : splits - 1;
            vq[t] = pr[s * pstride + cq];
            vk[t] = pr[s * pstride + ck];
            vv[t] = pr[s * pstride + cv];
            va[t] = j == 0 ? pr[s * pstride + ca] : 0.f;
        }
#pragma unroll
        for (int t = 0; t < SP; ++t) {
            const bool use = s0 + t < splits;
            sq = use ? sq + vq[t] : sq;
            sk = use ? sk + vk[t] : sk;
            sv = use ? sv + vv[t] : sv;
            sa = use ? sa + va[t] : sa;
        }
    }
    const int64_t o = ((int64_t)m * H + h) * D + j;
    q[o] = to_bf(sq);
    k[o] = to_bf(sk);
    v[o] = to_bf(sv);
    if (j == 0) {
        const float a = round_bf(sa);
        g[(int64_t)m * H + h] = a > 20.0f ? -a : -log1pf(expf(a));
    }
}

hipError_t reduce_rec(const float *P, int splits, int M, int N, int H, int D, bf16 *q, bf16 *k, bf16 *v,
                      float *g, hipStream_t st) {
    const dim3 grid((unsigned)M, (unsigned)H);
#define SV_RREC(SP) hipLaunchKernelGGL(reduce_rec_kernel<SP>, grid, dim3(D), 0, st, P, splits, M, N, H, D, q, k, v, g)
    if (splits <= 1) SV_RREC(1);
    else if (splits <= 2) SV_RREC(2);
    else if (splits <= 4) SV_RREC(4);
    else SV_RREC(8);
#undef SV_RREC
    return hipGetLastError();
}

// The tree pass's fp32 output [M][W] (W = H D) rounded to bf16 into the O projection's operand,
// fragment order (frag_off); one thread per 4 consecutive values.
__global__ __launch_bounds__(256) void rec_operand_kernel(const float *__restrict__ out, int M, int W,
                                                          bf16 *__restrict__ x) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)M * (W / 4)) return;
    const int m = (int)(i / (W / 4)), c = (int)(i % (W / 4)) * 4;
    const floatx4 o = *(const floatx4 *)(out + (int64_t)m * W + c);
    store4(x + frag_off(m, c, W), o[0], o[1], o[2], o[3]);
}

hipError_t rec_operand(const float *out, int M, int W, bf16 *x, hipStream_t st) {
    const int64_t n = (int64_t)M * (W / 4);
    hipLaunchKernelGGL(rec_operand_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, out, M, W, x);
    return hipGetLastError();
}

}  // namespace sv
