// k_elementwise.hip — the small kernels around the GEMMs and attention of the verify pass:
// draft-tree bookkeeping, RoPE angles, the embedding gather with the first RMSNorm, the split-K
// passes of the narrow projections (RoPE + KV store; residual add + RMSNorm), the vocab-wide
// greedy choice with the accepted-path walk, and the commit of the accepted path's KV rows.
//
// Lossless greedy verification: a draft token is accepted only if it equals the target's greedy
// choice after its parent, and only along a path whose every earlier token was accepted
// [SpecPilot digest, airadar.tv — "Risks"]; tree tokens are conditioned on their own root path
// [JetSpec article, seventnews.com — "Technical architecture"].
#include "kernels.hpp"

namespace sv {

// ---- draft tree: validation, depth, ancestor mask, position ---------------------------------
// One wavefront per request. A request is marked bad (status -1) for a token outside the
// vocabulary, a malformed parent array (parent[0] != -1, or parent[i] outside [0, i)), a
// negative context, or pages that do not cover positions [0, ctx + K).
__global__ __launch_bounds__(64) void tree_prep_kernel(
    const int32_t *__restrict__ tokens, const int32_t *__restrict__ parent,
    const int32_t *__restrict__ ctx_len, const int32_t *__restrict__ block_table, int max_pages,
    int n_pages, int K, int vocab, int32_t *__restrict__ depth, int32_t *__restrict__ pos,
    uint64_t *__restrict__ anc, int32_t *__restrict__ status) {
    __shared__ int32_t s_depth[64];
    __shared__ uint64_t s_anc[64];
    __shared__ int s_tree_bad;
    const int b = blockIdx.x, lane = threadIdx.x;
    int bad = 0;
    if (lane < K) {
        const int t = tokens[(int64_t)b * K + lane];
        bad |= (t < 0 || t >= vocab);
    }
    int ctx = 0;
    if (ctx_len != nullptr) {
        ctx = ctx_len[b];
        if (ctx < 0) {
            bad = 1;
        } else {
            const int64_t need = ((int64_t)ctx + K + 15) / 16;
            if (need > max_pages) {
                bad = 1;
            } else {
                for (int p = lane; p < need; p += 64) {
                    const int id = block_table[(int64_t)b * max_pages + p];
                    bad |= (id < 0 || id >= n_pages);
                }
            }
        }
    }
    if (lane == 0) {
        int tb = 0;
        s_depth[0] = 0;
        s_anc[0] = 1ull;
        if (parent != nullptr && parent[(int64_t)b * K] != -1) tb = 1;
        for (int i = 1; i < K; ++i) {
            int p = parent != nullptr ? parent[(int64_t)b * K + i] : i - 1;
            if (p < 0 || p >= i) { tb = 1; p = 0; }
            s_depth[i] = s_depth[p] + 1;
            s_anc[i] = s_anc[p] | (1ull << i);
        }
        s_tree_bad = tb;
    }
    __syncthreads();
    bad |= s_tree_bad;
    bad = __any(bad);
    if (lane < K) {
        const int64_t n = (int64_t)b * K + lane;
        const int dd = bad ? 0 : s_depth[lane];
        depth[n] = dd;
        pos[n] = ctx + dd;
        anc[n] = bad ? (1ull << lane) : s_anc[lane];
    }
    if (lane == 0) status[b] = bad ? -1 : 0;
}

hipError_t tree_prep(const int32_t *tokens, const int32_t *parent, const int32_t *ctx_len,
                     const int32_t *block_table, int max_pages, int n_pages, int B, int K,
                     int vocab, const NodeInfo &ni, hipStream_t st) {
    hipLaunchKernelGGL(tree_prep_kernel, dim3(B), dim3(64), 0, st, tokens, parent, ctx_len,
                       block_table, max_pages, n_pages, K, vocab, ni.depth, ni.pos, ni.anc,
                       ni.status);
    return hipGetLastError();
}

// ---- RoPE angles: (cos, sin) of pos * theta^(-2j/d), evaluated in double --------------------
__global__ void rope_table_kernel(const int32_t *__restrict__ pos, int D, double theta,
                                  float2 *__restrict__ cs) {
    const int row = blockIdx.x, j = threadIdx.x;
    const double inv_freq = pow(theta, -2.0 * (double)j / (double)D);
    const double ang = (double)pos[row] * inv_freq;
    cs[(int64_t)row * (D / 2) + j] = make_float2((float)cos(ang), (float)sin(ang));
}

hipError_t rope_table(const NodeInfo &ni, int M, int D, double theta, hipStream_t st) {
    hipLaunchKernelGGL(rope_table_kernel, dim3(M), dim3(D / 2), 0, st, ni.pos, D, theta, ni.rope);
    return hipGetLastError();
}

// ---- row-wise RMSNorm helpers (one 1024-thread workgroup per row) --------------------------------
// RMSNorm: u = bf16((x / sqrt(mean(x^2) + eps)) * g), the sum of squares in fp32. Thread t owns
// the column quads t, t + 1024, ... (NQ of them, H <= 4 * 1024 * NQ); quads past the row re-read
// the last one and take no part in sums or stores, so every load is unconditional and all of a
// row's loads are in flight together.
constexpr int kRowThreads = 1024;

__device__ __forceinline__ float block_sum_1024(float v, float *red) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < kRowThreads / 64; ++i) t += red[i];
    return t;
}

template <int NQ>
struct RowQuads {
    int off[NQ];                 // column of each quad (clamped into the row)
    bool live[NQ];
    __device__ __forceinline__ explicit RowQuads(int H) {
        const int nquad = H / 4;
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int q = threadIdx.x + i * kRowThreads;
            live[i] = q < nquad;
            off[i] = (live[i] ? q : nquad - 1) * 4;
        }
    }
};

__device__ __forceinline__ void unpack4(uint2 v, float (&o)[4]) {
    const bf16 *b = reinterpret_cast<const bf16 *>(&v);
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = to_f(b[j]);
}

// u is stored in fragment order (frag_off), the operand order of the next projection.
template <int NQ>
__device__ __forceinline__ void norm_store(const RowQuads<NQ> &rq, const float (&xv)[NQ][4],
                                           const uint2 (&g)[NQ], float ss, int row, int H,
                                           float eps, bf16 *__restrict__ u) {
    const float inv = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        if (!rq.live[i]) continue;
        float gf[4];
        unpack4(g[i], gf);
        float o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = (xv[i][j] * inv) * gf[j];
        store4(u + frag_off(row, rq.off[i], H), o[0], o[1], o[2], o[3]);
    }
}

// y[i] = sum over s of p[s * stride + off[i]], in split order. Loads go out SP splits at a time
// (slots past the last split re-read it and are not added).
template <int SP, int NQ>
__device__ __forceinline__ void split_sum(const float *__restrict__ p, const int (&off)[NQ],
                                          int64_t stride, int splits, floatx4 (&y)[NQ]) {
#pragma unroll
    for (int i = 0; i < NQ; ++i) y[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < splits; s0 += SP) {
        floatx4 v[SP][NQ];
#pragma unroll
        for (int t = 0; t < SP; ++t) {
            const int s = s0 + t < splits ? s0 + t : splits - 1;
#pragma unroll
            for (int i = 0; i < NQ; ++i) v[t][i] = *(const floatx4 *)(p + s * stride + off[i]);
        }
#pragma unroll
        for (int t = 0; t < SP; ++t) {
            // a select, not a branch: a branch lets the compiler sink the load behind it
            const bool use = s0 + t < splits;
#pragma unroll
            for (int i = 0; i < NQ; ++i) y[i] = use ? y[i] + v[t][i] : y[i];
        }
    }
}

// Split-load group for a split count: the next power of two, at most 8.
inline int split_group(int splits) { return splits <= 1 ? 1 : splits <= 2 ? 2 : splits <= 4 ? 4 : 8; }
// Quads per thread for a hidden size: 1, 2 or 4.
inline int row_quads(int H) {
    const int n = (H / 4 + kRowThreads - 1) / kRowThreads;
    return n <= 1 ? 1 : n <= 2 ? 2 : 4;
}

// ---- embedding gather + first RMSNorm ------------------------------------------------------------
template <int NQ>
__global__ __launch_bounds__(kRowThreads) void embed_norm_kernel(
    const int32_t *__restrict__ tokens, const bf16 *__restrict__ table, int H, int vocab,
    const bf16 *__restrict__ gain, float eps, bf16 *__restrict__ x, bf16 *__restrict__ u,
    bf16 *__restrict__ trace) {
    __shared__ float red[kRowThreads / 64];
    const int row = blockIdx.x;
    const RowQuads<NQ> rq(H);
    uint2 g[NQ];
#pragma unroll
    for (int i = 0; i < NQ; ++i) g[i] = *(const uint2 *)(gain + rq.off[i]);
    int tok = tokens[row];
    if (tok < 0 || tok >= vocab) tok = 0;   // the request is already marked bad; stay in bounds
    const bf16 *src = table + (int64_t)tok * H;
    uint2 e[NQ];
#pragma unroll
    for (int i = 0; i < NQ; ++i) e[i] = *(const uint2 *)(src + rq.off[i]);
    float xv[NQ][4];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        unpack4(e[i], xv[i]);
        if (!rq.live[i]) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) ss += xv[i][j] * xv[i][j];
        *(uint2 *)(x + (int64_t)row * H + rq.off[i]) = e[i];
        if (trace) *(uint2 *)(trace + (int64_t)row * H + rq.off[i]) = e[i];
    }
    ss = block_sum_1024(ss, red);
    norm_store(rq, xv, g, ss, row, H, eps, u);
}

hipError_t embed_norm(const int32_t *tokens, const bf16 *table, const bf16 *gain, int M, int H,
                      int vocab, float eps, bf16 *x, bf16 *u, bf16 *trace, hipStream_t st) {
#define SV_EMBED(NQ)                                                                              \
    hipLaunchKernelGGL(embed_norm_kernel<NQ>, dim3(M), dim3(kRowThreads), 0, st, tokens, table, H, \
                       vocab, gain, eps, x, u, trace)
    switch (row_quads(H)) {
        case 1: SV_EMBED(1); break;
        case 2: SV_EMBED(2); break;
        default: SV_EMBED(4); break;
    }
#undef SV_EMBED
    return hipGetLastError();
}

// ---- QKV split-K pass: sum, bf16, RoPE, q / K / V stores -----------------------------------------
// One workgroup per (row, head of q, k or v); thread j handles the rotation pair (j, j + D/2).
// The cache slot, the angles and every split's partials are requested before any is used.
template <int SP>
__global__ void reduce_qkv_kernel(const float *__restrict__ P, int splits, int M,
                                  const float2 *__restrict__ rope, const int32_t *__restrict__ status,
                                  const int32_t *__restrict__ ctx_len,
                                  const int32_t *__restrict__ block_table, int max_pages, int K,
                                  int nq, int nkv, int D, bf16 *__restrict__ q,
                                  bf16 *__restrict__ k_pool, bf16 *__restrict__ v_pool) {
#pragma clang fp contract(off)
    const int row = blockIdx.x, head = blockIdx.y, j = threadIdx.x;
    const int half = D / 2;
    const int N = (nq + 2 * nkv) * D;
    const int64_t pstride = (int64_t)M * N;
    const float *pr = P + (int64_t)row * N + head * D + j;
    const bool is_q = head < nq, is_k = !is_q && head < nq + nkv;
    const int b = row / K, il = row % K;
    int page = 0, slot = 0;
    bool store_kv = false;
    if (!is_q) {
        store_kv = status[b] == 0;
        const int pos = ctx_len[b] + il;
        if (store_kv) page = page_of(block_table, max_pages, b, pos);
        slot = pos & 15;
    }
    float2 cs = make_float2(1.f, 0.f);
    if (head < nq + nkv) cs = rope[(int64_t)row * half + j];
    float a = 0.f, c = 0.f;
    for (int s0 = 0; s0 < splits; s0 += SP) {
        float va[SP], vc[SP];
#pragma unroll
        for (int t = 0; t < SP; ++t) {
            const int s = s0 + t < splits ? s0 + t : splits - 1;
            va[t] = pr[s * pstride];
            vc[t] = pr[s * pstride + half];
        }
#pragma unroll
        for (int t = 0; t < SP; ++t) {
            const bool use = s0 + t < splits;   // a select, so the loads stay ahead of the sums
            a = use ? a + va[t] : a;
            c = use ? c + vc[t] : c;
        }
    }
    a = round_bf(a);
    c = round_bf(c);
    bf16 lo, hi;
    if (head < nq + nkv) {
        lo = to_bf(a * cs.x - c * cs.y);
        hi = to_bf(c * cs.x + a * cs.y);
    } else {
        lo = to_bf(a);
        hi = to_bf(c);
    }
    if (is_q) {
        bf16 *qh = q + ((int64_t)row * nq + head) * D;
        qh[j] = lo;
        qh[j + half] = hi;
        return;
    }
    if (!store_kv) return;
    if (is_k) {
        bf16 *kr = k_pool + (((int64_t)page * nkv + (head - nq)) * 16 + slot) * D;
        kr[j] = lo;
        kr[j + half] = hi;
    } else {
        bf16 *vr = v_pool + (((int64_t)page * nkv + (head - nq - nkv)) * D) * 16 + slot;
        vr[j * 16] = lo;
        vr[(j + half) * 16] = hi;
    }
}

hipError_t reduce_qkv(const float *P, int splits, const NodeInfo &ni, const int32_t *ctx_len,
                      const int32_t *block_table, int max_pages, int B, int K, int nq, int nkv,
                      int D, bf16 *q, bf16 *k_pool, bf16 *v_pool, hipStream_t st) {
#define SV_QKV(SP)                                                                                \
    hipLaunchKernelGGL(reduce_qkv_kernel<SP>, dim3(B * K, nq + 2 * nkv), dim3(D / 2), 0, st, P,    \
                       splits, B * K, ni.rope, ni.status, ctx_len, block_table, max_pages, K, nq, \
                       nkv, D, q, k_pool, v_pool)
    switch (split_group(splits)) {
        case 1: SV_QKV(1); break;
        case 2: SV_QKV(2); break;
        case 4: SV_QKV(4); break;
        default: SV_QKV(8); break;
    }
#undef SV_QKV
    return hipGetLastError();
}

// ---- residual split-K pass + RMSNorm: x = bf16(x + bf16(sum_s P[s])), u = RMSNorm(x) * g --------
template <int NQ, int SP>
__global__ __launch_bounds__(kRowThreads) void reduce_resid_norm_kernel(
    const float *__restrict__ P, int splits, int M, int H, const bf16 *__restrict__ gain, float eps,
    bf16 *__restrict__ x, bf16 *__restrict__ u, bf16 *__restrict__ trace) {
    __shared__ float red[kRowThreads / 64];
    const int row = blockIdx.x;
    const RowQuads<NQ> rq(H);
    bf16 *xr = x + (int64_t)row * H;
    uint2 xo[NQ], g[NQ];
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        xo[i] = *(const uint2 *)(xr + rq.off[i]);
        g[i] = *(const uint2 *)(gain + rq.off[i]);
    }
    floatx4 y[NQ];
    split_sum<SP>(P + (int64_t)row * H, rq.off, (int64_t)M * H, splits, y);
    float xv[NQ][4];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        float xf[4];
        unpack4(xo[i], xf);
        bf16 out[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            xv[i][j] = round_bf(xf[j] + round_bf(y[i][j]));
            out[j] = to_bf(xv[i][j]);
        }
        if (!rq.live[i]) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) ss += xv[i][j] * xv[i][j];
        *(uint2 *)(xr + rq.off[i]) = *reinterpret_cast<const uint2 *>(out);
        if (trace)
            *(uint2 *)(trace + (int64_t)row * H + rq.off[i]) = *reinterpret_cast<const uint2 *>(out);
    }
    ss = block_sum_1024(ss, red);
    norm_store(rq, xv, g, ss, row, H, eps, u);
}

hipError_t reduce_resid_norm(const float *P, int splits, int M, int H, const bf16 *gain, float eps,
                             bf16 *x, bf16 *u, bf16 *trace, hipStream_t st) {
#define SV_RRN(NQ, SP)                                                                            \
    hipLaunchKernelGGL((reduce_resid_norm_kernel<NQ, SP>), dim3(M), dim3(kRowThreads), 0, st, P,   \
                       splits, M, H, gain, eps, x, u, trace)
#define SV_RRN_SP(NQ)                        \
    switch (split_group(splits)) {           \
        case 1: SV_RRN(NQ, 1); break;        \
        case 2: SV_RRN(NQ, 2); break;        \
        case 4: SV_RRN(NQ, 4); break;        \
        default: SV_RRN(NQ, 8); break;       \
    }
    switch (row_quads(H)) {
        case 1: SV_RRN_SP(1); break;
        case 2: SV_RRN_SP(2); break;
        default: SV_RRN_SP(4); break;
    }
#undef SV_RRN_SP
#undef SV_RRN
    return hipGetLastError();
}

// ---- greedy choice from caller logits: per (row, chunk of 2048 columns) -----------------------
constexpr int kArgChunk = 2048;

__device__ __forceinline__ void block_best_256(float &bv, int &bi, float *rv, int *ri) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) { rv[w] = bv; ri[w] = bi; }
    __syncthreads();
    bv = rv[0];
    bi = ri[0];
    for (int k = 1; k < 4; ++k)
        if (better(rv[k], ri[k], bv, bi)) { bv = rv[k]; bi = ri[k]; }
}

__global__ __launch_bounds__(256) void argmax_partials_kernel(const float *__restrict__ logits,
                                                              int M, int V,
                                                              float *__restrict__ amax_val,
                                                              int *__restrict__ amax_idx) {
    __shared__ float rv[4];
    __shared__ int ri[4];
    const int row = blockIdx.x, c = blockIdx.y;
    const float *r = logits + (int64_t)row * V;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    const int end = min(V, (c + 1) * kArgChunk);
    for (int i = c * kArgChunk + threadIdx.x; i < end; i += 256)
        if (better(r[i], i, bv, bi)) { bv = r[i]; bi = i; }
    block_best_256(bv, bi, rv, ri);
    if (threadIdx.x == 0) {
        amax_val[(int64_t)c * M + row] = bv;
        amax_idx[(int64_t)c * M + row] = bi;
    }
}

hipError_t argmax_partials(const float *logits, int M, int V, float *amax_val, int *amax_idx,
                           int n_chunks, hipStream_t st) {
    hipLaunchKernelGGL(argmax_partials_kernel, dim3(M, n_chunks), dim3(256), 0, st, logits, M, V,
                       amax_val, amax_idx);
    return hipGetLastError();
}

int argmax_chunks(int V) { return (V + kArgChunk - 1) / kArgChunk; }

// ---- greedy choice per node + longest accepted root path, one workgroup per request ----------
// One workgroup per request. The per-group maxima are laid out [group][row], so thread t reads
// node i = t % K of groups t / K, t / K + G, ... (G = 1024 / K threads per node): the K rows of a
// request are adjacent, so each pass reads K contiguous floats per group. The per-thread bests are
// then merged in LDS over the G threads of each node (the order is total: larger value, then lower
// index), and thread 0 walks the tree.
__global__ __launch_bounds__(1024) void argmax_accept_kernel(
    const float *__restrict__ amax_val, const int *__restrict__ amax_idx, int n_groups,
    const int32_t *__restrict__ tokens, const int32_t *__restrict__ parent,
    const int32_t *__restrict__ depth, const int32_t *__restrict__ status, int M, int K,
    int32_t *__restrict__ greedy, int32_t *__restrict__ accepted_len, int32_t *__restrict__ bonus,
    int32_t *__restrict__ path, const uint32_t *__restrict__ err) {
    __shared__ float rv[1024];
    __shared__ int ri[1024];
    __shared__ int s_arg[64];
    const int b = blockIdx.x;
    const int t = threadIdx.x;
    const int G = 1024 / K;
    const int i = t % K, sub = t / K;
    const bool active = sub < G;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    if (active) {
        const int64_t row = (int64_t)b * K + i;
        constexpr int UN = 8;    // loads in flight per thread
        int g = sub;
        for (; g + (UN - 1) * G < n_groups; g += UN * G) {
            float v[UN];
            int ix[UN];
#pragma unroll
            for (int u = 0; u < UN; ++u) {
                v[u] = amax_val[(int64_t)(g + u * G) * M + row];
                ix[u] = amax_idx[(int64_t)(g + u * G) * M + row];
            }
#pragma unroll
            for (int u = 0; u < UN; ++u)
                if (better(v[u], ix[u], bv, bi)) { bv = v[u]; bi = ix[u]; }
        }
        for (; g < n_groups; g += G) {
            const float v = amax_val[(int64_t)g * M + row];
            const int ix = amax_idx[(int64_t)g * M + row];
            if (better(v, ix, bv, bi)) { bv = v; bi = ix; }
        }
    }
    rv[t] = bv;
    ri[t] = bi;
    __syncthreads();
    for (int s = 1; s < G; s <<= 1) {
        if (active && (sub & (2 * s - 1)) == 0 && sub + s < G) {
            const float ov = rv[t + s * K];
            const int oi = ri[t + s * K];
            if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
            rv[t] = bv;
            ri[t] = bi;
        }
        __syncthreads();
    }
    if (t < K) {
        s_arg[t] = ri[t];
        if (greedy) greedy[(int64_t)b * K + t] = ri[t];
    }
    __syncthreads();
    if (t != 0) return;
    int32_t *pr = path + (int64_t)b * K;
    for (int j = 0; j < K; ++j) pr[j] = -1;
    if (status[b] != 0 || (err != nullptr && *err != 0u)) {
        accepted_len[b] = -1;
        bonus[b] = -1;
        return;
    }
    uint64_t ok = 1ull;          // bit j: node j accepted
    int best = 0;
    const int32_t *tk = tokens + (int64_t)b * K;
    const int32_t *dp = depth + (int64_t)b * K;
    for (int j = 1; j < K; ++j) {
        const int p = parent != nullptr ? parent[(int64_t)b * K + j] : j - 1;
        if (((ok >> p) & 1ull) && tk[j] == s_arg[p]) {
            ok |= 1ull << j;
            if (dp[j] > dp[best]) best = j;
        }
    }
    accepted_len[b] = dp[best];
    bonus[b] = s_arg[best];
    for (int node = best; node >= 0; node = (node == 0 ? -1 : (parent != nullptr ? parent[(int64_t)b * K + node] : node - 1)))
        pr[dp[node]] = node;
}

hipError_t argmax_accept(const float *amax_val, const int *amax_idx, int n_groups,
                         const int32_t *tokens, const int32_t *parent, const NodeInfo &ni, int B,
                         int K, int32_t *greedy, int32_t *accepted_len, int32_t *bonus,
                         int32_t *path, hipStream_t st, const uint32_t *err) {
    hipLaunchKernelGGL(argmax_accept_kernel, dim3(B), dim3(1024), 0, st, amax_val, amax_idx, n_groups,
                       tokens, parent, ni.depth, ni.status, B * K, K, greedy, accepted_len, bonus,
                       path, err);
    return hipGetLastError();
}

// ---- commit: slot ctx + t <- slot ctx + path[t], t = 0..a, every layer, K and V -------------
// A request's commit is all or nothing, and both kernels below decide it by the same rule
// (commit_part_ok, evaluated over all parts): 0 <= a < K; the path starts at the root
// (path[0] = 0) and names a node at depth t or deeper in slot t (0 <= t <= a: t <= path[t] < K,
// node ids being topological); ctx >= 0, ctx + K fits the request's page budget and every page
// of positions ctx .. ctx + K - 1 is a valid page id. A request that fails keeps its rows and its
// context.

// Part i of the rule for request b: i = 0 checks a and ctx, i = 1..a+1 path entry i - 1 (i <= K),
// i = K+1..K+5 the pages of the draft slots (K <= 64 positions span at most 5 pages).
__device__ __forceinline__ bool commit_part_ok(int i, int a, int ctx, const int32_t *__restrict__ pr,
                                               const int32_t *__restrict__ block_table, int max_pages,
                                               int n_pages, int b, int K) {
    if (a < 0 || a >= K || ctx < 0 || (int64_t)ctx + K > (int64_t)max_pages * 16) return false;
    if (i >= 1 && i <= K) {
        const int t = i - 1;
        if (t > a) return true;
        const int id = pr[t];
        return t == 0 ? id == 0 : (id >= t && id < K);
    }
    if (i > K && i <= K + 5) {
        const int p = (ctx >> 4) + (i - K - 1);
        if (p * 16 >= ctx + K) return true;
        const int id = page_of(block_table, max_pages, b, p * 16);
        return id >= 0 && id < n_pages;
    }
    return true;
}

// One workgroup per (layer, request, kv head, K-or-V). All source rows are read into registers
// before any is written, so overlapping moves are safe (path[t] >= t).
__global__ __launch_bounds__(256) void commit_kv_kernel(
    const int32_t *__restrict__ accepted_len, const int32_t *__restrict__ path,
    const int32_t *__restrict__ ctx_len, const int32_t *__restrict__ block_table, int max_pages,
    int n_pages, int B, int K, int nkv, int D, int64_t layer_stride, bf16 *__restrict__ k_pool,
    bf16 *__restrict__ v_pool) {
    const int id = blockIdx.x;
    const int kv = id & 1;
    const int g = (id >> 1) % nkv;
    const int b = (id >> 1) / nkv % B;
    const int l = (id >> 1) / nkv / B;
    const int a = accepted_len[b];
    const int ctx = ctx_len[b];
    const int32_t *pr = path + (int64_t)b * K;
    const int part = threadIdx.x;     // 256 threads >= K + 6 parts
    const bool ok = commit_part_ok(part, a, ctx, pr, block_table, max_pages, n_pages, b, K);
    if (__syncthreads_and(ok) == 0) return;
    bf16 *pool = (kv == 0 ? k_pool : v_pool) + (int64_t)l * layer_stride;
    constexpr int kRegs = 64 * 128 / 256;
    bf16 vals[kRegs];
    const int n = (a + 1) * D;
    int r = 0;
    for (int e = threadIdx.x; e < n; e += 256, ++r) {
        const int t = e / D, d = e % D;
        const int ps = ctx + pr[t];
        const int page = page_of(block_table, max_pages, b, ps);
        const int64_t off = kv == 0 ? (((int64_t)page * nkv + g) * 16 + (ps & 15)) * D + d
                                    : (((int64_t)page * nkv + g) * D + d) * 16 + (ps & 15);
        vals[r] = pool[off];
    }
    __syncthreads();
    r = 0;
    for (int e = threadIdx.x; e < n; e += 256, ++r) {
        const int t = e / D, d = e % D;
        const int pd = ctx + t;
        const int page = page_of(block_table, max_pages, b, pd);
        const int64_t off = kv == 0 ? (((int64_t)page * nkv + g) * 16 + (pd & 15)) * D + d
                                    : (((int64_t)page * nkv + g) * D + d) * 16 + (pd & 15);
        pool[off] = vals[r];
    }
}

hipError_t commit_kv(const int32_t *accepted_len, const int32_t *path, const int32_t *ctx_len,
                     const int32_t *block_table, int max_pages, int n_pages, int L, int B, int K,
                     int nkv, int D, bf16 *k_pool, bf16 *v_pool, hipStream_t st) {
    const int64_t layer_stride = (int64_t)n_pages * nkv * 16 * D;
    hipLaunchKernelGGL(commit_kv_kernel, dim3(L * B * nkv * 2), dim3(256), 0, st, accepted_len, path,
                       ctx_len, block_table, max_pages, n_pages, B, K, nkv, D, layer_stride, k_pool,
                       v_pool);
    return hipGetLastError();
}

// ctx += a + 1 for every request whose commit applies (the rule above, checked part by part by
// one thread per request).
__global__ void commit_ctx_kernel(const int32_t *__restrict__ accepted_len,
                                  const int32_t *__restrict__ path,
                                  const int32_t *__restrict__ block_table, int max_pages, int n_pages,
                                  int K, int32_t *__restrict__ ctx_len, int B) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    const int a = accepted_len[b];
    const int ctx = ctx_len[b];
    const int32_t *pr = path + (int64_t)b * K;
    bool ok = true;
    for (int i = 0; i <= K + 5 && ok; ++i)
        ok = commit_part_ok(i, a, ctx, pr, block_table, max_pages, n_pages, b, K);
    if (ok) ctx_len[b] = ctx + a + 1;
}

hipError_t commit_ctx(const int32_t *accepted_len, const int32_t *path, const int32_t *block_table,
                      int max_pages, int n_pages, int K, int32_t *ctx_len, int B, hipStream_t st) {
    hipLaunchKernelGGL(commit_ctx_kernel, dim3((B + 255) / 256), dim3(256), 0, st, accepted_len,
                       path, block_table, max_pages, n_pages, K, ctx_len, B);
    return hipGetLastError();
}

// ---- streaming-read probe (measurement aid) ---------------------------------------------------
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4 *__restrict__ p, int64_t n16,
                                                         uint32_t *__restrict__ out) {
    uint32_t acc = 0;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
        const uint4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9E3779B9u) out[0] = acc;   // keeps the loads; practically never taken
}

hipError_t read_probe(const void *buf, int64_t bytes, uint32_t *out, hipStream_t st) {
    hipLaunchKernelGGL(read_probe_kernel, dim3(2048), dim3(256), 0, st,
                       static_cast<const uint4 *>(buf), bytes / 16, out);
    return hipGetLastError();
}

}  // namespace sv
