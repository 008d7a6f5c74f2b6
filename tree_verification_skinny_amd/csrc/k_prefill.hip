// k_prefill.hip — the prompt prefill: the prompt of every request runs through the target in
// chunks of up to thousands of positions per pass (a chunk is a block whose tokens are all given,
// so every row is kept and its K/V committed as it is written). The projections of such a chunk
// are matrix-core bound and run the tile kernel; attention is causal over the committed context
// and the chunk itself, a block of query rows per workgroup streaming key blocks from the paged
// cache with an online softmax; the output head runs only for each request's last position.
#include "kernels.hpp"

namespace sv {

__global__ void prefill_init_kernel(int32_t *__restrict__ failed, int B) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B) failed[b] = 0;
}

// The chunk [c0, c0 + n) of every request's prompt row, contiguous: out [B][n].
__global__ void prefill_gather_kernel(const int32_t *__restrict__ prompt, int p, int c0, int n, int B,
                                      int32_t *__restrict__ out) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < B * n) out[i] = prompt[(int64_t)(i / n) * p + c0 + i % n];
}

// Row r = b * n + i of a chunk [c0, c0 + n): position ctx_len[b] + i. Request b's status is 1
// (it fails, for this and every later chunk) when it failed before, a token is outside the
// vocabulary, or its pages do not cover positions 0 .. ctx_len + n - 1 (the context the chunk
// attends to and the chunk itself) with valid page ids.
__global__ __launch_bounds__(256) void prefill_prep_kernel(
    const int32_t *__restrict__ tokens, int n, int vocab, const int32_t *__restrict__ ctx_len,
    const int32_t *__restrict__ block_table, int max_pages, int n_pages, const int32_t *__restrict__ failed,
    int32_t *__restrict__ pos, int32_t *__restrict__ status) {
    const int b = blockIdx.x;
    const int ctx = ctx_len[b];
    int bad = failed[b] != 0 || ctx < 0 || (int64_t)ctx + n > (int64_t)max_pages * kPage;
    for (int i = threadIdx.x; i < n; i += 256) {
        const int t = tokens[(int64_t)b * n + i];
        bad |= t < 0 || t >= vocab;
        pos[(int64_t)b * n + i] = ctx + i;
    }
    if (!bad) {
        const int p1 = (ctx + n - 1) >> 4;
        for (int pg = (int)threadIdx.x; pg <= p1; pg += 256) {
            const int id = block_table[(int64_t)b * max_pages + pg];
            bad |= id < 0 || id >= n_pages;
        }
    }
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) status[b] = bad ? 1 : 0;
}

// ---- causal attention of a chunk ------------------------------------------------------------
// One workgroup per (block of QB = 32 query rows, kv head, request); its 2 * group waves take one
// 16-column query tile each, columns = (q head hh of the group, row i) with hh = tile / 2. Row i of
// request b sits at position ctx + i and sees every key position <= ctx + i (the committed context
// and the chunk's earlier rows, already in the cache). Keys and values pass through LDS in blocks
// of 64 positions (four pages); per block each wave forms S^T = K . Q^T (16 x 16 x 32 MFMA), masks,
// updates its running maximum and sum per column (log2 domain) and rescales, then O^T += V^T . P^T
// with P as a bf16 high part plus a bf16 low part (as the verify pass's attention). The result,
// divided by the sum, is written in bf16 straight into the O projection's operand (fragment
// order). A failed request's rows are written as zeros.
constexpr int kPQB = 32, kPKB = 64;

template <int D, int GQ>
__global__ __launch_bounds__(128 * GQ) void prefill_attn_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k_pool, const bf16 *__restrict__ v_pool,
    const int32_t *__restrict__ block_table, int max_pages, const int32_t *__restrict__ ctx_len,
    const int32_t *__restrict__ status, int n, int nq, int nkv, float scale_log2, bf16 *__restrict__ out) {
    constexpr int KP = D + 8, VP = kPKB + 8;
    __shared__ __attribute__((aligned(16))) bf16 Ks[kPKB * KP];
    __shared__ __attribute__((aligned(16))) bf16 Vt[D * VP];
    // the longest row blocks (most keys) are dispatched first, so the short ones fill the tail
    const int i0 = (gridDim.x - 1 - blockIdx.x) * kPQB, g = blockIdx.y, b = blockIdx.z;
    constexpr int group = GQ;                              // q heads per kv head
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
    const int hh = wave >> 1;                              // q head of this wave's tile
    const int i = i0 + (wave & 1) * 16 + r16;              // query row of this lane
    const bool row_ok = i < n;
    const int ic = row_ok ? i : n - 1;
    const int head = g * group + hh;
    const int W = nq * D;
    const int64_t row = (int64_t)b * n + ic;
    if (status[b] != 0) {
        if (row_ok && grp == 0)
            for (int d0 = 0; d0 < D; d0 += 4) store4(out + frag_off(row, head * D + d0, W), 0.f, 0.f, 0.f, 0.f);
        return;
    }
    const int ctx = ctx_len[b];
    const int last = min(i0 + kPQB, n) - 1;
    const int kend = ctx + last + 1;                       // keys 0 .. kend - 1 may be visible
    const int qpos = ctx + ic;

    bf16x8 qf[D / 32];
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds)
        qf[ds] = *(const bf16x8 *)(q + (row * nq + head) * D + ds * 32 + grp * 8);
    floatx4 o[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;
    const int kr0 = 8 * (r16 >> 2) + (r16 & 3);
    const int32_t *bt = block_table + (int64_t)b * max_pages;
    constexpr int nthreads = 128 * GQ;
    const int nkb = (kend + kPKB - 1) / kPKB;

    // Staging slots of a key block (4 pages of keys [16][D], then of values [D][16], 16 bytes each);
    // thread t takes slots t + nthreads r. Its data for block j + 1 and its page ids for block
    // j + 2 are requested while block j is multiplied.
    constexpr int kSlots = 2 * 4 * 16 * D / 8;
    constexpr int kPer = (kSlots + nthreads - 1) / nthreads;
    auto slot_page = [&](int r) { return ((threadIdx.x + nthreads * r) % (kSlots / 2)) / (16 * D / 8); };
    auto load_pages = [&](int j, int (&pg)[kPer]) {
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const int kpos = j * kPKB + 16 * slot_page(r);
            pg[r] = (threadIdx.x + nthreads * r < kSlots && j < nkb && kpos < kend) ? bt[min(kpos >> 4, max_pages - 1)] : -1;
        }
    };
    auto load_kv = [&](const int (&pg)[kPer], bf16x8 (&val)[kPer]) {
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const int sl = threadIdx.x + nthreads * r;
            const bool is_v = sl >= kSlots / 2;
            const int e = ((is_v ? sl - kSlots / 2 : sl) % (16 * D / 8)) * 8;
            val[r] = pg[r] >= 0 ? stream_load((const bf16x8 *)((is_v ? v_pool : k_pool) + ((int64_t)pg[r] * nkv + g) * 16 * D + e))
                                : bf16x8{};
        }
    };
    int pg_next[kPer], pg_after[kPer];
    bf16x8 kvr[kPer];
    load_pages(0, pg_next);
    load_pages(1, pg_after);
    load_kv(pg_next, kvr);

    for (int j = 0; j < nkb; ++j) {
        const int kb = j * kPKB;
        const int nvalid = min(kPKB, kend - kb);
        __syncthreads();                                   // the previous block's products are done
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const int sl = threadIdx.x + nthreads * r;
            if (sl >= kSlots) continue;
            const bool is_v = sl >= kSlots / 2;
            const int s2 = is_v ? sl - kSlots / 2 : sl;
            const int pgi = s2 / (16 * D / 8), e = (s2 % (16 * D / 8)) * 8;
            bf16x8 val = kvr[r];
            if (!is_v) {
                *(bf16x8 *)&Ks[(16 * pgi + e / D) * KP + e % D] = val;
            } else {
                const int d = e >> 4, slot = e & 15;
#pragma unroll
                for (int jj = 0; jj < 8; ++jj)
                    if (16 * pgi + slot + jj >= nvalid) val[jj] = (bf16)0.0f;
                *(bf16x8 *)&Vt[d * VP + 16 * pgi + slot] = val;
            }
        }
        __syncthreads();
        // the next block's keys and values, and the page ids of the one after, while this one runs
#pragma unroll
        for (int r = 0; r < kPer; ++r) pg_next[r] = pg_after[r];
        load_kv(pg_next, kvr);
        load_pages(j + 2, pg_after);
        // S^T: step st (32 keys), half h: key rows st*32 + kr0 + 4h; lane's keys st*32 + 8 grp + e
        floatx4 sc[2][2];
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ds = 0; ds < D / 32; ++ds) {
                    const bf16x8 kf = *(const bf16x8 *)&Ks[(st * 32 + kr0 + 4 * hf) * KP + grp * 8 + ds * 32];
                    acc = mfma16x16x32(kf, qf[ds], acc);
                }
                sc[st][hf] = acc;
            }
        float sv[2][8];
        float mb = -INFINITY;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int kp = kb + st * 32 + 8 * grp + e;
                const float raw = (e < 4 ? sc[st][0][e] : sc[st][1][e - 4]) * scale_log2;
                sv[st][e] = (kp <= qpos && kp < kend) ? raw : -INFINITY;
                mb = fmaxf(mb, sv[st][e]);
            }
        mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
        mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
        const float mn = fmaxf(m, mb);
        const bool none = mn == -INFINITY;
        const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m - mn);
        bf16x8 ph[2], pl[2];
        float ps = 0.f;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pv = none ? 0.f : __builtin_amdgcn_exp2f(sv[st][e] - mn);
                const bf16 hi = to_bf(pv);
                ph[st][e] = hi;
                pl[st][e] = to_bf(pv - to_f(hi));
                ps += pv;
            }
        l = l * alpha + ps;
        m = mn;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[dt] = o[dt] * alpha;
        // O^T += V^T . P^T: value rows r16 + 16 dt, keys of step st
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                const bf16x8 vf = *(const bf16x8 *)&Vt[(r16 + 16 * dt) * VP + st * 32 + grp * 8];
                o[dt] = mfma16x16x32(vf, ph[st], o[dt]);
                o[dt] = mfma16x16x32(vf, pl[st], o[dt]);
            }
    }
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (!row_ok) return;
    const float inv = 1.0f / l;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
        store4(out + frag_off(row, head * D + dt * 16 + 4 * grp, W), o[dt][0] * inv, o[dt][1] * inv,
               o[dt][2] * inv, o[dt][3] * inv);
}

// The last row of each request's chunk (row b * n + n - 1 of x, fragment order [.][H]) into row b
// of the output head's operand (fragment order [B][H]); one thread per 8 values.
__global__ __launch_bounds__(256) void prefill_last_rows_kernel(const bf16 *__restrict__ u, int n, int B, int H,
                                                                bf16 *__restrict__ out) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (int64_t)B * (H / 8)) return;
    const int b = (int)(t / (H / 8)), c = (int)(t % (H / 8)) * 8;
    *(bf16x8 *)(out + frag_off(b, c, H)) = *(const bf16x8 *)(u + frag_off((int64_t)b * n + n - 1, c, H));
}

// The output head's per-group maxima [groups][B] of each request's last row merged (largest value,
// then lowest index) into its next token; -1 for a failed request. Then the committed context of
// every request that did not fail advances by the chunk. One workgroup per request: a strided
// scan over the groups, then a tree merge in LDS (the order-free rule gives the same winner).
__global__ __launch_bounds__(256) void prefill_finish_kernel(const float *__restrict__ amv, const int *__restrict__ ami,
                                                             int groups, int B, int n, int last,
                                                             const int32_t *__restrict__ status,
                                                             int32_t *__restrict__ failed,
                                                             int32_t *__restrict__ ctx_len,
                                                             int32_t *__restrict__ next_token) {
    __shared__ float sv[256];
    __shared__ int si[256];
    const int b = blockIdx.x, t = threadIdx.x;
    const bool bad = failed[b] != 0 || status[b] != 0;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    if (last)
        for (int gi = t; gi < groups; gi += 256) {
            const float v = amv[(int64_t)gi * B + b];
            const int ix = ami[(int64_t)gi * B + b];
            if (better(v, ix, bv, bi)) { bv = v; bi = ix; }
        }
    sv[t] = bv;
    si[t] = bi;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (t < w && better(sv[t + w], si[t + w], sv[t], si[t])) {
            sv[t] = sv[t + w];
            si[t] = si[t + w];
        }
        __syncthreads();
    }
    if (t != 0) return;
    if (bad) failed[b] = 1;
    else ctx_len[b] += n;
    if (last) next_token[b] = bad ? -1 : si[0];
}

hipError_t prefill_prep(const int32_t *tokens, int n, int B, int vocab, const int32_t *ctx_len,
                        const int32_t *block_table, int max_pages, int n_pages, const int32_t *failed,
                        int32_t *pos, int32_t *status, hipStream_t st) {
    hipLaunchKernelGGL(prefill_prep_kernel, dim3((unsigned)B), dim3(256), 0, st, tokens, n, vocab, ctx_len,
                       block_table, max_pages, n_pages, failed, pos, status);
    return hipGetLastError();
}

hipError_t prefill_attention(const bf16 *q, const bf16 *k_pool, const bf16 *v_pool, const int32_t *block_table,
                             int max_pages, const int32_t *ctx_len, const int32_t *status, int B, int n, int nq,
                             int nkv, int D, bf16 *out, hipStream_t st) {
    const int group = nq / nkv;
    if (group < 1 || group > 8 || (D != 64 && D != 128)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((n + kPQB - 1) / kPQB), (unsigned)nkv, (unsigned)B);
    const float scale_log2 = kLog2e / sqrtf((float)D);
#define SV_PA(DD, G)                                                                                           \
    hipLaunchKernelGGL((prefill_attn_kernel<DD, G>), grid, dim3(128 * G), 0, st, q, k_pool, v_pool, block_table, \
                       max_pages, ctx_len, status, n, nq, nkv, scale_log2, out)
#define SV_PA_G(DD)                   \
    switch (group) {                  \
        case 1: SV_PA(DD, 1); break;  \
        case 2: SV_PA(DD, 2); break;  \
        case 3: SV_PA(DD, 3); break;  \
        case 4: SV_PA(DD, 4); break;  \
        case 5: SV_PA(DD, 5); break;  \
        case 6: SV_PA(DD, 6); break;  \
        case 7: SV_PA(DD, 7); break;  \
        default: SV_PA(DD, 8); break; \
    }
    if (D == 128) {
        SV_PA_G(128)
    } else {
        SV_PA_G(64)
    }
#undef SV_PA_G
#undef SV_PA
    return hipGetLastError();
}

hipError_t prefill_last_rows(const bf16 *u, int n, int B, int H, bf16 *out, hipStream_t st) {
    const int64_t total = (int64_t)B * (H / 8);
    hipLaunchKernelGGL(prefill_last_rows_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, u, n, B,
                       H, out);
    return hipGetLastError();
}

hipError_t prefill_finish(const float *amv, const int *ami, int groups, int B, int n, bool last,
                          const int32_t *status, int32_t *failed, int32_t *ctx_len, int32_t *next_token,
                          hipStream_t st) {
    hipLaunchKernelGGL(prefill_finish_kernel, dim3((unsigned)B), dim3(256), 0, st, amv, ami, groups, B, n,
                       last ? 1 : 0, status, failed, ctx_len, next_token);
    return hipGetLastError();
}

hipError_t prefill_init(int32_t *failed, int B, hipStream_t st) {
    hipLaunchKernelGGL(prefill_init_kernel, dim3((B + 255) / 256), dim3(256), 0, st, failed, B);
    return hipGetLastError();
}

hipError_t prefill_gather(const int32_t *prompt, int p, int c0, int n, int B, int32_t *out, hipStream_t st) {
    hipLaunchKernelGGL(prefill_gather_kernel, dim3((B * n + 255) / 256), dim3(256), 0, st, prompt, p, c0, n,
                       B, out);
    return hipGetLastError();
}

}  // namespace sv
