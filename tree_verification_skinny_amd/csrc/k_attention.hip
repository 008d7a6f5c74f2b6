// k_attention.hip — tree-masked grouped-query attention of the draft nodes over the paged KV
// cache, on gfx950 MFMA with the KV chunk staged in LDS.
//
// Each draft token sees the committed context plus the nodes on its own root path: tree tokens
// are conditioned on the path that leads to them [JetSpec article, seventnews.com — "Technical
// architecture"]. The path is a 64-bit ancestor mask per node (bit j set = node j is on the
// path), so the mask test in the inner loop is one shift and one AND.
//
// Work split (split-KV): one workgroup per (request, kv head, chunk of 128 key positions). The
// 4 waves stage the chunk's keys [128][D] and transposed values [D][128] from the cache pages
// into LDS with 128-bit loads, then each wave takes 16-column query tiles: the columns are the
// (q head of this kv group, draft node) pairs, so one K/V tile in LDS serves every q head of the
// group. Per 32 keys and tile:
//   S^T = K . Q^T   (A = keys from LDS, B = Q^T held in registers for the whole chunk)
//   online softmax per query column, in the log2 domain
//   O^T += V^T . P^T (A = transposed values from LDS, B = the probabilities this lane already
//                     holds, as a bf16 high part plus a bf16 low part)
// The S^T tiles take their 16 key rows in the order 8*(r/4) + 4*tile + r%4, which leaves each
// lane holding 8 consecutive keys: exactly the P^T fragment the V^T MFMA wants, so no lane
// exchange is needed between the two products. Chunk partials (unnormalised O, running max,
// running sum) are merged by attn_combine.
#include "kernels.hpp"

namespace sv {

template <int D>
__global__ __launch_bounds__(256) void attn_partial_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k_pool, const bf16 *__restrict__ v_pool,
    const int32_t *__restrict__ block_table, int max_pages, const int32_t *__restrict__ ctx_len,
    const uint64_t *__restrict__ anc, const int32_t *__restrict__ status, int K, int nq, int nkv,
    int n_chunks, float scale_log2, float *__restrict__ part_o, float2 *__restrict__ part_ml) {
    constexpr int CH = kAttnChunk;
    constexpr int KP = D + 8;    // padded LDS row of K (bf16)
    constexpr int VP = CH + 8;   // padded LDS row of V^T (bf16)
    __shared__ __attribute__((aligned(16))) bf16 Ks[CH * KP];
    __shared__ __attribute__((aligned(16))) bf16 Vt[D * VP];

    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    constexpr int NP = CH / 16;
    // Page ids of this chunk and the request's status and context are read together: the index
    // is clamped to the request's table row (max_pages entries), so these reads are in bounds
    // whatever the context turns out to be; entries past the context are masked below.
    const int32_t *bt = block_table + (int64_t)b * max_pages;
    int pages[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) pages[p] = bt[min((c * CH >> 4) + p, max_pages - 1)];
    const int st_b = status[b];
    const int ctx = ctx_len[b];
    if (st_b != 0) return;
    const int T = ctx + K;
    const int kb = c * CH;
    if (kb >= T) return;
    const int nvalid = min(CH, T - kb);
    const int npages = (nvalid + 15) >> 4;
    const int group = nq / nkv;
    const int R = group * K;
    const int QT = (R + 15) >> 4;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
    // the first query tile's fragments are fetched before the chunk, so the two overlap
    bf16x8 qf_next[D / 32];
    auto q_ptr = [&](int t, bool &col_ok, int &tok, int &hh) {
        const int rho = 16 * t + r16;
        col_ok = rho < R;
        hh = col_ok ? rho / K : 0;
        tok = col_ok ? rho % K : 0;
        return q + ((int64_t)(b * K + tok) * nq + g * group + hh) * D;
    };
    if (wave < QT) {
        bool ok_;
        int tok_, hh_;
        const bf16 *qrow = q_ptr(wave, ok_, tok_, hh_);
#pragma unroll
        for (int ds = 0; ds < D / 32; ++ds) qf_next[ds] = *(const bf16x8 *)(qrow + ds * 32 + grp * 8);
    }

    // ---- stage the chunk: K rows as stored, V already transposed in the page ---------------
    // Every thread issues all of its page loads before the first LDS store, so the chunk's
    // 2 x 8 x 16 B per thread are in flight together.
    {
        const int e = threadIdx.x * 8;           // element offset inside a 16 x D page
        const bool has = e < 16 * D;
#pragma unroll
        for (int p = 0; p < NP; ++p)
            if (!(has && p < npages)) pages[p] = -1;
        bf16x8 kr[NP], vr[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            if (pages[p] >= 0) {
                kr[p] = *(const bf16x8 *)(k_pool + ((int64_t)pages[p] * nkv + g) * 16 * D + e);
                vr[p] = *(const bf16x8 *)(v_pool + ((int64_t)pages[p] * nkv + g) * D * 16 + e);
            } else {
                kr[p] = bf16x8{};
                vr[p] = bf16x8{};
            }
        }
        if (has) {
            const int row = e / D, col = e % D;
            const int d = e >> 4, slot = e & 15;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                *(bf16x8 *)&Ks[(p * 16 + row) * KP + col] = kr[p];
                bf16x8 vv = vr[p];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (p * 16 + slot + j >= nvalid) vv[j] = (bf16)0.0f;   // never multiply stale data
                *(bf16x8 *)&Vt[d * VP + p * 16 + slot] = vv;
            }
        }
    }
    __syncthreads();

    const int nsteps = (nvalid + 31) >> 5;
    const int kr0 = 8 * (r16 >> 2) + (r16 & 3);   // S^T tile 0 key row of this lane (tile 1: +4)

    for (int t = wave; t < QT; t += 4) {
        const int rho = 16 * t + r16;             // query column of this lane
        bool col_ok;
        int tok, hh;
        q_ptr(t, col_ok, tok, hh);
        const uint64_t am = anc[b * K + tok];
        bf16x8 qf[D / 32];
#pragma unroll
        for (int ds = 0; ds < D / 32; ++ds) qf[ds] = qf_next[ds];
        if (t + 4 < QT) {                         // next tile's fragments, one tile ahead
            bool o2;
            int t2, h2;
            const bf16 *qn = q_ptr(t + 4, o2, t2, h2);
#pragma unroll
            for (int ds = 0; ds < D / 32; ++ds) qf_next[ds] = *(const bf16x8 *)(qn + ds * 32 + grp * 8);
        }
        floatx4 o[D / 16];
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
        float m_run = -INFINITY, l_run = 0.f;

        for (int st = 0; st < nsteps; ++st) {
            floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
            const bf16 *k0 = &Ks[(st * 32 + kr0) * KP + grp * 8];
            const bf16 *k1 = k0 + 4 * KP;
#pragma unroll
            for (int ds = 0; ds < D / 32; ++ds) {
                s0 = mfma16x16x32(*(const bf16x8 *)(k0 + ds * 32), qf[ds], s0);
                s1 = mfma16x16x32(*(const bf16x8 *)(k1 + ds * 32), qf[ds], s1);
            }
            float sv[8];
            float mloc = -INFINITY;
            // a 32-key step wholly inside the committed context needs no mask
            const bool plain = col_ok && st * 32 + 32 <= nvalid && kb + st * 32 + 32 <= ctx;
            if (plain) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sv[e] = (e < 4 ? s0[e] : s1[e - 4]) * scale_log2;
                    mloc = fmaxf(mloc, sv[e]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float raw = e < 4 ? s0[e] : s1[e - 4];
                    const int kl = st * 32 + 8 * grp + e;
                    const int ka = kb + kl;
                    const bool vis = col_ok && kl < nvalid && (ka < ctx || ((am >> (ka - ctx)) & 1ull));
                    sv[e] = vis ? raw * scale_log2 : -INFINITY;
                    mloc = fmaxf(mloc, sv[e]);
                }
            }
            mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
            mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
            const float m_new = fmaxf(m_run, mloc);
            const bool none = (m_new == -INFINITY);
            const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
            // p = p_hi + p_lo, both bf16: the two products carry ~16 bits of p, so the weighted
            // sum of values is as precise as the fp32 probabilities it stands for.
            bf16x8 ph, pl;
            float psum = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pv = none ? 0.f : __builtin_amdgcn_exp2f(sv[e] - m_new);
                const bf16 hi = to_bf(pv);
                ph[e] = hi;
                pl[e] = to_bf(pv - to_f(hi));
                psum += pv;
            }
            l_run = l_run * alpha + psum;
            m_run = m_new;
            // the accumulators need rescaling only when some column's running maximum moved
            if (__any(alpha != 1.f)) {
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt) o[dt] *= alpha;
            }
            const bf16 *vrow = &Vt[r16 * VP + st * 32 + grp * 8];
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                const bf16x8 vf = *(const bf16x8 *)(vrow + dt * 16 * VP);
                o[dt] = mfma16x16x32(vf, ph, o[dt]);
                o[dt] = mfma16x16x32(vf, pl, o[dt]);
            }
        }
        l_run += __shfl_xor(l_run, 16, 64);
        l_run += __shfl_xor(l_run, 32, 64);
        if (col_ok) {
            const int64_t base = (((int64_t)b * nkv + g) * n_chunks + c) * R + rho;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt)
                *(floatx4 *)(part_o + base * D + dt * 16 + 4 * grp) = o[dt];
            if (grp == 0) part_ml[base] = make_float2(m_run, l_run);
        }
    }
}

// Merge the chunk partials of one (node, q head): o = sum_c 2^(m_c - m*) O_c / sum_c 2^(m_c - m*) l_c.
// 256 threads = (D/4) column quads x CG chunk groups; each thread merges its chunks c = cg,
// cg + CG, ... with every load issued before the arithmetic, then the CG states are merged in
// LDS in chunk-group order.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(
    const float *__restrict__ part_o, const float2 *__restrict__ part_ml,
    const int32_t *__restrict__ ctx_len, const int32_t *__restrict__ status, int K, int nq,
    int nkv, int n_chunks, bf16 *__restrict__ out) {
    constexpr int TQ = D / 4;            // threads per column quad set
    constexpr int CG = 256 / TQ;         // chunk groups: 8 (D=128) or 16 (D=64)
    constexpr int PER = 8;               // chunks per thread held in flight
    __shared__ float s_m[CG][TQ], s_l[CG][TQ];
    __shared__ floatx4 s_o[CG][TQ];
    const int row = blockIdx.x, h = blockIdx.y;
    const int d4 = (threadIdx.x % TQ) * 4, cg = threadIdx.x / TQ;
    const int b = row / K, tok = row % K;
    bf16 *dst = out + frag_off(row, h * D + d4, nq * D);   // fragment order: the O operand
    if (status[b] != 0) {
        if (cg == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[j] = (bf16)0.0f;
        }
        return;
    }
    const int group = nq / nkv, g = h / group, hh = h % group;
    const int R = group * K, rho = hh * K + tok;
    const int nc = (ctx_len[b] + K + kAttnChunk - 1) / kAttnChunk;
    const int64_t base = ((int64_t)b * nkv + g) * n_chunks * R + rho;
    float m = -INFINITY, l = 0.f;
    floatx4 o = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = cg; c0 < nc; c0 += CG * PER) {
        float2 ml[PER];
        floatx4 oc[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = c0 + i * CG;
            if (c < nc) {
                ml[i] = part_ml[base + (int64_t)c * R];
                oc[i] = *(const floatx4 *)(part_o + (base + (int64_t)c * R) * D + d4);
            } else {
                ml[i] = make_float2(-INFINITY, 0.f);
                oc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
            }
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (ml[i].x == -INFINITY) continue;
            const float mn = fmaxf(m, ml[i].x);
            const float a = exp2f(m - mn), w = exp2f(ml[i].x - mn);
            l = l * a + ml[i].y * w;
            o = o * a + oc[i] * w;
            m = mn;
        }
    }
    s_m[cg][threadIdx.x % TQ] = m;
    s_l[cg][threadIdx.x % TQ] = l;
    s_o[cg][threadIdx.x % TQ] = o;
    __syncthreads();
    if (cg != 0) return;
    for (int k = 1; k < CG; ++k) {
        const float mk = s_m[k][threadIdx.x], lk = s_l[k][threadIdx.x];
        if (mk == -INFINITY) continue;
        const floatx4 ok = s_o[k][threadIdx.x];
        const float mn = fmaxf(m, mk);
        const float a = exp2f(m - mn), w = exp2f(mk - mn);
        l = l * a + lk * w;
        o = o * a + ok * w;
        m = mn;
    }
    store4(dst, o[0] / l, o[1] / l, o[2] / l, o[3] / l);
}

hipError_t attention(const AttnArgs &a, hipStream_t st) {
    const float scale_log2 = kLog2e / sqrtf((float)a.D);
    dim3 grid(a.n_chunks, a.nkv, a.B);
    if (a.D == 128) {
        hipLaunchKernelGGL(attn_partial_kernel<128>, grid, dim3(256), 0, st, a.q, a.k_pool, a.v_pool,
                           a.block_table, a.max_pages, a.ctx_len, a.anc, a.status, a.K, a.nq, a.nkv,
                           a.n_chunks, scale_log2, a.part_o, a.part_ml);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(attn_combine_kernel<128>, dim3(a.B * a.K, a.nq), dim3(256), 0, st,
                           a.part_o, a.part_ml, a.ctx_len, a.status, a.K, a.nq, a.nkv, a.n_chunks, a.out);
    } else {
        hipLaunchKernelGGL(attn_partial_kernel<64>, grid, dim3(256), 0, st, a.q, a.k_pool, a.v_pool,
                           a.block_table, a.max_pages, a.ctx_len, a.anc, a.status, a.K, a.nq, a.nkv,
                           a.n_chunks, scale_log2, a.part_o, a.part_ml);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(attn_combine_kernel<64>, dim3(a.B * a.K, a.nq), dim3(256), 0, st,
                           a.part_o, a.part_ml, a.ctx_len, a.status, a.K, a.nq, a.nkv, a.n_chunks, a.out);
    }
    return hipGetLastError();
}

}  // namespace sv
