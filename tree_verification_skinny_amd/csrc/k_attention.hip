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

// HPW kv heads per workgroup (NW waves each) share the chunk's page reads and halve the number
// of workgroups, so that a typical grid is resident at once.
template <int D, int NW, int HPW>
__global__ __launch_bounds__(64 * NW * HPW) void attn_partial_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k_pool, const bf16 *__restrict__ v_pool,
    const int32_t *__restrict__ block_table, int max_pages, const int32_t *__restrict__ ctx_len,
    const uint64_t *__restrict__ anc, const int32_t *__restrict__ status, int K, int nq, int nkv,
    int n_chunks, float scale_log2, float *__restrict__ part_o, float2 *__restrict__ part_ml) {
    constexpr int CH = kAttnChunk;
    constexpr int NS = CH / 32;  // 32-key steps per chunk
    constexpr int KP = D + 8;    // padded LDS row of K (bf16)
    constexpr int VP = CH + 8;   // padded LDS row of V^T (bf16)
    constexpr int STAGERS = 16 * D / 8;   // threads that stage one head's 16-position page
    static_assert(STAGERS <= 64 * NW, "staging needs one thread per 16 bytes of a page");
    __shared__ __attribute__((aligned(16))) bf16 Ks_all[HPW * CH * KP];
    __shared__ __attribute__((aligned(16))) bf16 Vt_all[HPW * D * VP];

    const int c = blockIdx.x, b = blockIdx.z;
    const int wave_all = threadIdx.x >> 6;
    const int hl = wave_all / NW;                 // this wave's head within the workgroup
    const int g = blockIdx.y * HPW + hl;          // its kv head
    const bf16 *Ks = Ks_all + hl * CH * KP;
    const bf16 *Vt = Vt_all + hl * D * VP;
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

    const int lane = threadIdx.x & 63, wave = wave_all % NW;
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
    uint64_t am_next = 0;
    if (wave < QT) {
        bool ok_;
        int tok_, hh_;
        const bf16 *qrow = q_ptr(wave, ok_, tok_, hh_);
#pragma unroll
        for (int ds = 0; ds < D / 32; ++ds) qf_next[ds] = *(const bf16x8 *)(qrow + ds * 32 + grp * 8);
        am_next = anc[b * K + tok_];
    }

    // ---- stage the chunk: K rows as stored, V already transposed in the page ---------------
    // Every staging thread issues all of its page loads before the first LDS store, so the
    // chunk's 2 x 8 x 16 B per thread are in flight together.
    {
        const int hs = threadIdx.x / STAGERS;          // head this thread stages
        const int gs = blockIdx.y * HPW + hs;
        const int e = (threadIdx.x % STAGERS) * 8;     // element offset inside a 16 x D page
        const bool has = hs < HPW;
#pragma unroll
        for (int p = 0; p < NP; ++p)
            if (!(has && p < npages)) pages[p] = -1;
        bf16x8 kr[NP], vr[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            if (pages[p] >= 0) {
                kr[p] = *(const bf16x8 *)(k_pool + ((int64_t)pages[p] * nkv + gs) * 16 * D + e);
                vr[p] = *(const bf16x8 *)(v_pool + ((int64_t)pages[p] * nkv + gs) * D * 16 + e);
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
                *(bf16x8 *)&Ks_all[hs * CH * KP + (p * 16 + row) * KP + col] = kr[p];
                bf16x8 vv = vr[p];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (p * 16 + slot + j >= nvalid) vv[j] = (bf16)0.0f;   // never multiply stale data
                *(bf16x8 *)&Vt_all[hs * D * VP + d * VP + p * 16 + slot] = vv;
            }
        }
    }
    __syncthreads();

    const int kr0 = 8 * (r16 >> 2) + (r16 & 3);   // S^T tile 0 key row of this lane (tile 1: +4)
    // the whole chunk lies inside the committed context: no key needs the mask
    const bool chunk_plain = nvalid == CH && kb + CH <= ctx;

    for (int t = wave; t < QT; t += NW) {
        const int rho = 16 * t + r16;             // query column of this lane
        bool col_ok;
        int tok, hh;
        q_ptr(t, col_ok, tok, hh);
        const uint64_t am = am_next;
        bf16x8 qf[D / 32];
#pragma unroll
        for (int ds = 0; ds < D / 32; ++ds) qf[ds] = qf_next[ds];

        // S^T for the whole chunk: step st, half h holds key rows st*32 + kr0 + 4h; with the row
        // order above, this lane ends up with keys st*32 + 8*grp + e, e = 0..7. The staged chunk
        // is zero past its valid keys, so all NS steps run (masked below). Key fragments are
        // read from LDS one step ahead of the products that use them.
        floatx4 s[NS][2];
        {
            // stage i = (step i / 2, half i % 2): D/32 key fragments, D/32 products
            constexpr int NST = 2 * NS, FK = D / 32;
            bf16x8 kf0[FK], kf1[FK];
            auto kload = [&](bf16x8 (&kf)[FK], int i) {
#pragma unroll
                for (int ds = 0; ds < FK; ++ds)
                    kf[ds] = *(const bf16x8 *)&Ks[((i >> 1) * 32 + kr0 + 4 * (i & 1)) * KP + grp * 8 + ds * 32];
            };
            kload(kf0, 0);
#pragma unroll
            for (int i = 0; i < NST; ++i) {
                auto &cur = (i & 1) ? kf1 : kf0;
                auto &nxt = (i & 1) ? kf0 : kf1;
                if (i + 1 < NST) {
                    kload(nxt, i + 1);
                    __builtin_amdgcn_sched_group_barrier(0x100, FK, 0);   // LDS reads
                }
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ds = 0; ds < FK; ++ds) acc = mfma16x16x32(cur[ds], qf[ds], acc);
                s[i >> 1][i & 1] = acc;
                __builtin_amdgcn_sched_group_barrier(0x008, FK, 0);       // MFMAs
            }
        }
        // one softmax over the chunk, in the log2 domain: m = max, p = 2^(s - m), l = sum p
        float sv[NS][8];
        float mloc = -INFINITY;
        if (chunk_plain) {
            // every key is committed context, visible to every node (columns past R are
            // computed on a stand-in query and never stored)
#pragma unroll
            for (int st = 0; st < NS; ++st)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sv[st][e] = (e < 4 ? s[st][0][e] : s[st][1][e - 4]) * scale_log2;
                    mloc = fmaxf(mloc, sv[st][e]);
                }
        } else {
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                // visibility of this lane's 8 keys ka = k0 .. k0 + 7 as a bit mask: committed
                // positions (< ctx) always, draft positions ctx + j when node j is an ancestor
                const int k0 = kb + st * 32 + 8 * grp;
                const int n_ctx = min(max(ctx - k0, 0), 8);
                const int j0 = max(k0 + n_ctx - ctx, 0);     // first draft index among them
                const unsigned anc8 = j0 < 64 ? (unsigned)(am >> j0) & 0xffu : 0u;
                const int n_in = min(max(kb + nvalid - k0, 0), 8);   // keys inside the chunk
                unsigned vis = (((1u << n_ctx) - 1u) | (anc8 << n_ctx)) & ((1u << n_in) - 1u);
                if (!col_ok) vis = 0u;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float raw = (e < 4 ? s[st][0][e] : s[st][1][e - 4]) * scale_log2;
                    sv[st][e] = ((vis >> e) & 1u) ? raw : -INFINITY;
                    mloc = fmaxf(mloc, sv[st][e]);
                }
            }
        }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
        const bool none = (mloc == -INFINITY);
        // p = p_hi + p_lo, both bf16: the two products carry ~16 bits of p, so the weighted sum
        // of values is as precise as the fp32 probabilities it stands for.
        bf16x8 ph[NS], pl[NS];
        float psum = 0.f;
#pragma unroll
        for (int st = 0; st < NS; ++st) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pv = none ? 0.f : __builtin_amdgcn_exp2f(sv[st][e] - mloc);
                const bf16 hi = to_bf(pv);
                ph[st][e] = hi;
                pl[st][e] = to_bf(pv - to_f(hi));
                psum += pv;
            }
        }
        psum += __shfl_xor(psum, 16, 64);
        psum += __shfl_xor(psum, 32, 64);

        // O^T = V^T . P^T over the chunk, value fragments read one step ahead
        floatx4 o[D / 16];
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
        {
            // stage i = (step i / 2, value rows half i % 2): FV fragments, 2 FV products
            constexpr int NST = 2 * NS, FV = D / 32;
            bf16x8 vf0[FV], vf1[FV];
            auto vload = [&](bf16x8 (&vf)[FV], int i) {
#pragma unroll
                for (int j = 0; j < FV; ++j)
                    vf[j] = *(const bf16x8 *)&Vt[(r16 + ((i & 1) * FV + j) * 16) * VP + (i >> 1) * 32 + grp * 8];
            };
            vload(vf0, 0);
#pragma unroll
            for (int i = 0; i < NST; ++i) {
                auto &cur = (i & 1) ? vf1 : vf0;
                auto &nxt = (i & 1) ? vf0 : vf1;
                if (i + 1 < NST) {
                    vload(nxt, i + 1);
                    __builtin_amdgcn_sched_group_barrier(0x100, FV, 0);        // LDS reads
                }
#pragma unroll
                for (int j = 0; j < FV; ++j) {
                    const int dt = (i & 1) * FV + j;
                    o[dt] = mfma16x16x32(cur[j], ph[i >> 1], o[dt]);
                    o[dt] = mfma16x16x32(cur[j], pl[i >> 1], o[dt]);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 2 * FV, 0);    // MFMAs
            }
        }
        if (t + NW < QT) {   // the next tile's operands, fetched while this tile's results drain
            bool o2;
            int t2, h2;
            const bf16 *qn = q_ptr(t + NW, o2, t2, h2);
#pragma unroll
            for (int ds = 0; ds < D / 32; ++ds) qf_next[ds] = *(const bf16x8 *)(qn + ds * 32 + grp * 8);
            am_next = anc[b * K + t2];
        }
        if (col_ok) {
            const int64_t base = (((int64_t)b * nkv + g) * n_chunks + c) * R + rho;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt)
                *(floatx4 *)(part_o + base * D + dt * 16 + 4 * grp) = o[dt];
            if (grp == 0) part_ml[base] = make_float2(mloc, psum);
        }
    }
}

// Large grids (a batch, or a draft tree with hundreds of query rows): one kv head per workgroup
// (two workgroups share a compute unit, so one stages while the other multiplies), a range of CPR
// chunks walked in order with the online-softmax rescale so that a range leaves one partial
// instead of CPR of them, and tile groups (grid z = request x tile group) so that no wave holds
// more than one 16-column query tile. The page ids of the next chunk are fetched while the
// current chunk is multiplied.
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void attn_range_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k_pool, const bf16 *__restrict__ v_pool,
    const int32_t *__restrict__ block_table, int max_pages, const int32_t *__restrict__ ctx_len,
    const uint64_t *__restrict__ anc, const int32_t *__restrict__ status, int K, int nq, int nkv,
    int n_ranges, int cpr, int n_tg, float scale_log2, float *__restrict__ part_o,
    float2 *__restrict__ part_ml) {
    constexpr int CH = kAttnChunk;
    constexpr int NS = CH / 32;
    constexpr int KP = D + 8;
    constexpr int VP = CH + 8;
    constexpr int STAGERS = 16 * D / 8;
    constexpr int NP = CH / 16;
    static_assert(STAGERS <= 64 * NW, "staging needs one thread per 16 bytes of a page");
    __shared__ __attribute__((aligned(16))) bf16 Ks[CH * KP];
    __shared__ __attribute__((aligned(16))) bf16 Vt[D * VP];

    const int rg = blockIdx.x, g = blockIdx.y;
    const int b = blockIdx.z / n_tg, tg = blockIdx.z % n_tg;
    const int st_b = status[b];
    const int ctx = ctx_len[b];
    if (st_b != 0) return;
    const int T = ctx + K;
    const int nc = (T + CH - 1) / CH;
    const int c_begin = rg * cpr;
    if (c_begin >= nc) return;
    const int c_end = min(c_begin + cpr, nc);
    const int group = nq / nkv;
    const int R = group * K;
    const int QT = (R + 15) >> 4;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
    const int t = tg * NW + wave;
    const bool has_tile = t < QT;
    const int rho = 16 * t + r16;
    const bool col_ok = has_tile && rho < R;
    const int hh = col_ok ? rho / K : 0;
    const int tok = col_ok ? rho % K : 0;
    bf16x8 qf[D / 32];
    uint64_t am = 0;
    if (has_tile) {
        const bf16 *qrow = q + ((int64_t)(b * K + tok) * nq + g * group + hh) * D;
#pragma unroll
        for (int ds = 0; ds < D / 32; ++ds) qf[ds] = *(const bf16x8 *)(qrow + ds * 32 + grp * 8);
        am = anc[b * K + tok];
    }
    const int kr0 = 8 * (r16 >> 2) + (r16 & 3);
    const int32_t *bt = block_table + (int64_t)b * max_pages;
    const bool stager = threadIdx.x < STAGERS;
    const int e = (threadIdx.x % STAGERS) * 8;
    const int srow = e / D, scol = e % D, sd = e >> 4, sslot = e & 15;
    auto page_ids = [&](int c, int (&pg)[NP]) {
        const int np = (min(CH, T - c * CH) + 15) >> 4;
#pragma unroll
        for (int p = 0; p < NP; ++p) pg[p] = (stager && p < np) ? bt[(c * CH >> 4) + p] : -1;
    };
    int pg[NP];
    page_ids(c_begin, pg);

    float m_run = -INFINITY, l_run = 0.f;
    floatx4 o[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};

    for (int c = c_begin; c < c_end; ++c) {
        const int kb = c * CH;
        const int nvalid = min(CH, T - kb);
        {
            bf16x8 kr[NP], vr[NP];
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                if (pg[p] >= 0) {
                    kr[p] = *(const bf16x8 *)(k_pool + ((int64_t)pg[p] * nkv + g) * 16 * D + e);
                    vr[p] = *(const bf16x8 *)(v_pool + ((int64_t)pg[p] * nkv + g) * D * 16 + e);
                } else {
                    kr[p] = bf16x8{};
                    vr[p] = bf16x8{};
                }
            }
            if (c + 1 < c_end) page_ids(c + 1, pg);   // next chunk's pages, in flight meanwhile
            if (c > c_begin) __syncthreads();          // the previous chunk is consumed
            if (stager) {
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    *(bf16x8 *)&Ks[(p * 16 + srow) * KP + scol] = kr[p];
                    bf16x8 vv = vr[p];
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        if (p * 16 + sslot + j >= nvalid) vv[j] = (bf16)0.0f;   // never multiply stale data
                    *(bf16x8 *)&Vt[sd * VP + p * 16 + sslot] = vv;
                }
            }
        }
        __syncthreads();
        if (!has_tile) continue;
        const bool chunk_plain = nvalid == CH && kb + CH <= ctx;

        floatx4 s[NS][2];
        {
            constexpr int NST = 2 * NS, FK = D / 32;
            bf16x8 kf0[FK], kf1[FK];
            auto kload = [&](bf16x8 (&kf)[FK], int i) {
#pragma unroll
                for (int ds = 0; ds < FK; ++ds)
                    kf[ds] = *(const bf16x8 *)&Ks[((i >> 1) * 32 + kr0 + 4 * (i & 1)) * KP + grp * 8 + ds * 32];
            };
            kload(kf0, 0);
#pragma unroll
            for (int i = 0; i < NST; ++i) {
                auto &cur = (i & 1) ? kf1 : kf0;
                auto &nxt = (i & 1) ? kf0 : kf1;
                if (i + 1 < NST) {
                    kload(nxt, i + 1);
                    __builtin_amdgcn_sched_group_barrier(0x100, FK, 0);
                }
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ds = 0; ds < FK; ++ds) acc = mfma16x16x32(cur[ds], qf[ds], acc);
                s[i >> 1][i & 1] = acc;
                __builtin_amdgcn_sched_group_barrier(0x008, FK, 0);
            }
        }
        float mloc = -INFINITY;
        if (chunk_plain) {
#pragma unroll
            for (int st = 0; st < NS; ++st)
#pragma unroll
                for (int e2 = 0; e2 < 8; ++e2) {
                    s[st][e2 >> 2][e2 & 3] *= scale_log2;
                    mloc = fmaxf(mloc, s[st][e2 >> 2][e2 & 3]);
                }
        } else {
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                const int k0 = kb + st * 32 + 8 * grp;
                const int n_ctx = min(max(ctx - k0, 0), 8);
                const int j0 = max(k0 + n_ctx - ctx, 0);
                const unsigned anc8 = j0 < 64 ? (unsigned)(am >> j0) & 0xffu : 0u;
                const int n_in = min(max(kb + nvalid - k0, 0), 8);
                unsigned vis = (((1u << n_ctx) - 1u) | (anc8 << n_ctx)) & ((1u << n_in) - 1u);
                if (!col_ok) vis = 0u;
#pragma unroll
                for (int e2 = 0; e2 < 8; ++e2) {
                    const float raw = s[st][e2 >> 2][e2 & 3] * scale_log2;
                    s[st][e2 >> 2][e2 & 3] = ((vis >> e2) & 1u) ? raw : -INFINITY;
                    mloc = fmaxf(mloc, s[st][e2 >> 2][e2 & 3]);
                }
            }
        }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
        const float m_new = fmaxf(m_run, mloc);
        const bool none = (m_new == -INFINITY);
        const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        if (__any(alpha != 1.f)) {
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) o[dt] *= alpha;
        }
        float psum = 0.f;
        {
            constexpr int NST = 2 * NS, FV = D / 32;
            bf16x8 vf0[FV], vf1[FV];
            auto vload = [&](bf16x8 (&vf)[FV], int i) {
#pragma unroll
                for (int j = 0; j < FV; ++j)
                    vf[j] = *(const bf16x8 *)&Vt[(r16 + ((i & 1) * FV + j) * 16) * VP + (i >> 1) * 32 + grp * 8];
            };
            vload(vf0, 0);
            bf16x8 ph, pl;
#pragma unroll
            for (int i = 0; i < NST; ++i) {
                auto &cur = (i & 1) ? vf1 : vf0;
                auto &nxt = (i & 1) ? vf0 : vf1;
                if (i + 1 < NST) {
                    vload(nxt, i + 1);
                    __builtin_amdgcn_sched_group_barrier(0x100, FV, 0);
                }
                if ((i & 1) == 0) {
                    const int st = i >> 1;
#pragma unroll
                    for (int e2 = 0; e2 < 8; ++e2) {
                        const float pv = none ? 0.f : __builtin_amdgcn_exp2f(s[st][e2 >> 2][e2 & 3] - m_new);
                        const bf16 hi = to_bf(pv);
                        ph[e2] = hi;
                        pl[e2] = to_bf(pv - to_f(hi));
                        psum += pv;
                    }
                }
#pragma unroll
                for (int j = 0; j < FV; ++j) {
                    const int dt = (i & 1) * FV + j;
                    o[dt] = mfma16x16x32(cur[j], ph, o[dt]);
                    o[dt] = mfma16x16x32(cur[j], pl, o[dt]);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 2 * FV, 0);
            }
        }
        psum += __shfl_xor(psum, 16, 64);
        psum += __shfl_xor(psum, 32, 64);
        l_run = l_run * alpha + psum;
        m_run = m_new;
    }
    if (col_ok) {
        const int64_t base = (((int64_t)b * nkv + g) * n_ranges + rg) * R + rho;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
            *(floatx4 *)(part_o + base * D + dt * 16 + 4 * grp) = o[dt];
        if (grp == 0) part_ml[base] = make_float2(m_run, l_run);
    }
}

// Merge the partials of one (node, q head): o = sum_c 2^(m_c - m*) O_c / sum_c 2^(m_c - m*) l_c
// over the partials c (one per chunk, or per range of cpr chunks). 256 threads = (D/4) column
// quads x CG groups; each thread merges partials c = cg, cg + CG, ... with every load issued
// before the arithmetic, then the CG states are merged in LDS in group order.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(
    const float *__restrict__ part_o, const float2 *__restrict__ part_ml,
    const int32_t *__restrict__ ctx_len, const int32_t *__restrict__ status, int K, int nq,
    int nkv, int n_chunks, int cpr, bf16 *__restrict__ out) {
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
    const int nc = ((ctx_len[b] + K + kAttnChunk - 1) / kAttnChunk + cpr - 1) / cpr;   // partials
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
    // waves per kv head: 5 when that takes fewer query tiles per wave than 4 (one tile each for
    // a group of 5 q heads and a block of 16), else 4
    const int R = a.nq / a.nkv * a.K;
    const int QT = (R + 15) / 16;
    const int nw = (QT + 4) / 5 < (QT + 3) / 4 ? 5 : 4;
    const int n_tg = (QT + nw - 1) / nw;
    // A small grid (one request, a short draft) runs one chunk per workgroup, two kv heads each,
    // so that it is resident at once. A large one (a batch, or hundreds of query rows) runs
    // ranges of chunks, one kv head per workgroup: chunks per range are chosen so that a
    // range's partial stays below about a quarter of the keys and values it covers, while at
    // least ~512 workgroups remain.
    const int64_t wgs1 = (int64_t)a.n_chunks * a.nkv * a.B * n_tg;
    int cpr = 1, stride = a.n_chunks;
    hipError_t e;
    if (wgs1 <= 512) {
        const int hpw = a.nkv % 2 == 0 ? 2 : 1;
        const dim3 grid_h(a.n_chunks, a.nkv / hpw, a.B);
#define SV_ATTN(DD, NWV, HP)                                                                      \
    hipLaunchKernelGGL((attn_partial_kernel<DD, NWV, HP>), grid_h, dim3(64 * NWV * HP), 0, st,    \
                       a.q, a.k_pool, a.v_pool, a.block_table, a.max_pages, a.ctx_len, a.anc,      \
                       a.status, a.K, a.nq, a.nkv, a.n_chunks, scale_log2, a.part_o, a.part_ml)
#define SV_ATTN_H(DD, NWV)          \
    if (hpw == 2) SV_ATTN(DD, NWV, 2); \
    else SV_ATTN(DD, NWV, 1)
        if (a.D == 128) {
            if (nw == 4) { SV_ATTN_H(128, 4); }
            else { SV_ATTN_H(128, 5); }
        } else {
            if (nw == 4) { SV_ATTN_H(64, 4); }
            else { SV_ATTN_H(64, 5); }
        }
#undef SV_ATTN_H
#undef SV_ATTN
    } else {
        cpr = (R + 31) / 32;
        if (cpr > 8) cpr = 8;
        while (cpr > 1 && (int64_t)((a.n_chunks + cpr - 1) / cpr) * a.nkv * a.B * n_tg < 512) --cpr;
        const int n_ranges = (a.n_chunks + cpr - 1) / cpr;
        stride = n_ranges;
        const dim3 grid_r(n_ranges, a.nkv, a.B * n_tg);
#define SV_RANGE(DD, NWV)                                                                         \
    hipLaunchKernelGGL((attn_range_kernel<DD, NWV>), grid_r, dim3(64 * NWV), 0, st, a.q, a.k_pool, \
                       a.v_pool, a.block_table, a.max_pages, a.ctx_len, a.anc, a.status, a.K,     \
                       a.nq, a.nkv, n_ranges, cpr, n_tg, scale_log2, a.part_o, a.part_ml)
        if (a.D == 128) {
            if (nw == 4) SV_RANGE(128, 4);
            else SV_RANGE(128, 5);
        } else {
            if (nw == 4) SV_RANGE(64, 4);
            else SV_RANGE(64, 5);
        }
#undef SV_RANGE
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.D == 128)
        hipLaunchKernelGGL(attn_combine_kernel<128>, dim3(a.B * a.K, a.nq), dim3(256), 0, st,
                           a.part_o, a.part_ml, a.ctx_len, a.status, a.K, a.nq, a.nkv, stride, cpr, a.out);
    else
        hipLaunchKernelGGL(attn_combine_kernel<64>, dim3(a.B * a.K, a.nq), dim3(256), 0, st,
                           a.part_o, a.part_ml, a.ctx_len, a.status, a.K, a.nq, a.nkv, stride, cpr, a.out);
    return hipGetLastError();
}

}  // namespace sv
