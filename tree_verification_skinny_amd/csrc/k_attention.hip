// k_attention.hip — tree-masked grouped-query attention of the draft nodes over the paged KV
// cache, on gfx950 MFMA with the KV chunk staged in LDS.
//
// Each draft token sees the committed context plus the nodes on its own root path: tree tokens
// are conditioned on the path that leads to them [JetSpec article, seventnews.com — "Technical
// architecture"]. The path is a 64-bit ancestor mask per node (bit j set = node j is on the
// path), so the mask test in the inner loop is one shift and one AND.
//
// Two work splits (split-KV): for one request with few query tiles (a block of 16) one
// workgroup per (request, kv head, chunk of 192 keys), whose waves stage the chunk's keys
// [192][D] and values [D][192] from the cache pages into LDS and take 16-column query tiles
// (attn_partial_kernel); for everything else (a draft tree's many tiles, a batch of requests)
// one workgroup of eight waves per (request, kv head, group of query tiles, range of keys),
// which streams the range through LDS 32 keys at a time for all of the group's tiles
// (attn_group_kernel). The query columns are (q head of this kv group, draft node) pairs, so
// one K/V tile in LDS serves every q head of the group. Per 32 keys and tile:
//   S^T = K . Q^T   (A = keys from LDS, B = Q^T held in registers)
//   softmax per query column, in the log2 domain
//   O^T += V^T . P^T (A = transposed values from LDS, B = the probabilities this lane already
//                     holds, as a bf16 high part plus a bf16 low part)
// The S^T tiles take their 16 key rows in the order 8*(r/4) + 4*tile + r%4, which leaves each
// lane holding 8 consecutive keys: exactly the P^T fragment the V^T MFMA wants, so no lane
// exchange is needed between the two products. Chunk and range partials (unnormalised O,
// softmax reference, running sum) are merged by attn_combine / attn_combine_few.
#include "kernels.hpp"

namespace sv {

// A workgroup takes one chunk of CH keys for HPW kv heads; each head's query tiles are spread
// over NW tile slots of KS waves, the KS waves of a slot splitting the chunk's 32-key steps
// evenly and merging their states in LDS (fixed order). More heads per workgroup share one
// chunk's page reads; more waves per tile shorten each wave's serial chain of products and
// softmax at the same LDS traffic.
template <int D, int NW, int HPW, int CH, int KS>
__global__ __launch_bounds__(64 * NW * HPW * KS) void attn_partial_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k_pool, const bf16 *__restrict__ v_pool,
    const int32_t *__restrict__ block_table, int max_pages, const int32_t *__restrict__ ctx_len,
    const uint64_t *__restrict__ anc, const int32_t *__restrict__ status, int K, int nq, int nkv,
    int n_chunks, float scale_log2, float *__restrict__ part_o, float2 *__restrict__ part_ml) {
    constexpr int NS = CH / 32;  // 32-key steps per chunk
    static_assert(CH % 32 == 0 && NS % KS == 0, "key steps split evenly over a tile's waves");
    constexpr int MS = NS / KS;  // key steps per wave
    constexpr int KP = D + 8;    // padded LDS row of K (bf16)
    constexpr int VP = CH + 8;   // padded LDS row of V^T (bf16)
    constexpr int WPH = NW * KS; // waves per head
    constexpr int STAGERS = 16 * D / 8;   // threads that stage one head's 16-position page
    static_assert(STAGERS <= 64 * WPH, "staging needs one thread per 16 bytes of a page");
    constexpr int MSL = KS > 1 ? HPW * NW * (KS - 1) : 1;   // merge slots
    __shared__ __attribute__((aligned(16))) bf16 Ks_all[HPW * CH * KP];
    __shared__ __attribute__((aligned(16))) bf16 Vt_all[HPW * D * VP];
    __shared__ floatx4 mg_o[MSL * (D / 16) * 64];
    __shared__ float mg_m[MSL * 64], mg_l[MSL * 64];

    const int c = blockIdx.x, b = blockIdx.z;
    const int wave_all = threadIdx.x >> 6;
    const int hl = wave_all / WPH;                // this wave's head within the workgroup
    const int g = blockIdx.y * HPW + hl;          // its kv head
    const int wv = wave_all % WPH;
    const int tw = wv / KS, kp = wv % KS;         // tile slot, key part
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

    const int lane = threadIdx.x & 63;
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
    if (tw < QT) {
        bool ok_;
        int tok_, hh_;
        const bf16 *qrow = q_ptr(tw, ok_, tok_, hh_);
#pragma unroll
        for (int ds = 0; ds < D / 32; ++ds) qf_next[ds] = *(const bf16x8 *)(qrow + ds * 32 + grp * 8);
        am_next = anc[b * K + tok_];
    }

    // ---- stage the chunk: K rows as stored, V already transposed in the page ---------------
    // Every staging thread issues all of its page loads before the first LDS store, so the
    // chunk's 2 x NP x 16 B per thread are in flight together.
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
                kr[p] = stream_load((const bf16x8 *)(k_pool + ((int64_t)pages[p] * nkv + gs) * 16 * D + e));
                vr[p] = stream_load((const bf16x8 *)(v_pool + ((int64_t)pages[p] * nkv + gs) * D * 16 + e));
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
    const int s0 = kp * MS;                       // this wave's first key step
    // the wave's keys all lie inside the committed context: no key needs the mask
    const bool part_plain = kb + (s0 + MS) * 32 <= min(ctx, kb + nvalid);
    const int n_iter = (QT + NW - 1) / NW;        // the same for every wave (merge barriers)

    for (int it = 0; it < n_iter; ++it) {
        const int t = tw + it * NW;
        const bool has = t < QT;
        const int rho = 16 * t + r16;             // query column of this lane
        bool col_ok = false;
        int tok = 0, hh = 0;
        if (has) q_ptr(t, col_ok, tok, hh);
        const uint64_t am = am_next;
        bf16x8 qf[D / 32];
#pragma unroll
        for (int ds = 0; ds < D / 32; ++ds) qf[ds] = qf_next[ds];

        floatx4 o[D / 16];
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
        float mloc = -INFINITY, psum = 0.f;
        if (has) {
            // S^T over the wave's steps: stage i = (step s0 + i / 2, half i % 2) holds key rows
            // step*32 + kr0 + 4 half; with the row order above, this lane ends up with keys
            // step*32 + 8*grp + e, e = 0..7. The staged chunk is zero past its valid keys
            // (masked below). Key fragments are read from LDS one stage ahead of their products.
            floatx4 sc[MS][2];
            {
                constexpr int NST = 2 * MS, FK = D / 32;
                bf16x8 kf0[FK], kf1[FK];
                auto kload = [&](bf16x8 (&kf)[FK], int i) {
#pragma unroll
                    for (int ds = 0; ds < FK; ++ds)
                        kf[ds] = *(const bf16x8 *)&Ks[((s0 + (i >> 1)) * 32 + kr0 + 4 * (i & 1)) * KP + grp * 8 + ds * 32];
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
                    sc[i >> 1][i & 1] = acc;
                    __builtin_amdgcn_sched_group_barrier(0x008, FK, 0);       // MFMAs
                }
            }
            // one softmax over the wave's keys, in the log2 domain: m = max, p = 2^(s - m)
            float sv[MS][8];
            if (part_plain) {
                // committed context only, visible to every node (columns past R are computed
                // on a stand-in query and never stored)
#pragma unroll
                for (int st = 0; st < MS; ++st)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        sv[st][e] = (e < 4 ? sc[st][0][e] : sc[st][1][e - 4]) * scale_log2;
                        mloc = fmaxf(mloc, sv[st][e]);
                    }
            } else {
#pragma unroll
                for (int st = 0; st < MS; ++st) {
                    // visibility of this lane's 8 keys as a bit mask: committed positions
                    // (< ctx) always, draft positions ctx + j when node j is an ancestor
                    const int k0 = kb + (s0 + st) * 32 + 8 * grp;
                    const int n_ctx = min(max(ctx - k0, 0), 8);
                    const int j0 = max(k0 + n_ctx - ctx, 0);     // first draft index among them
                    const unsigned anc8 = j0 < 64 ? (unsigned)(am >> j0) & 0xffu : 0u;
                    const int n_in = min(max(kb + nvalid - k0, 0), 8);   // keys inside the chunk
                    unsigned vis = (((1u << n_ctx) - 1u) | (anc8 << n_ctx)) & ((1u << n_in) - 1u);
                    if (!col_ok) vis = 0u;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float raw = (e < 4 ? sc[st][0][e] : sc[st][1][e - 4]) * scale_log2;
                        sv[st][e] = ((vis >> e) & 1u) ? raw : -INFINITY;
                        mloc = fmaxf(mloc, sv[st][e]);
                    }
                }
            }
            mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
            mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
            const bool none = (mloc == -INFINITY);
            // p = p_hi + p_lo, both bf16: the two products carry ~16 bits of p, so the weighted
            // sum of values is as precise as the fp32 probabilities it stands for.
            bf16x8 ph[MS], pl[MS];
#pragma unroll
            for (int st = 0; st < MS; ++st) {
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

            // O^T = V^T . P^T over the wave's steps, value fragments read one stage ahead
            {
                constexpr int NST = 2 * MS, FV = D / 32;
                bf16x8 vf0[FV], vf1[FV];
                auto vload = [&](bf16x8 (&vf)[FV], int i) {
#pragma unroll
                    for (int j = 0; j < FV; ++j)
                        vf[j] = *(const bf16x8 *)&Vt[(r16 + ((i & 1) * FV + j) * 16) * VP + (s0 + (i >> 1)) * 32 + grp * 8];
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
        }
        if (t + NW < QT) {   // the next tile's operands, fetched while this tile's results drain
            bool o2;
            int t2, h2;
            const bf16 *qn = q_ptr(t + NW, o2, t2, h2);
#pragma unroll
            for (int ds = 0; ds < D / 32; ++ds) qf_next[ds] = *(const bf16x8 *)(qn + ds * 32 + grp * 8);
            am_next = anc[b * K + t2];
        }
        if constexpr (KS > 1) {
            // the tile's key parts merged into part 0, in part order
            const int slot0 = (hl * NW + tw) * (KS - 1);
            if (kp > 0) {
                const int sl = slot0 + kp - 1;
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt) mg_o[(sl * (D / 16) + dt) * 64 + lane] = o[dt];
                mg_m[sl * 64 + lane] = mloc;
                mg_l[sl * 64 + lane] = psum;
            }
            __syncthreads();
            if (kp == 0 && has) {
#pragma unroll
                for (int k2 = 0; k2 < KS - 1; ++k2) {
                    const int sl = slot0 + k2;
                    const float mk = mg_m[sl * 64 + lane], lk = mg_l[sl * 64 + lane];
                    if (mk == -INFINITY) continue;
                    const float mn = fmaxf(mloc, mk);
                    const float a0 = exp2f(mloc - mn), a1 = exp2f(mk - mn);
                    psum = psum * a0 + lk * a1;
#pragma unroll
                    for (int dt = 0; dt < D / 16; ++dt) o[dt] = o[dt] * a0 + mg_o[(sl * (D / 16) + dt) * 64 + lane] * a1;
                    mloc = mn;
                }
            }
            __syncthreads();
        }
        if (kp == 0 && has && col_ok) {
            const int64_t base = (((int64_t)b * nkv + g) * n_chunks + c) * R + rho;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt)
                *(floatx4 *)(part_o + base * D + dt * 16 + 4 * grp) = o[dt];
            if (grp == 0) part_ml[base] = make_float2(mloc, psum);
        }
    }
}

// Staged key/value layout of the group kernel: a 32-key stage is written into LDS 1 KB per wave
// instruction (global_load_lds, lane l fills bytes 16 l .. 16 l + 15):
//   keys   [32][D]; 16-byte column c of key k is stored at column c ^ key_swz(k), so the 16 key
//          rows an S^T fragment read touches fall in 16 different bank groups;
//   values page by page as the cache holds them, [page][D][16 slots]; the two 8-slot halves of
//          row d trade places when bit 3 of d is set, which does the same for V^T reads.
template <int D>
__device__ __forceinline__ int key_swz(int k) {
    if constexpr (D == 128) return (k & 3) | (((k >> 3) & 3) << 2);
    else return (k & 3) | (((k >> 3) & 1) << 2);
}

// s_waitcnt with vmcnt <= n (n < 64) and the other counters unconstrained
template <int n>
__device__ __forceinline__ void wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00);
}

// Many query columns per kv head (a draft tree of tens of nodes, 5 q heads per kv head: 20 query
// tiles), or many requests: one workgroup of eight waves per (request, kv head, group of up to
// 8 TW query tiles, range of rk keys), the group's query tiles dealt to the waves in turn
// (wave w: tiles w, w + 8, w + 16 of the group). Each 32-key stage of
// the range is fetched once, straight into LDS (global_load_lds, the stage's 2 D/16 blocks of
// 1 KB spread over the waves, in the wave kernel's layout), NBUF - 1 stages ahead, and every
// wave multiplies all of its tiles against it, so the keys and values cross HBM once whatever
// the number of tiles. One barrier per stage: the stage has landed for every wave, and the buffer
// refilled next was released by all of them. Online softmax per column in the log2 domain; o is
// rescaled only when some column's maximum moved; P as a bf16 high part plus a bf16 low part as
// in the other attention kernels; one partial per (range, column) for the combine.
constexpr int kGroupWaves = 8;
typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
#ifndef SV_GROUP_TARGET
#define SV_GROUP_TARGET 256                             // workgroups one launch aims at
#endif
#ifndef SV_GROUP_RK_MAX
#define SV_GROUP_RK_MAX 1024                            // keys per range at most (64 pages)
#endif
#ifndef SV_GROUP_NBUF
#define SV_GROUP_NBUF 4
#endif
#ifndef SV_GROUP_COMBINE_FEW
#define SV_GROUP_COMBINE_FEW 1
#endif

template <int D, int TW>
__global__ __launch_bounds__(64 * kGroupWaves) void attn_group_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k_pool, const bf16 *__restrict__ v_pool,
    const int32_t *__restrict__ block_table, int max_pages, const int32_t *__restrict__ ctx_len,
    const uint64_t *__restrict__ anc, const int32_t *__restrict__ status, int K, int nq, int nkv,
    int n_rg, int rk, int n_tg, float scale_log2, float *__restrict__ part_o, float2 *__restrict__ part_ml) {
    constexpr int NW = kGroupWaves;
    constexpr int SK = 32;                 // keys per stage
    constexpr int CD = D / 8;              // 16-byte columns of a key row
    constexpr int KB = D / 16;             // 1 KB blocks per stage, keys (values alike)
    constexpr int SLOTS = 2 * KB * 64;     // 16-byte slots per stage
    constexpr int LPW = 2 * KB / NW;       // blocks each wave loads per stage
    static_assert(2 * KB % NW == 0 && LPW >= 1, "a stage's blocks split evenly over the waves");
    constexpr int NBUF = SV_GROUP_NBUF;    // stage buffers (NBUF - 1 stages in flight)
    static_assert(NBUF >= 3 && NBUF <= 6, "stage buffers");
    constexpr int FK = D / 32, DT = D / 16;
    __shared__ bf16x8 lds[NBUF * SLOTS];

    const int r = blockIdx.x, g = blockIdx.y / n_tg, b = blockIdx.z;
    const int t0 = (blockIdx.y % n_tg) * (kGroupWaves * TW);   // this workgroup's first query tile
    if (status[b] != 0) return;            // uniform over the workgroup
    const int ctx = ctx_len[b];
    const int T = ctx + K;
    const int kbeg = r * rk;
    if (kbeg >= T) return;                 // uniform over the workgroup
    const int n_st = (min(rk, T - kbeg) + SK - 1) / SK;
    const int group = nq / nkv;
    const int R = group * K;
    const int QT = (R + 15) >> 4;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, grp = lane >> 4;

    // page ids of the range, lane i holding page i (rk <= 1024 keys: 64 pages); pages past the
    // request's last one stand in for the range's first (in bounds; values zeroed before use)
    const int np_req = (T + 15) >> 4;
    int pg;
    {
        const int p0 = kbeg >> 4, pidx = p0 + lane;
        pg = block_table[(int64_t)b * max_pages + (pidx < np_req ? pidx : p0)];
    }
    // this wave's tiles: query fragments and ancestor masks
    bf16x8 qf[TW][FK];
    uint64_t am[TW];
    bool col_ok[TW];
#pragma unroll
    for (int j = 0; j < TW; ++j) {
        const int rho = 16 * (t0 + wave + NW * j) + r16;
        col_ok[j] = rho < R;
        const int hh = col_ok[j] ? rho / K : 0, tok = col_ok[j] ? rho % K : 0;
        const bf16 *qrow = q + ((int64_t)(b * K + tok) * nq + g * group + hh) * D;
#pragma unroll
        for (int ds = 0; ds < FK; ++ds) qf[j][ds] = *(const bf16x8 *)(qrow + ds * 32 + grp * 8);
        am[j] = anc[b * K + tok];
    }

    auto issue = [&](int sl) __attribute__((always_inline)) {
        const int64_t p0 = __builtin_amdgcn_readlane(pg, 2 * sl);
        const int64_t p1 = __builtin_amdgcn_readlane(pg, 2 * sl + 1);
        bf16x8 *dst = lds + (sl % NBUF) * SLOTS;
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int j = wave + NW * i;   // keys: blocks 0 .. KB - 1; values: KB .. 2 KB - 1
            const bf16 *src;
            if (j < KB) {
                const int key = j * (512 / D) + lane / CD;
                const int64_t page = (j * (512 / D)) < 16 ? p0 : p1;
                const int col = (lane % CD) ^ key_swz<D>(key);
                src = k_pool + ((page * nkv + g) * 16 + (key & 15)) * D + col * 8;
            } else {
                const int jv = j - KB;
                const int64_t page = jv < D / 32 ? p0 : p1;
                const int d = (jv % (D / 32)) * 32 + (lane >> 1);
                const int half = (lane & 1) ^ ((d >> 3) & 1);
                src = v_pool + ((page * nkv + g) * D + d) * 16 + half * 8;
            }
            __builtin_amdgcn_global_load_lds((const void *)src,
                                             (__attribute__((address_space(3))) void *)(dst + j * 64),
                                             16, 0, 2);   // 2: non-temporal
        }
    };

    float m_ref[TW], l_run[TW];
    floatx4 o[TW][DT];
#pragma unroll
    for (int j = 0; j < TW; ++j) {
        m_ref[j] = -INFINITY;
        l_run[j] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[j][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    const int kr0 = 8 * (r16 >> 2) + (r16 & 3);   // S^T half 0 key row of this lane (half 1: +4)

    // Softmax against a reference per column that moves only when a score passes it by more than
    // 32 (log2 units): p = 2^(s - m_ref) stays below 2^32, which the fp32 sums and the bf16 high +
    // low parts carry as well as p <= 1, and o is rescaled (with a wave-wide exchange of the
    // column maxima) only then: at the first stage where the column sees a key, and practically
    // never after.
#pragma unroll
    for (int s0 = 0; s0 < NBUF - 1; ++s0)
        if (s0 < n_st) issue(s0);
    for (int sl = 0; sl < n_st; ++sl) {
        const int ahead = min(NBUF - 2, n_st - 1 - sl);   // later stages this wave has in flight
        if (ahead >= 4) wait_vm<4 * LPW>();
        else if (ahead == 3) wait_vm<3 * LPW>();
        else if (ahead == 2) wait_vm<2 * LPW>();
        else if (ahead == 1) wait_vm<LPW>();
        else wait_vm<0>();
        __syncthreads();                   // stage sl landed for every wave; stage sl - 1 released
        if (sl + NBUF - 1 < n_st) issue(sl + NBUF - 1);
        const int kb = kbeg + sl * SK;
        const int nvalid = min(SK, T - kb);
        bf16x8 *ks = lds + (sl % NBUF) * SLOTS;
        const bf16x8 *vs = ks + KB * 64;
        if (nvalid < SK) {
            // the request's last keys: values past them (stale slots, stand-in pages) are zeroed,
            // since a zero probability times a non-finite value is not zero
            bf16x8 *vz = ks + KB * 64;
            for (int idx = threadIdx.x; idx < 2 * D * 2; idx += 64 * NW) {
                const int pi = idx / (2 * D), d = (idx >> 1) % D, h = idx & 1;
                const int k0 = pi * 16 + h * 8;
                if (k0 + 8 <= nvalid) continue;
                bf16x8 *slot = vz + pi * 2 * D + d * 2 + (h ^ ((d >> 3) & 1));
                bf16x8 v = *slot;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (k0 + e >= nvalid) v[e] = (bf16)0.0f;
                *slot = v;
            }
            __syncthreads();
        }
        // key fragments: half h covers key rows kr0 + 4h, so each lane ends with keys
        // 8 grp .. 8 grp + 7 of every tile's S^T
        bf16x8 kf[2][FK];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int key = kr0 + 4 * h;
            const int sw = key_swz<D>(key);
#pragma unroll
            for (int ds = 0; ds < FK; ++ds) kf[h][ds] = ks[key * CD + ((grp + 4 * ds) ^ sw)];
        }
        const bool plain = nvalid == SK && kb + SK <= ctx;
        const int k0 = kb + 8 * grp;
        const int n_ctx = min(max(ctx - k0, 0), 8);
        const int j0 = max(k0 + n_ctx - ctx, 0);       // first draft index among the lane's keys
        const int n_in = min(max(kb + nvalid - k0, 0), 8);
        bf16x8 ph[TW], pl[TW];
        {
#pragma unroll
            for (int j = 0; j < TW; ++j) {
                if (t0 + wave + NW * j >= QT) continue;      // uniform over the wave
                floatx4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ds = 0; ds < FK; ++ds) {
                    sa = mfma16x16x32(kf[0][ds], qf[j][ds], sa);
                    sb = mfma16x16x32(kf[1][ds], qf[j][ds], sb);
                }
                float sv[8];                            // raw scores q . k
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sv[e] = sa[e];
                    sv[e + 4] = sb[e];
                }
                if (!plain) {
                    // committed positions always, draft positions on the column's root path
                    const unsigned anc8 = j0 < 64 ? (unsigned)(am[j] >> j0) & 0xffu : 0u;
                    unsigned vis = (((1u << n_ctx) - 1u) | (anc8 << n_ctx)) & ((1u << n_in) - 1u);
                    if (!col_ok[j]) vis = 0u;
#pragma unroll
                    for (int e = 0; e < 8; ++e) sv[e] = ((vis >> e) & 1u) ? sv[e] : -INFINITY;
                }
                const float mloc = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                                         fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7]))) * scale_log2;
                if (__any(mloc > m_ref[j] + 32.f)) {
                    float mc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
                    mc = fmaxf(mc, __shfl_xor(mc, 32, 64));
                    const float mn = fmaxf(m_ref[j], mc);
                    if (mn > m_ref[j]) {
                        // o and l are still zero where the reference was -inf
                        const float alpha = m_ref[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref[j] - mn);
                        l_run[j] *= alpha;
#pragma unroll
                        for (int dt = 0; dt < DT; ++dt) o[j][dt] = o[j][dt] * alpha;
                        m_ref[j] = mn;
                    }
                }
                // a column with no visible key yet has only -inf scores: any finite reference
                // gives p = 0 there
                const float m_use = m_ref[j] == -INFINITY ? 0.f : m_ref[j];
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const float2v pv = {__builtin_amdgcn_exp2f(__builtin_fmaf(sv[e], scale_log2, -m_use)),
                                        __builtin_amdgcn_exp2f(__builtin_fmaf(sv[e + 1], scale_log2, -m_use))};
                    const bf16x2v hi = __builtin_convertvector(pv, bf16x2v);
                    const float2v rest = {pv.x - (float)hi.x, pv.y - (float)hi.y};
                    const bf16x2v lo = __builtin_convertvector(rest, bf16x2v);
                    ph[j][e] = hi.x;
                    ph[j][e + 1] = hi.y;
                    pl[j][e] = lo.x;
                    pl[j][e + 1] = lo.y;
                    l_run[j] += pv.x + pv.y;
                }
            }
        }
        // O^T += V^T . P^T: one value fragment per 16 rows of d serves every tile
        const int vp = grp >> 1, vh = grp & 1;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int d = r16 + 16 * dt;
            const bf16x8 vf = vs[vp * 2 * D + d * 2 + (vh ^ ((d >> 3) & 1))];
#pragma unroll
            for (int j = 0; j < TW; ++j) {
                if (t0 + wave + NW * j >= QT) continue;
                o[j][dt] = mfma16x16x32(vf, ph[j], o[j][dt]);
                o[j][dt] = mfma16x16x32(vf, pl[j], o[j][dt]);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < TW; ++j) {
        float l = l_run[j];
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        if (t0 + wave + NW * j >= QT || !col_ok[j]) continue;
        const int rho = 16 * (t0 + wave + NW * j) + r16;
        const int64_t base = (((int64_t)b * nkv + g) * n_rg + r) * R + rho;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            *(floatx4 *)(part_o + base * D + dt * 16 + 4 * grp) = o[j][dt];
        if (grp == 0) part_ml[base] = make_float2(m_ref[j], l);
    }
}

// Merge the partials of one (node, q head): o = sum_c 2^(m_c - m*) O_c / sum_c 2^(m_c - m*) l_c
// over the partials c (one per chunk, or per range of chunks; kpp keys each). 256 threads = (D/4) column
// quads x CG groups; each thread merges partials c = cg, cg + CG, ... with every load issued
// before the arithmetic, then the CG states are merged in LDS in group order.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(
    const float *__restrict__ part_o, const float2 *__restrict__ part_ml,
    const int32_t *__restrict__ ctx_len, const int32_t *__restrict__ status, int K, int nq,
    int nkv, int n_chunks, int kpp, bf16 *__restrict__ out) {
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
    const int nc = (ctx_len[b] + K + kpp - 1) / kpp;   // partials (kpp keys each)
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

// Merge for few partials per (node, q head), as the wave kernel leaves them: one thread per
// (node, q head, column quad), the partials merged in order with every load of a batch of 4 in
// flight before the arithmetic.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_few_kernel(
    const float *__restrict__ part_o, const float2 *__restrict__ part_ml,
    const int32_t *__restrict__ ctx_len, const int32_t *__restrict__ status, int K, int nq,
    int nkv, int stride, int kpp, int64_t total, bf16 *__restrict__ out) {
    constexpr int NQD = D / 4;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const int quad = (int)(i % NQD);
    const int64_t rh = i / NQD;
    const int h = (int)(rh % nq), row = (int)(rh / nq);
    const int b = row / K, tok = row % K;
    bf16 *dst = out + frag_off(row, h * D + quad * 4, nq * D);   // fragment order: the O operand
    if (status[b] != 0) {
        store4(dst, 0.f, 0.f, 0.f, 0.f);
        return;
    }
    const int group = nq / nkv, g = h / group, hh = h % group;
    const int R = group * K, rho = hh * K + tok;
    const int nc = (ctx_len[b] + K + kpp - 1) / kpp;   // partials (kpp keys each)
    const int64_t base = ((int64_t)b * nkv + g) * stride * R + rho;
    float m = -INFINITY, l = 0.f;
    floatx4 o = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < nc; c0 += 4) {
        float2 ml[4];
        floatx4 oc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int c = min(c0 + t, nc - 1);
            ml[t] = part_ml[base + (int64_t)c * R];
            oc[t] = *(const floatx4 *)(part_o + (base + (int64_t)c * R) * D + quad * 4);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (c0 + t >= nc || ml[t].x == -INFINITY) continue;
            const float mn = fmaxf(m, ml[t].x);
            const float a = exp2f(m - mn), w = exp2f(ml[t].x - mn);
            l = l * a + ml[t].y * w;
            o = o * a + oc[t] * w;
            m = mn;
        }
    }
    store4(dst, o[0] / l, o[1] / l, o[2] / l, o[3] / l);
}

// Tunables: the largest chunk-kernel grid (workgroups) before the group kernel takes over, and
// the chunk kernel's keys per workgroup and waves per query tile.
#ifndef SV_ATTN_SMALL_GRID
#define SV_ATTN_SMALL_GRID 512
#endif
#ifndef SV_ATTN_CH
#define SV_ATTN_CH 192                                  // keys per chunk-kernel workgroup
#endif
#ifndef SV_ATTN_KS
#define SV_ATTN_KS 1                                    // waves per query tile (key parts)
#endif

hipError_t attention(const AttnArgs &a, hipStream_t st) {
    const float scale_log2 = kLog2e / sqrtf((float)a.D);
    const int R = a.nq / a.nkv * a.K;
    const int QT = (R + 15) / 16;
    // One request and few query tiles (a block of 16 with 5 q heads per kv head: 5 tiles): one
    // chunk of SV_ATTN_CH keys and one kv head per workgroup, a tile per wave (one workgroup per
    // compute unit: 176 at a 4096-token context and 8 kv heads, 13.4 us on the 27B block against
    // 14.4 for 128-key chunks over two heads, which leave half the units idle, and 16.2 for
    // 128-key chunks over one head, eight workgroups too many for one round; two waves per tile
    // measured 14.6). Everything else (a draft tree's many tiles, a batch of requests) runs the
    // group kernel.
    const int nw = (QT + 4) / 5 < (QT + 3) / 4 ? 5 : 4;   // chunk kernel: 5 tile slots or 4
    const int64_t max_keys = (int64_t)a.max_pages * kPage;
    const int n_small = (int)((max_keys + SV_ATTN_CH - 1) / SV_ATTN_CH);
    const int64_t wgs1 = (int64_t)n_small * a.nkv * a.B;
    const bool small = QT < 8 && wgs1 <= SV_ATTN_SMALL_GRID && n_small <= a.n_chunks;
    int kpp, stride;
    bool few;
    if (!small) {
        // the group kernel: a kv head's query tiles in groups of up to 24 (three per wave),
        // ranges sized so that the (range, tile group, kv head, request) workgroups fill the
        // compute units about once, each range a whole number of 32-key stages, at least one
        // chunk and at most 64 pages. A 64-node tree at 5 q heads per kv head is one group of 20
        // tiles (ranges of 288 keys at an 8192-token context); a batch of 32 requests x 16 at
        // contexts up to 8192 is one group of 5 per request (ranges of 1024 keys): 134 us per
        // layer against 185 for a kernel whose waves each held all five tiles at one wave per
        // SIMD, 33.6 us on the tree against 49.3 for that kernel's four tile groups, each of
        // which streamed the same keys
        const int n_tg = (QT + 3 * kGroupWaves - 1) / (3 * kGroupWaves);
        const int tpg = (QT + n_tg - 1) / n_tg;                 // tiles per group
        const int tw = (tpg + kGroupWaves - 1) / kGroupWaves;   // tiles per wave
        const int64_t per = (max_keys * a.nkv * n_tg * a.B + SV_GROUP_TARGET - 1) / SV_GROUP_TARGET;
        int64_t rk64 = (per + 31) / 32 * 32;
        if (rk64 < kAttnChunk) rk64 = kAttnChunk;
        if (rk64 > SV_GROUP_RK_MAX) rk64 = SV_GROUP_RK_MAX;
        const int rk = (int)rk64;
        const int n_rg = (int)((max_keys + rk - 1) / rk);
        stride = n_rg;
        kpp = rk;
        few = SV_GROUP_COMBINE_FEW != 0;
        const dim3 grid_g(n_rg, a.nkv * n_tg, a.B);
#define SV_GROUP(DD, TWV)                                                                          \
    hipLaunchKernelGGL((attn_group_kernel<DD, TWV>), grid_g, dim3(64 * kGroupWaves), 0, st, a.q,     \
                       a.k_pool, a.v_pool, a.block_table, a.max_pages, a.ctx_len, a.anc, a.status,  \
                       a.K, a.nq, a.nkv, n_rg, rk, n_tg, scale_log2, a.part_o, a.part_ml)
        if (a.D == 128) {
            if (tw == 1) SV_GROUP(128, 1);
            else if (tw == 2) SV_GROUP(128, 2);
            else SV_GROUP(128, 3);
        } else {
            if (tw == 1) SV_GROUP(64, 1);
            else if (tw == 2) SV_GROUP(64, 2);
            else SV_GROUP(64, 3);
        }
#undef SV_GROUP
    } else {
        kpp = SV_ATTN_CH;
        stride = n_small;
        few = false;
        const dim3 grid_h(n_small, a.nkv, a.B);
#define SV_ATTN(DD, NWV)                                                                          \
    hipLaunchKernelGGL((attn_partial_kernel<DD, NWV, 1, SV_ATTN_CH, SV_ATTN_KS>), grid_h,          \
                       dim3(64 * NWV * SV_ATTN_KS), 0, st, a.q, a.k_pool, a.v_pool, a.block_table, \
                       a.max_pages, a.ctx_len, a.anc, a.status, a.K, a.nq, a.nkv, n_small,         \
                       scale_log2, a.part_o, a.part_ml)
        if (a.D == 128) {
            if (nw == 4) { SV_ATTN(128, 4); }
            else { SV_ATTN(128, 5); }
        } else {
            if (nw == 4) { SV_ATTN(64, 4); }
            else { SV_ATTN(64, 5); }
        }
#undef SV_ATTN
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (few) {
        // tens of partials per (node, q head) at most: one thread per (node, q head, column quad)
        const int64_t total = (int64_t)a.B * a.K * a.nq * (a.D / 4);
        const dim3 grid_c((unsigned)((total + 255) / 256));
        if (a.D == 128)
            hipLaunchKernelGGL(attn_combine_few_kernel<128>, grid_c, dim3(256), 0, st, a.part_o,
                               a.part_ml, a.ctx_len, a.status, a.K, a.nq, a.nkv, stride, kpp, total, a.out);
        else
            hipLaunchKernelGGL(attn_combine_few_kernel<64>, grid_c, dim3(256), 0, st, a.part_o,
                               a.part_ml, a.ctx_len, a.status, a.K, a.nq, a.nkv, stride, kpp, total, a.out);
    } else if (a.D == 128) {
        hipLaunchKernelGGL(attn_combine_kernel<128>, dim3(a.B * a.K, a.nq), dim3(256), 0, st,
                           a.part_o, a.part_ml, a.ctx_len, a.status, a.K, a.nq, a.nkv, stride, kpp, a.out);
    } else {
        hipLaunchKernelGGL(attn_combine_kernel<64>, dim3(a.B * a.K, a.nq), dim3(256), 0, st,
                           a.part_o, a.part_ml, a.ctx_len, a.status, a.K, a.nq, a.nkv, stride, kpp, a.out);
    }
    return hipGetLastError();
}

}  // namespace sv
