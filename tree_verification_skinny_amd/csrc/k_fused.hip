// k_fused.hip — the layers of a verify pass with at most 16 rows (a block of 16 draft tokens, or a
// few small blocks or trees) as one persistent kernel per group of up to 16 layers.
//
// At batch 1 the pass reads every target weight for a handful of tokens [SpecPilot digest,
// airadar.tv — summary paragraph], so the time should be the weight stream and nothing else.
// Launched as one kernel per step of the layer (projection, split-K add, RoPE, attention and its
// merge, residual + RMSNorm), every dependent step drains the chip and refills it: a few
// microseconds per boundary, most of the gap to the HBM roofline. Here every compute unit runs
// one workgroup of 8 waves for the whole group of layers, and the steps hand data to each other
// through memory, inside the kernel:
//   * each projection is split evenly over the workgroups as a range of (64-column group,
//     32-wide K step) units of its packed weights (4 MFMA fragments, 4 KB, per unit). A group
//     whose K steps fall to several workgroups is finished by the last of them to arrive (a
//     per-group counter with a handful of arrivals), which adds the parts in workgroup order,
//     so results do not depend on timing;
//   * that finisher runs the projection's epilogue: for QKV the bf16 rounding, RoPE (a group
//     holds the two 32-column halves j and j + D/2 of a head's rotation pairs) and the q rows
//     and draft K/V cache slots; for O and down the residual add and the group's sums of
//     squares; for gate/up SwiGLU. The RMSNorm before QKV and gate/up is applied by the
//     consumer while it loads its activation operand (row scale from the groups' sums);
//   * attention runs as (kv head, request, chunk of keys) items whose committed-context keys
//     and values are staged into LDS before the item waits for this layer's q, k and v, then
//     merge tasks add the chunks (log2-domain softmax partials) into the O projection's operand;
//   * a consumer waits for its inputs by polling one epoch word per producer group, item or
//     task (one wave, device-scope loads), not by a grid barrier, and every wait is bounded:
//     past one second it sets an error word, the workgroup leaves, and the pass reports every
//     request failed.
// Data one workgroup hands to another is written with device-scope (write-through) stores, and a
// writer waits for its stores to complete before it publishes the epoch or the arrival. Small
// hand-offs (flags, partial sums, sums of squares, the residual read by the finisher) are read
// with device-scope loads. The large operands (the residual stream, q, the attention output, the
// SwiGLU output, the draft K/V rows) are read with plain, cached loads, without a cache
// invalidation per phase (measured far too slow: every wave's acquire invalidates its L2): each
// has one slot per layer of the launch, written once in it, and every reader waits for all
// writers of the lines it reads, so no cache can hold a line of it from before its write in this
// launch; across launches the kernel boundary makes the earlier writes visible. The one slot read
// both before and after its rewrite (the launch's input, rewritten by its last layer) is read with
// device-scope loads after the rewrite. Weights and committed KV rows use non-temporal loads.
//
// Arithmetic is that of the per-step kernels (bf16 storage between steps, fp32 accumulation and
// softmax, P as a bf16 high part plus a bf16 low part); only the order of the split-K sums and
// of the norm's sum of squares differs.
#include "kernels.hpp"

namespace sv {

namespace {

constexpr int kFW = 8;                       // waves per persistent workgroup
constexpr int kFT = kFW * 64;
constexpr int kCHS = 160;                    // most keys per attention item
constexpr int kSC1 = 16;                     // buffer-instruction cache policy: device scope
constexpr uint64_t kWaitTicks = 100000000ull;   // one second of s_memrealtime (100 MHz)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---- device-scope loads and stores -----------------------------------------------------------
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ bf16x8 ld_dev16(const void *base, uint32_t off) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rsrc(base), off, 0, kSC1));
}
__device__ __forceinline__ void st_dev16B(void *base, uint32_t off, floatx4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rsrc(base), off, 0, kSC1);
}
__device__ __forceinline__ uint32_t ld_dev32(const void *p) {
    return __hip_atomic_load(reinterpret_cast<uint32_t *>(const_cast<void *>(p)), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_devf(const float *p) { return __uint_as_float(ld_dev32(p)); }
__device__ __forceinline__ uint64_t ld_dev64(const void *p) {
    return __hip_atomic_load(reinterpret_cast<uint64_t *>(const_cast<void *>(p)), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev16(void *p, uint16_t v) {
    __hip_atomic_store(reinterpret_cast<uint16_t *>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev32(void *p, uint32_t v) {
    __hip_atomic_store(reinterpret_cast<uint32_t *>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev64(void *p, uint64_t v) {
    __hip_atomic_store(reinterpret_cast<uint64_t *>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t pack2f(float a, float b) {
    return (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
}
__device__ __forceinline__ float lo_f(uint64_t v) { return __uint_as_float((uint32_t)v); }
__device__ __forceinline__ float hi_f(uint64_t v) { return __uint_as_float((uint32_t)(v >> 32)); }
__device__ __forceinline__ uint32_t pack2bf(float a, float b) {
    const bf16 x = to_bf(a), y = to_bf(b);
    return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}
__device__ __forceinline__ float bf_lo(uint32_t v) { return (float)__builtin_bit_cast(bf16, (uint16_t)(v & 0xffffu)); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return (float)__builtin_bit_cast(bf16, (uint16_t)(v >> 16)); }

// This wave's stores have completed (and so are visible at device scope: they were written
// through) before anything after this point is issued.
__device__ __forceinline__ void stores_done() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---- LDS, shared by the steps (one workgroup per compute unit) ----------------------------------
template <int D>
struct Smem {
    union {
        floatx4 red[4 * kFW * 4 * 64];                      // the waves' accumulators, 4 groups (128 KB)
        struct {
            bf16 ks[kCHS * (D + 8)];                         // keys of the item, rows padded
            bf16 vt[D * (kCHS + 8)];                         // values transposed
        } kv;
        struct {
            floatx4 o[8 * (D / 16) * 64];                    // a tile's key-part partials
            float m[8 * 16], l[8 * 16];
        } mrg;
    } u;
    float y[1024];                                           // a finished group's 16 x 64 sums
    float ss[kFT];
    float rs[16];
    int flag;
    int last[4];
};

// Epoch wait: every word of the ranges f_i[0..n_i) reaches `epoch`. Wave 0 polls; false on a
// timeout or when another workgroup has already timed out (the caller leaves the kernel).
template <int D>
__device__ bool wait_ranges(const uint32_t *f0, int n0, const uint32_t *f1, int n1, const uint32_t *f2,
                            int n2, uint32_t epoch, uint32_t *err, Smem<D> &sm) {
    if (threadIdx.x < 64) {
        int ok = 1;
        const int lane = threadIdx.x;
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while (true) {
            if (ld_dev32(err) != 0u) { ok = 0; break; }
            // every flag load of a round is issued before any is tested
            uint32_t mn = 0xffffffffu;
            const uint32_t *fs[3] = {f0, f1, f2};
            const int ns[3] = {n0, n1, n2};
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                for (int i0 = 0; i0 < ns[r]; i0 += 64 * 16) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int i = i0 + lane + 64 * j;
                        const uint32_t v = i < ns[r] ? ld_dev32(fs[r] + i) : 0xffffffffu;
                        mn = v < mn ? v : mn;
                    }
                }
            }
            if (__all(mn >= epoch)) break;
            if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
                if (lane == 0) st_dev32(err, 1u);
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (lane == 0) sm.flag = ok;
    }
    __syncthreads();
    const bool ok = sm.flag != 0;
    __syncthreads();
    return ok;
}

template <int D>
__device__ __forceinline__ bool wait_all(const uint32_t *f, int n, uint32_t epoch, uint32_t *err, Smem<D> &sm) {
    return wait_ranges<D>(f, n, nullptr, 0, nullptr, 0, epoch, err, sm);
}

// Per-layer operand slots of layer li of this launch.
__device__ __forceinline__ bf16 *x_in(const FusedArgs &a, int li) {
    return a.x_d + (int64_t)(li == 0 ? kFusedMaxLayers - 1 : li - 1) * 16 * a.H;
}
__device__ __forceinline__ bf16 *x_mid(const FusedArgs &a, int li) { return a.x_o + (int64_t)li * 16 * a.H; }
__device__ __forceinline__ bf16 *x_out(const FusedArgs &a, int li) { return a.x_d + (int64_t)li * 16 * a.H; }
__device__ __forceinline__ bf16 *q_of(const FusedArgs &a, int li) { return a.q + (int64_t)li * a.M * a.nq * a.D; }
__device__ __forceinline__ bf16 *ao_of(const FusedArgs &a, int li) { return a.ao + (int64_t)li * 16 * a.nq * a.D; }
__device__ __forceinline__ bf16 *h_of(const FusedArgs &a, int li) { return a.h + (int64_t)li * 16 * a.F; }

// Phase trace (optional): s_memrealtime of event ev of workgroup blockIdx.x in layer l.
__device__ __forceinline__ void stamp(const FusedArgs &a, int l, int ev) {
    if (a.trace_t != nullptr && threadIdx.x == 0)
        a.trace_t[((int64_t)l * gridDim.x + blockIdx.x) * kFusedTraceEvents + ev] = __builtin_amdgcn_s_memrealtime();
}

// Publish an epoch after every wave's stores are complete.
template <int D>
__device__ __forceinline__ void publish(uint32_t *f, uint32_t epoch) {
    stores_done();
    __syncthreads();
    if (threadIdx.x == 0) st_dev32(f, epoch);
}

// The workgroup that holds unit u of a projection split as even ranges over g_eff workgroups.
__device__ __forceinline__ int wg_of(int u, const FusedPhase &p) {
    return (int)(((int64_t)(u + 1) * p.g_eff - 1) / p.units);
}

// 16-row weight tile of local tile t (0..3) of a 64-column group.
template <int PH, int D>
__device__ __forceinline__ int tile_of(int g, int t, const FusedArgs &a) {
    if constexpr (PH == FUSED_QKV) {
        // the rotation pairs (j, j + D/2) of a head in one group: its tiles 2a, 2a + 1 and the
        // two D/32 tiles further on
        constexpr int tph = D / 16, gph = D / 64;
        const int hd = g / gph, ha = g % gph;
        return hd * tph + (t < 2 ? 2 * ha + t : 2 * ha + (t - 2) + D / 32);
    } else if constexpr (FUSED_GU == PH) {
        // gate columns 32g .. 32g + 31 and the matching up columns F + 32g ..
        return t < 2 ? 2 * g + t : a.F / 16 + 2 * g + (t - 2);
    } else {
        return 4 * g + t;
    }
}

// u = bf16((x * r) * gain) for one operand fragment (8 columns of one row).
__device__ __forceinline__ bf16x8 norm_frag(bf16x8 x, float r, bf16x8 g) {
#pragma clang fp contract(off)
    bf16x8 o;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = to_bf((to_f(x[j]) * r) * to_f(g[j]));
    return o;
}

// ---- projection epilogues on a finished group's sums: thread tau holds sums (y0, y1) of tile
// t = tau / 128, lane ln = (tau / 2) % 64, values 2 (tau % 2) and +1 of that MFMA lane, i.e.
// row m = ln % 16, columns 16 t + 4 (ln / 16) + 2 (tau % 2) and +1 of the group ----------------
template <int D>
__device__ void epi_qkv(const FusedArgs &a, int li, int g, float y0, float y1, Smem<D> &sm) {
#pragma clang fp contract(off)
    const int tau = threadIdx.x;
    sm.y[2 * tau] = y0;
    sm.y[2 * tau + 1] = y1;
    __syncthreads();
    if (tau < 256) {
        const float p0 = sm.y[2 * (tau + 256)], p1 = sm.y[2 * (tau + 256) + 1];   // the partners
        const int t = tau >> 7, ln = (tau >> 1) & 63, jp = tau & 1;
        const int m = ln & 15;
        const int hd = g / (D / 64), ha = g % (D / 64);
        const int j = (2 * ha + t) * 16 + 4 * (ln >> 4) + 2 * jp;   // first dim, j + 1 the second
        if (m < a.M) {
            const float a0 = round_bf(y0), a1 = round_bf(y1), c0 = round_bf(p0), c1 = round_bf(p1);
            float lo0 = a0, lo1 = a1, hi0 = c0, hi1 = c1;
            if (hd < a.nq + a.nkv) {
                const float2 r0 = a.rope[(int64_t)m * (D / 2) + j], r1 = a.rope[(int64_t)m * (D / 2) + j + 1];
                lo0 = a0 * r0.x - c0 * r0.y;
                hi0 = c0 * r0.x + a0 * r0.y;
                lo1 = a1 * r1.x - c1 * r1.y;
                hi1 = c1 * r1.x + a1 * r1.y;
            }
            const int b = m / a.K, node = m % a.K;
            if (hd < a.nq) {
                bf16 *qr = q_of(a, li) + ((int64_t)m * a.nq + hd) * D;
                st_dev32(qr + j, pack2bf(lo0, lo1));
                st_dev32(qr + j + D / 2, pack2bf(hi0, hi1));
            } else if (a.status[b] == 0) {
                const int pos = a.ctx_len[b] + node;
                const int page = page_of(a.block_table, a.max_pages, b, pos);
                const int slot = pos & 15;
                const int64_t lofs = (int64_t)(a.L0 + li) * a.layer_stride;
                if (hd < a.nq + a.nkv) {
                    bf16 *kr = a.k_pool + lofs + (((int64_t)page * a.nkv + (hd - a.nq)) * 16 + slot) * D;
                    st_dev32(kr + j, pack2bf(lo0, lo1));
                    st_dev32(kr + j + D / 2, pack2bf(hi0, hi1));
                } else {
                    bf16 *vr = a.v_pool + lofs + (((int64_t)page * a.nkv + (hd - a.nq - a.nkv)) * D) * 16 + slot;
                    st_dev16(vr + (int64_t)j * 16, __builtin_bit_cast(uint16_t, to_bf(lo0)));
                    st_dev16(vr + (int64_t)(j + 1) * 16, __builtin_bit_cast(uint16_t, to_bf(lo1)));
                    st_dev16(vr + (int64_t)(j + D / 2) * 16, __builtin_bit_cast(uint16_t, to_bf(hi0)));
                    st_dev16(vr + (int64_t)(j + 1 + D / 2) * 16, __builtin_bit_cast(uint16_t, to_bf(hi1)));
                }
            }
        }
    }
}

// x = bf16(x + bf16(y)) on the group's 64 columns, and the group's sum of squares per row; xo is
// this thread's pair of x (requested by the caller ahead of the fix-up).
template <int D>
__device__ void epi_resid(const FusedArgs &a, int li, int l, int g, bool down, float y0, float y1, uint32_t xo,
                          Smem<D> &sm) {
#pragma clang fp contract(off)
    const int tau = threadIdx.x;
    const int t = tau >> 7, ln = (tau >> 1) & 63, jp = tau & 1;
    const int m = ln & 15;
    const int col = 64 * g + 16 * t + 4 * (ln >> 4) + 2 * jp;
    float x0 = 0.f, x1 = 0.f;
    if (m < a.M) {
        const int64_t xo_off = frag_off(m, col, a.H);
        x0 = round_bf(bf_lo(xo) + round_bf(y0));
        x1 = round_bf(bf_hi(xo) + round_bf(y1));
        const uint32_t xn = pack2bf(x0, x1);
        st_dev32((down ? x_out(a, li) : x_mid(a, li)) + xo_off, xn);
        if (down && a.trace != nullptr)
            *reinterpret_cast<uint32_t *>(a.trace + ((int64_t)(l + 1) * a.M + m) * a.H + col) = xn;
    }
    sm.ss[tau] = x0 * x0 + x1 * x1;
    __syncthreads();
    if (tau < 16) {
        float s = 0.f;
        for (int tt = 0; tt < 4; ++tt)
            for (int q4 = 0; q4 < 4; ++q4)
                for (int j2 = 0; j2 < 2; ++j2) s += sm.ss[tt * 128 + (16 * q4 + tau) * 2 + j2];
        st_dev32((down ? a.ssq_d : a.ssq_o) + g * 16 + tau, __float_as_uint(s));
    }
}

// h = silu(bf16(gate)) * bf16(up) for the group's 32 columns.
template <int D>
__device__ void epi_swiglu(const FusedArgs &a, int li, int g, float y0, float y1, Smem<D> &sm) {
#pragma clang fp contract(off)
    const int tau = threadIdx.x;
    sm.y[2 * tau] = y0;
    sm.y[2 * tau + 1] = y1;
    __syncthreads();
    if (tau < 256) {
        const float p0 = sm.y[2 * (tau + 256)], p1 = sm.y[2 * (tau + 256) + 1];
        const int t = tau >> 7, ln = (tau >> 1) & 63, jp = tau & 1;
        const int m = ln & 15;
        if (m < a.M) {
            const int col = 32 * g + 16 * t + 4 * (ln >> 4) + 2 * jp;
            const float g0 = round_bf(y0), g1 = round_bf(y1), u0 = round_bf(p0), u1 = round_bf(p1);
            const float h0 = (g0 / (1.0f + expf(-g0))) * u0, h1 = (g1 / (1.0f + expf(-g1))) * u1;
            st_dev32(h_of(a, li) + frag_off(m, col, a.F), pack2bf(h0, h1));
        }
    }
}

// ---- one projection of layer l (li within this launch) -------------------------------------------
template <int PH, int MAXSEG, int D>
__device__ bool gemm_phase(const FusedArgs &a, int li, int l, Smem<D> &sm) {
    const FusedPhase &p = a.ph[PH];
    const int wg = blockIdx.x;
    if (wg >= p.g_eff) return true;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t ep = (uint32_t)l + 1;
    const int S = p.S;
    const int u0 = (int)((int64_t)p.units * wg / p.g_eff);
    const int u1 = (int)((int64_t)p.units * (wg + 1) / p.g_eff);
    const int gA = u0 / S, gB = (u1 - 1) / S;

    constexpr int ev0 = PH == FUSED_QKV ? 0 : (PH == FUSED_O ? 6 : (PH == FUSED_GU ? 10 : 14));
    constexpr bool kNorm = PH == FUSED_QKV || PH == FUSED_GU;
    stamp(a, l, ev0);
    floatx4 acc[MAXSEG][4];
#pragma unroll
    for (int s = 0; s < MAXSEG; ++s)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[s][t] = floatx4{0.f, 0.f, 0.f, 0.f};

    // the wave's units are u0 + wave + 8 i: batches of two (units k and k + 8, k = wave + 16 j),
    // two batches in flight while one is multiplied. Weights do not depend on the inputs: the
    // first two batches' weights are requested before the wait for the inputs.
    const bf16 *W = a.w[li][PH];
    const int n = u1 - u0;
    struct Batch {
        bf16x8 w[2][4], x[2], g[2];
        int slot[2], s[2];
        bool live[2];
    };
    auto issue_w = [&](Batch &bt, int k, int g, int st) {
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) {
            bt.live[uu] = k + 8 * uu < n;
            int gg = g, ss = st;
            if (uu == 1) {
                ss += 8;
                while (ss >= S) { ss -= S; ++gg; }
            }
            bt.slot[uu] = gg - gA;
            bt.s[uu] = ss;
            if (!bt.live[uu]) continue;
            const bf16 *wb = W + ((int64_t)ss * 64 + lane) * 8;
#pragma unroll
            for (int t = 0; t < 4; ++t)
                bt.w[uu][t] = stream_load((const bf16x8 *)(wb + (int64_t)tile_of<PH, D>(gg, t, a) * S * 512));
        }
    };
    const bf16 *X = PH == FUSED_QKV ? x_in(a, li) : (PH == FUSED_GU ? x_mid(a, li) : (PH == FUSED_O ? ao_of(a, li) : h_of(a, li)));
    const bf16 *gain = PH == FUSED_QKV ? a.g_attn[li] : a.g_mlp[li];
    auto issue_x = [&](Batch &bt) {
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) {
            if (!bt.live[uu]) continue;
            bt.x[uu] = *(const bf16x8 *)(X + (bt.s[uu] * 64 + lane) * 8);
            if constexpr (kNorm) bt.g[uu] = *(const bf16x8 *)(gain + bt.s[uu] * 32 + 8 * (lane >> 4));
        }
    };
    auto advance = [&](int &g, int &st) {
        st += 16;
        while (st >= S) { st -= S; ++g; }
    };
    Batch A, B;
    int k = wave;
    int gk = (u0 + wave) / S, sk = (u0 + wave) - gk * S;   // (group, step) of unit u0 + k
    int gB_ = gk, sB_ = sk;
    advance(gB_, sB_);                                    // ... of unit u0 + k + 16
    if (k < n) issue_w(A, k, gk, sk);
    if (k + 16 < n) issue_w(B, k + 16, gB_, sB_);

    // inputs of this projection
    bool ok = true;
    if constexpr (PH == FUSED_QKV) {
        if (l > 0) ok = wait_all(a.ph[FUSED_DOWN].flag, a.ph[FUSED_DOWN].groups, (uint32_t)l, a.err, sm);
    } else if constexpr (PH == FUSED_O) {
        ok = wait_all(a.f_comb, a.n_tasks, ep, a.err, sm);
    } else if constexpr (PH == FUSED_GU) {
        ok = wait_all(a.ph[FUSED_O].flag, a.ph[FUSED_O].groups, ep, a.err, sm);
    } else {
        ok = wait_all(a.ph[FUSED_GU].flag, a.ph[FUSED_GU].groups, ep, a.err, sm);
    }
    if (!ok) return false;
    stamp(a, l, ev0 + 1);

    float rs = 1.f;
    if constexpr (kNorm) {
        if (threadIdx.x < 16) {
            const float *ssq = PH == FUSED_QKV ? a.ssq_d : a.ssq_o;
            float s = 0.f;
            for (int gg = 0; gg < a.H / 64; ++gg) s += ld_devf(ssq + gg * 16 + threadIdx.x);
            sm.rs[threadIdx.x] = 1.0f / sqrtf(s / (float)a.H + a.eps);
        }
        __syncthreads();
        rs = sm.rs[lane & 15];
    }
    auto consume = [&](const Batch &bt) {
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) {
            if (!bt.live[uu]) continue;
            bf16x8 b = bt.x[uu];
            if constexpr (kNorm) b = norm_frag(b, rs, bt.g[uu]);
#pragma unroll
            for (int sl = 0; sl < MAXSEG; ++sl)
                if (bt.slot[uu] == sl) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) acc[sl][t] = mfma16x16x32(bt.w[uu][t], b, acc[sl][t]);
                }
        }
    };
    if (k < n) {
        issue_x(A);
        if (k + 16 < n) issue_x(B);
        // (g3, s3): unit of the next batch to request (k + 32)
        int g3 = gB_, s3 = sB_;
        advance(g3, s3);
        // A, B hold batches k, k + 16 (as far as they exist); each consumed batch's registers
        // take the batch two ahead
#define SV_STAGE(X_)                                      \
        consume(X_);                                      \
        k += 16;                                          \
        if (k >= n) break;                                \
        if (k + 16 < n) {                                 \
            issue_w(X_, k + 16, g3, s3);                  \
            issue_x(X_);                                  \
        }                                                 \
        advance(g3, s3);
        while (true) {
            SV_STAGE(A)
            SV_STAGE(B)
        }
#undef SV_STAGE
    }

    stamp(a, l, ev0 + 2);
    // the groups this workgroup touched: every wave's sums into LDS, one barrier, each thread
    // adds its element over the waves in wave order
    const int nseg = gB - gA + 1;
    const int tau = threadIdx.x;
    // the residual's old values of this thread's pairs, requested before the fix-up's round trips
    uint32_t xo_pre[MAXSEG];
#pragma unroll
    for (int sl = 0; sl < MAXSEG; ++sl) {
        xo_pre[sl] = 0u;
        if constexpr (PH == FUSED_O || PH == FUSED_DOWN) {
            const int t = tau >> 7, ln = (tau >> 1) & 63, jp = tau & 1, m = ln & 15;
            if (sl < nseg && m < a.M) {
                const bf16 *xs = PH == FUSED_DOWN ? x_mid(a, li) : x_in(a, li);
                xo_pre[sl] = ld_dev32(xs + frag_off(m, 64 * (gA + sl) + 16 * t + 4 * (ln >> 4) + 2 * jp, a.H));
            }
        }
    }
#pragma unroll
    for (int sl = 0; sl < MAXSEG; ++sl)
        if (sl < nseg) {
#pragma unroll
            for (int t = 0; t < 4; ++t) sm.u.red[((sl * kFW + wave) * 4 + t) * 64 + lane] = acc[sl][t];
        }
    __syncthreads();
    float y0[MAXSEG], y1[MAXSEG];
    {
        const int t = tau >> 7, ln = (tau >> 1) & 63, jp = tau & 1;
#pragma unroll
        for (int sl = 0; sl < MAXSEG; ++sl) {
            y0[sl] = 0.f;
            y1[sl] = 0.f;
            if (sl >= nseg) continue;
#pragma unroll
            for (int w = 0; w < kFW; ++w) {
                const floatx4 v = sm.u.red[((sl * kFW + w) * 4 + t) * 64 + ln];
                y0[sl] += jp ? v[2] : v[0];
                y1[sl] += jp ? v[3] : v[1];
            }
        }
    }
    __syncthreads();
    // groups shared with other workgroups: partial sums out, one completion wait, the arrivals;
    // the last to arrive at a group finishes it
    unsigned split = 0u, fin = 0u;
    int np_[MAXSEG];
#pragma unroll
    for (int sl = 0; sl < MAXSEG; ++sl) {
        np_[sl] = 1;
        if (sl >= nseg) continue;
        const int g = gA + sl;
        if (u0 <= g * S && u1 >= (g + 1) * S) {
            fin |= 1u << sl;
            continue;
        }
        split |= 1u << sl;
        const int wfst = wg_of(g * S, p), wlst = wg_of((g + 1) * S - 1, p);
        np_[sl] = wlst - wfst + 1;
        float *pp = p.part + ((int64_t)g * p.max_parts + (wg - wfst)) * 1024;
        st_dev64(pp + 2 * tau, pack2f(y0[sl], y1[sl]));
    }
    if (split != 0u) {
        stores_done();
        __syncthreads();
        if (tau < nseg && ((split >> tau) & 1u)) {
            uint32_t target = 1u;
#pragma unroll
            for (int sl = 0; sl < MAXSEG; ++sl)
                if (sl == tau) target = (uint32_t)np_[sl] * ep;
            const uint32_t old = __hip_atomic_fetch_add(p.cnt + gA + tau, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sm.last[tau] = old + 1 == target;
        }
        __syncthreads();
#pragma unroll
        for (int sl = 0; sl < MAXSEG; ++sl)
            if (((split >> sl) & 1u) && sm.last[sl]) fin |= 1u << sl;
        // every finishing group's parts, loads issued together, added in workgroup order
#pragma unroll
        for (int sl = 0; sl < MAXSEG; ++sl) {
            if (!((split >> sl) & 1u) || !((fin >> sl) & 1u)) continue;
            const float *pb = p.part + (int64_t)(gA + sl) * p.max_parts * 1024 + 2 * tau;
            float a0 = 0.f, a1 = 0.f;
            for (int pi = 0; pi < np_[sl]; ++pi) {
                const uint64_t v = ld_dev64(pb + (int64_t)pi * 1024);
                a0 += lo_f(v);
                a1 += hi_f(v);
            }
            y0[sl] = a0;
            y1[sl] = a1;
        }
    }
    // epilogues of the finished groups, one completion wait, their epochs
#pragma unroll
    for (int sl = 0; sl < MAXSEG; ++sl) {
        if (!((fin >> sl) & 1u)) continue;
        if constexpr (PH == FUSED_QKV) epi_qkv<D>(a, li, gA + sl, y0[sl], y1[sl], sm);
        else if constexpr (PH == FUSED_GU) epi_swiglu<D>(a, li, gA + sl, y0[sl], y1[sl], sm);
        else epi_resid<D>(a, li, l, gA + sl, PH == FUSED_DOWN, y0[sl], y1[sl], xo_pre[sl], sm);
        __syncthreads();
    }
    if (fin != 0u) {
        stores_done();
        __syncthreads();
        if (tau < nseg && ((fin >> tau) & 1u)) st_dev32(p.flag + gA + tau, ep);
    }
    stamp(a, l, ev0 + 3);
    return true;
}

// ---- attention item: (kv head h, request b, chunk c of CH keys) -------------------------------------
template <int D>
__device__ bool attn_item(const FusedArgs &a, int li, int l, int item, Smem<D> &sm) {
#pragma clang fp contract(off)
    constexpr int NPL = (kCHS / 16) * 4 * D / kFT;   // 16-byte staging loads per thread (most)
    const int c = item % a.n_chunks, hb = item / a.n_chunks;
    const int b = hb % a.B, h = hb / a.B;
    const uint32_t ep = (uint32_t)l + 1;
    const int gq = a.nq / a.nkv;
    const int st_b = a.status[b];
    const int ctx = a.ctx_len[b];
    const int T = ctx + a.K;
    const int kb = c * a.CH;
    const int tau = threadIdx.x, lane = tau & 63, wave = tau >> 6;
    if (st_b != 0 || kb >= T) {
        // nothing to attend (a failed request, or a chunk past this request's keys); the epoch
        // is still published, after this layer's q, k and v exist like for any other item
        publish<D>(a.f_att + item, ep);
        __syncthreads();
        return true;
    }
    const int nvalid = min(a.CH, T - kb);
    const int npages = (nvalid + 15) >> 4;
    const int nst = (nvalid + 31) >> 5;           // steps holding valid keys
    const int64_t lofs = (int64_t)(a.L0 + li) * a.layer_stride;
    const bf16 *kpool = a.k_pool + lofs, *vpool = a.v_pool + lofs;
    const int32_t *bt = a.block_table + (int64_t)b * a.max_pages;
    // staging slots: 16-byte slot q of the chunk's first 2 * nst pages (whole 32-key steps) is
    // page q / (4D), then K slot (< 2D) or V slot; pages past the valid ones are zero
    bf16x8 kv[NPL];
    const int nslots = 2 * nst * 4 * D;
    // pages that hold only committed context first (plain loads), before waiting for q, k, v
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int q = tau + i * kFT;
        kv[i] = bf16x8{};
        const int p = q / (4 * D), s4 = q % (4 * D);
        if (q < nslots && p < npages && kb + 16 * p + 16 <= ctx) {
            const bool is_v = s4 >= 2 * D;
            const int page = bt[(kb >> 4) + p];
            kv[i] = stream_load((const bf16x8 *)((is_v ? vpool : kpool) + ((int64_t)page * a.nkv + h) * 16 * D +
                                                 (is_v ? s4 - 2 * D : s4) * 8));
        }
    }
    // this layer's q of the group's heads and the draft K/V rows of head h
    {
        const int gph = D / 64;
        const uint32_t *fq = a.ph[FUSED_QKV].flag;
        if (!wait_ranges<D>(fq + h * gq * gph, gq * gph, fq + (a.nq + h) * gph, gph,
                            fq + (a.nq + a.nkv + h) * gph, gph, ep, a.err, sm))
            return false;
    }
    stamp(a, li + a.L0, 18);
    // tasks: (query tile t, key part kp), at most one per wave; tile columns rho = (q head of the
    // group, node); a part covers whole 32-key steps of the valid ones. The task's query rows
    // are requested first, ahead of the draft rows' keys and values.
    const int R = gq * a.K;
    const int T_ = (R + 15) >> 4;                 // <= 8 (at most 8 q heads per kv head)
    const int KP = kFW / T_;
    const int ntask = T_ * KP;
    const int r16 = lane & 15, grp = lane >> 4;
    const bool has = wave < ntask;
    const int t = has ? wave % T_ : 0, kp = has ? wave / T_ : 0;
    const int s_lo = kp * nst / KP, s_hi = (kp + 1) * nst / KP;
    constexpr int MS = kCHS / 32;
    const int rho = 16 * t + r16;
    const bool col_ok = rho < R;
    const int hh = col_ok ? rho / a.K : 0, node = col_ok ? rho % a.K : 0;
    bf16x8 qf[D / 32];
    uint64_t am = 0;
    if (has) {
        const int qrow = (b * a.K + node) * a.nq + h * gq + hh;
#pragma unroll
        for (int ds = 0; ds < D / 32; ++ds)
            qf[ds] = *(const bf16x8 *)(q_of(a, li) + (int64_t)qrow * D + ds * 32 + grp * 8);
        am = a.anc[b * a.K + node];
    }
    floatx4 o[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    float mloc = -INFINITY, psum = 0.f;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int q = tau + i * kFT;
        const int p = q / (4 * D), s4 = q % (4 * D);
        if (q < nslots && p < npages && kb + 16 * p + 16 > ctx) {
            const bool is_v = s4 >= 2 * D;
            const int page = bt[(kb >> 4) + p];
            kv[i] = *(const bf16x8 *)((is_v ? vpool : kpool) + ((int64_t)page * a.nkv + h) * 16 * D +
                                      (is_v ? s4 - 2 * D : s4) * 8);
        }
    }
    // into LDS: keys [key][D + 8]; values transposed [d][CHS + 8], slots past the valid keys zero
    constexpr int KP_ = D + 8, VP_ = kCHS + 8;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int q = tau + i * kFT;
        if (q < nslots) {
            const int p = q / (4 * D), s4 = q % (4 * D);
            if (s4 < 2 * D) {
                const int r = s4 / (D / 8), col = (s4 % (D / 8)) * 8;
                *(bf16x8 *)&sm.u.kv.ks[(16 * p + r) * KP_ + col] = kv[i];
            } else {
                const int sl = s4 - 2 * D;
                const int d = sl >> 1, half = sl & 1;
                bf16x8 v = kv[i];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (16 * p + 8 * half + j >= nvalid) v[j] = (bf16)0.0f;
                *(bf16x8 *)&sm.u.kv.vt[d * VP_ + 16 * p + 8 * half] = v;
            }
        }
    }
    __syncthreads();
    stamp(a, li + a.L0, 19);

    if (has) {
        const int kr0 = 8 * (r16 >> 2) + (r16 & 3);
        const int nps = s_hi - s_lo;
        floatx4 s[MS][2];
#pragma unroll
        for (int st = 0; st < MS; ++st) {
            if (st >= nps) break;
            const int ks0 = (s_lo + st) * 32;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ds = 0; ds < D / 32; ++ds) {
                    const bf16x8 kf = *(const bf16x8 *)&sm.u.kv.ks[(ks0 + kr0 + 4 * hf) * KP_ + grp * 8 + ds * 32];
                    acc = mfma16x16x32(kf, qf[ds], acc);
                }
                s[st][hf] = acc;
            }
        }
        // masked log2-domain softmax over the part's keys: committed positions always visible,
        // draft position ctx + j when node j is on this column's root path
        float sv[MS][8];
#pragma unroll
        for (int st = 0; st < MS; ++st) {
            if (st >= nps) break;
            const int k0 = kb + (s_lo + st) * 32 + 8 * grp;
            const int n_ctx = min(max(ctx - k0, 0), 8);
            const int j0 = max(k0 + n_ctx - ctx, 0);
            const unsigned anc8 = j0 < 64 ? (unsigned)(am >> j0) & 0xffu : 0u;
            const int n_in = min(max(kb + nvalid - k0, 0), 8);
            unsigned vis = (((1u << n_ctx) - 1u) | (anc8 << n_ctx)) & ((1u << n_in) - 1u);
            if (!col_ok) vis = 0u;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float raw = (e < 4 ? s[st][0][e] : s[st][1][e - 4]) * a.scale_log2;
                sv[st][e] = ((vis >> e) & 1u) ? raw : -INFINITY;
                mloc = fmaxf(mloc, sv[st][e]);
            }
        }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
        const bool none = mloc == -INFINITY;
        bf16x8 ph[MS], pl[MS];
#pragma unroll
        for (int st = 0; st < MS; ++st) {
            if (st >= nps) break;
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
#pragma unroll
        for (int st = 0; st < MS; ++st) {
            if (st >= nps) break;
            const int ks0 = (s_lo + st) * 32;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                const bf16x8 vf = *(const bf16x8 *)&sm.u.kv.vt[(16 * dt + r16) * VP_ + ks0 + grp * 8];
                o[dt] = mfma16x16x32(vf, ph[st], o[dt]);
                o[dt] = mfma16x16x32(vf, pl[st], o[dt]);
            }
        }
    }
    stamp(a, li + a.L0, 20);
    if (KP == 1) {
        if (has) {
            const int64_t base = ((int64_t)item * T_ + t) * 16 + r16;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt)
                st_dev16B(a.att_o, (uint32_t)((base * D + dt * 16 + 4 * grp) * 4), o[dt]);
            if (grp == 0) st_dev64(a.att_ml + base, pack2f(mloc, psum));
        }
    } else {
        __syncthreads();   // every task has read its keys and values: LDS takes the parts
        if (has) {
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) sm.u.mrg.o[(wave * (D / 16) + dt) * 64 + lane] = o[dt];
            if (grp == 0) {
                sm.u.mrg.m[wave * 16 + r16] = mloc;
                sm.u.mrg.l[wave * 16 + r16] = psum;
            }
        }
        __syncthreads();
        // merge each tile's key parts in part order: thread -> (tile, column, dims quad)
        for (int e = tau; e < T_ * 16 * (D / 4); e += kFT) {
            const int tt = e / (16 * (D / 4)), r = e % (16 * (D / 4));
            const int col = r % 16, dq4 = r / 16;           // dims 4 dq4 .. 4 dq4 + 3
            const int dt = dq4 / 4, g4 = dq4 % 4;            // MFMA lane of (col, dims): 16 g4 + col
            float mx = -INFINITY;
            for (int k2 = 0; k2 < KP; ++k2) mx = fmaxf(mx, sm.u.mrg.m[(k2 * T_ + tt) * 16 + col]);
            float lsum = 0.f;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int k2 = 0; k2 < KP; ++k2) {
                const int w = k2 * T_ + tt;
                const float mk = sm.u.mrg.m[w * 16 + col];
                if (mk == -INFINITY) continue;
                const float sw = exp2f(mk - mx);
                lsum += sm.u.mrg.l[w * 16 + col] * sw;
                acc += sm.u.mrg.o[(w * (D / 16) + dt) * 64 + 16 * g4 + col] * sw;
            }
            const int64_t base = ((int64_t)item * T_ + tt) * 16 + col;
            st_dev16B(a.att_o, (uint32_t)((base * D + 16 * dt + 4 * g4) * 4), acc);
            if (dq4 == 0) st_dev64(a.att_ml + base, pack2f(mx, lsum));
        }
    }
    publish<D>(a.f_att + item, ep);
    __syncthreads();
    return true;
}

// ---- merge task: (kv head h, request b, tile t, quarter dq of the head's dims) ---------------------
template <int D>
__device__ bool combine_task(const FusedArgs &a, int li, int l, int task, Smem<D> &sm) {
#pragma clang fp contract(off)
    const int dq = task & 3, rest = task >> 2;
    const int gq = a.nq / a.nkv;
    const int R = gq * a.K, T_ = (R + 15) >> 4;
    const int t = rest % T_, hb = rest / T_;
    const int b = hb % a.B, h = hb / a.B;
    const uint32_t ep = (uint32_t)l + 1;
    if (!wait_all(a.f_att + (int64_t)hb * a.n_chunks, a.n_chunks, ep, a.err, sm)) return false;
    stamp(a, l, 21);
    const int tau = threadIdx.x;
    constexpr int TPC = D / 8;                  // threads per column, two dims each
    if (tau < 16 * TPC) {
        const int col = tau / TPC, dp = tau % TPC;
        const int d = dq * (D / 4) + 2 * dp;
        const int rho = 16 * t + col;
        if (rho < R) {
            const int hh = rho / a.K, node = rho % a.K;
            const int m = b * a.K + node, head = h * gq + hh;
            float o0 = 0.f, o1 = 0.f, lsum = 0.f;
            if (a.status[b] == 0) {
                const int nc = (a.ctx_len[b] + a.K + a.CH - 1) / a.CH;
                float mx = -INFINITY;
                // chunk partials requested 16 at a time
                for (int c0 = 0; c0 < nc; c0 += 16) {
                    uint64_t ml[16], ov[16];
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int c = min(c0 + i, nc - 1);
                        const int64_t base = ((int64_t)(hb * a.n_chunks + c) * T_ + t) * 16 + col;
                        ml[i] = ld_dev64(a.att_ml + base);
                        ov[i] = ld_dev64(a.att_o + base * D + d);
                    }
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        if (c0 + i >= nc) break;
                        const float mk = lo_f(ml[i]), lk = hi_f(ml[i]);
                        if (mk == -INFINITY) continue;
                        const float mn = fmaxf(mx, mk);
                        const float sa = exp2f(mx - mn), sw = exp2f(mk - mn);
                        lsum = lsum * sa + lk * sw;
                        o0 = o0 * sa + lo_f(ov[i]) * sw;
                        o1 = o1 * sa + hi_f(ov[i]) * sw;
                        mx = mn;
                    }
                }
                o0 = o0 / lsum;
                o1 = o1 / lsum;
            }
            st_dev32(ao_of(a, li) + frag_off(m, head * D + d, a.nq * D), pack2bf(o0, o1));
        }
    }
    stamp(a, l, 22);
    publish<D>(a.f_comb + task, ep);
    __syncthreads();
    return true;
}

// ---- the persistent kernel ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kFT, 1) void fused_layers_kernel(FusedArgs a) {
    __shared__ Smem<D> sm;
    for (int li = 0; li < a.nl; ++li) {
        const int l = a.L0 + li;
        if (!gemm_phase<FUSED_QKV, 2, D>(a, li, l, sm)) return;
        for (int it = blockIdx.x; it < a.n_items; it += gridDim.x)
            if (!attn_item<D>(a, li, l, it, sm)) return;
        stamp(a, l, 4);
        for (int tk = (int)gridDim.x - 1 - (int)blockIdx.x; tk < a.n_tasks; tk += gridDim.x)
            if (!combine_task<D>(a, li, l, tk, sm)) return;
        stamp(a, l, 5);
        if (!gemm_phase<FUSED_O, 2, D>(a, li, l, sm)) return;
        if (!gemm_phase<FUSED_GU, 4, D>(a, li, l, sm)) return;
        if (!gemm_phase<FUSED_DOWN, 2, D>(a, li, l, sm)) return;
    }
    if (a.L0 + a.nl == a.Lt) {
        // the output head's operand: u = RMSNorm(x) * final gain, fragment order, 16 rows
        const int nfrag = a.H / 32 * 64;
        if ((int)blockIdx.x * kFT >= nfrag) return;
        if (!wait_all(a.ph[FUSED_DOWN].flag, a.ph[FUSED_DOWN].groups, (uint32_t)a.Lt, a.err, sm)) return;
        if (threadIdx.x < 16) {
            float s = 0.f;
            for (int gg = 0; gg < a.H / 64; ++gg) s += ld_devf(a.ssq_d + gg * 16 + threadIdx.x);
            sm.rs[threadIdx.x] = 1.0f / sqrtf(s / (float)a.H + a.eps);
        }
        __syncthreads();
        const int fi = blockIdx.x * kFT + threadIdx.x;
        if (fi < nfrag) {
            const int s = fi / 64, ln = fi % 64;
            // device scope: this slot is also the launch's input, read (and cached) by its
            // first layer before the last layer rewrote it
            const bf16x8 x = ld_dev16(x_out(a, a.nl - 1), (uint32_t)(fi * 16));
            const bf16x8 g = *(const bf16x8 *)(a.g_final + s * 32 + 8 * (ln >> 4));
            *(bf16x8 *)(a.u_head + (int64_t)fi * 8) = norm_frag(x, sm.rs[ln & 15], g);
        }
    }
}

// ---- before the first launch: sync words and operands cleared, embedding rows ---------------------
// blocks 0..15: row m of x (fragment order; zero past the M rows), its per-group sums of squares
// and the trace's first row; blocks 16..: zero the sync words and the attention and SwiGLU operands.
__global__ __launch_bounds__(256) void fused_prep_kernel(FusedArgs a, const int32_t *__restrict__ tokens,
                                                         const bf16 *__restrict__ table, int vocab,
                                                         uint32_t *sync_words, int n_sync) {
    const int tid = threadIdx.x;
    if (blockIdx.x >= 16) {
        const int64_t stride = (int64_t)(gridDim.x - 16) * 256;
        const int64_t base = (int64_t)(blockIdx.x - 16) * 256 + tid;
        for (int64_t i = base; i < n_sync; i += stride) sync_words[i] = 0u;
        const int64_t nao = (int64_t)kFusedMaxLayers * 16 * a.nq * a.D / 2;
        const int64_t nh = (int64_t)kFusedMaxLayers * 16 * a.F / 2;
        for (int64_t i = base; i < nao; i += stride) reinterpret_cast<uint32_t *>(a.ao)[i] = 0u;
        for (int64_t i = base; i < nh; i += stride) reinterpret_cast<uint32_t *>(a.h)[i] = 0u;
        return;
    }
    __shared__ float part[256];
    const int m = blockIdx.x;
    int tok = m < a.M ? tokens[m] : -1;
    const bool live = m < a.M && tok >= 0 && tok < vocab;
    if (!live) tok = 0;
    const bf16 *src = table + (int64_t)tok * a.H;
    // thread tid: groups of 64 columns in turn, 4 columns per step of 16 threads
    for (int g0 = 0; g0 < a.H / 64; g0 += 16) {
        const int g = g0 + tid / 16;
        float ss = 0.f;
        if (g < a.H / 64) {
            const int col = 64 * g + 4 * (tid % 16);
            uint2 v = live ? *(const uint2 *)(src + col) : make_uint2(0u, 0u);
            if (m >= a.M) v = make_uint2(0u, 0u);
            *(uint2 *)(a.x_d + (int64_t)(kFusedMaxLayers - 1) * 16 * a.H + frag_off(m, col, a.H)) = v;
            if (a.trace != nullptr && m < a.M) *(uint2 *)(a.trace + (int64_t)m * a.H + col) = v;
            const float f0 = bf_lo(v.x), f1 = bf_hi(v.x), f2 = bf_lo(v.y), f3 = bf_hi(v.y);
            ss = ((f0 * f0 + f1 * f1) + f2 * f2) + f3 * f3;
        }
        part[tid] = ss;
        __syncthreads();
        if (tid % 16 == 0 && g < a.H / 64) {
            float s = 0.f;
            for (int i = 0; i < 16; ++i) s += part[tid + i];
            a.ssq_d[g * 16 + m] = s;
        }
        __syncthreads();
    }
}

}  // namespace

int fused_occupancy(int D) {
    int n = 0;
    hipError_t e = D == 128 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fused_layers_kernel<128>, kFT, 0)
                            : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fused_layers_kernel<64>, kFT, 0);
    return e == hipSuccess ? n : 0;
}

hipError_t fused_prep(const FusedArgs &a, const int32_t *tokens, const bf16 *embed, int vocab,
                      uint32_t *sync_words, int n_sync, hipStream_t st) {
    hipLaunchKernelGGL(fused_prep_kernel, dim3(16 + 64), dim3(256), 0, st, a, tokens, embed, vocab, sync_words,
                       n_sync);
    return hipGetLastError();
}

hipError_t fused_layers(const FusedArgs &a, hipStream_t st) {
    if (a.D == 128)
        hipLaunchKernelGGL(fused_layers_kernel<128>, dim3(a.G), dim3(kFT), 0, st, a);
    else
        hipLaunchKernelGGL(fused_layers_kernel<64>, dim3(a.G), dim3(kFT), 0, st, a);
    return hipGetLastError();
}

}  // namespace sv
