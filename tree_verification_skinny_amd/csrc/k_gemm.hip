// k_gemm.hip — weight-streaming skinny GEMM for the verify pass (M = draft nodes, 1..64 rows
// per launch) on gfx950 MFMA, with the split-K reduction and the consumer's elementwise work
// fused into its tail.
//
// At batch 1 the verify pass reads every target weight for a handful of tokens, so it is bound
// by HBM, not by arithmetic [SpecPilot digest, airadar.tv — summary paragraph]. The kernel is
// built around the weight stream:
//   * Y^T = W . X^T on v_mfma_f32_16x16x32_bf16. The weight is the A operand, and it is stored
//     pre-packed in MFMA fragment order (see spec_pack_weight): fragment (tile of 16 rows,
//     32-wide K step) is 1 KB, lane l's 16 bytes are W[16 tile + l%16][32 step + 8(l/16) .. +7],
//     and a tile's K steps follow each other. One 128-bit load per lane reads a whole fragment
//     as 1 KB of contiguous HBM, straight into the registers the MFMA consumes. The loads are
//     non-temporal (each weight byte is used once per pass), which measured 6 % faster over the
//     whole block-of-16 step than plain loads.
//   * The activations X [M][Kd] (cache resident, already normalised where an RMSNorm precedes
//     the projection) are the B operand, in the same fragment order (16-row blocks instead of
//     16-row tiles): the kernels that produce them write them that way, so an activation load
//     is one contiguous 1 KB read as well.
//   * A workgroup of W waves (4 or 8) owns NT weight tiles over a K range; its waves interleave
//     over the 32-wide K steps (so together they read each tile front to back) and add their
//     sums in LDS in wave order. Projections with few output columns split K over workgroups
//     and leave fp32 partials that a separate pass adds in split order (an in-kernel "last
//     workgroup adds" fixup for every column group costs more on this chip than the extra
//     pass); wide projections run whole and finish their epilogue in place, except that a
//     whole-K SwiGLU launch with a few more groups than its workgroups splits its leftover pairs
//     by K and lets the last of a pair's parts finish it (BAL, in both kernels). No workgroup
//     waits for another and results do not depend on timing.
//   * Epilogues of the whole-K projections: SwiGLU (gate/up; a group holds gate tiles and the
//     matching up tiles, so gate n and up n sit in the same lane) and the per-group greedy
//     maximum of the output head.
//   * The weights may instead come in W12, the lossless 12-bit layout of k_w12.hip (a lossless
//     12-bit format of three 4-bit planes rebuilt in registers [SpecPilot digest, airadar.tv —
//     "Reasons"]): a quarter fewer bytes to stream. Each fragment is rebuilt to bf16 in
//     registers (w12_decode), exceptions are written over it (w12_fixup), and the products,
//     their order and the epilogues are the bf16 kernel's, so results are bit-identical.
// MFMA lane layout (16x16x32): lane l supplies A row l%16, K elements 8*(l/16)..+7, and B
// column l%16, the same K elements; it receives D rows 4*(l/16)..+3 of column l%16.
#include <type_traits>

#include "kernels.hpp"

#ifndef SV_W12_U
#define SV_W12_U 2                // K steps per batch over W12 weights, split-K projections
#endif
#ifndef SV_W12_U_WHOLE
#define SV_W12_U_WHOLE 2          // the same for whole-K projections (SwiGLU, output head)
#endif
#ifndef SV_W12_WHOLE_WAVES
#define SV_W12_WHOLE_WAVES 8      // waves per workgroup of the whole-K projections over W12
#endif

namespace sv {

// ---- packing ------------------------------------------------------------------------------------
// Row-major [n][kd] -> fragment order (frag_off), rows past n (up to the next multiple of 16)
// zero. One thread per 16-byte slot (block, step, lane).
__global__ __launch_bounds__(256) void pack_kernel(const bf16 *__restrict__ w, int n, int kd,
                                                   bf16 *__restrict__ out) {
    const int64_t steps = kd / 32;
    const int64_t total = (int64_t)((n + 15) / 16) * steps * 64;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int lane = (int)(i & 63);
        const int64_t frag = i >> 6;
        const int64_t tile = frag / steps, step = frag % steps;
        const int64_t row = tile * 16 + (lane & 15);
        const int64_t col = step * 32 + 8 * (lane >> 4);
        bf16x8 v = {};
        if (row < n) v = *(const bf16x8 *)(w + row * kd + col);
        *(bf16x8 *)(out + i * 8) = v;
    }
}

hipError_t pack_weight(const bf16 *w, int n, int kd, bf16 *out, hipStream_t st) {
    const int64_t total = (int64_t)((n + 15) / 16) * (kd / 32) * 64;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, st, w, n, kd, out);
    return hipGetLastError();
}

// ---- column layout of a tile group --------------------------------------------------------------
// Contiguous for plain outputs; paired halves for SwiGLU (gate column n with up column F + n) and
// for QKV (column i of a head with column i + D/2, its rotation partner; D in the F argument) so
// that a lane holds both operands of its outputs.
template <int NT, int EPI>
__device__ __forceinline__ int tile_col(int ng, int t, int F) {
    if constexpr (EPI == EPI_SWIGLU) {
        constexpr int PH = 8 * NT;   // columns in each half of a paired group
        return t < NT / 2 ? ng * PH + 16 * t : F + ng * PH + 16 * (t - NT / 2);
    } else if constexpr (EPI == EPI_QKV) {
        static_assert(NT == 2, "a QKV group is one 16-column tile and its rotation partner");
        const int pph = F / 32;      // groups per head
        return (ng / pph) * F + 16 * (ng % pph) + t * (F / 2);
    } else {
        return ng * 16 * NT + 16 * t;
    }
}

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;

// The QKV epilogue's rotation of a pair (a, c) = (x_i, x_{i + D/2}), both already rounded to bf16,
// by the angle of (cos, sin) = cs, each output rounded to bf16 (no contraction, the arithmetic of
// the split-K pass it replaces).
__device__ __forceinline__ void rope_pair(float a, float c, float2 cs, bf16 &lo, bf16 &hi) {
#pragma clang fp contract(off)
    lo = (bf16)(a * cs.x - c * cs.y);
    hi = (bf16)(c * cs.x + a * cs.y);
}

// ---- W12 weights (k_w12.hip) ----------------------------------------------------------------------
// Lane l's three dwords of a fragment (low bytes of v0..v3, of v4..v7, and the nibbles) back
// to its 8 bf16 values: a pair's low bytes by one byte permute, its high bytes as
// (sign << 7) | (b/2 + nibble bits 0..2) from the pair's two nibbles shifted under them. cb holds
// b/2 in both high bytes; b/2 + 7 <= 127, so the add never reaches the sign bit.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t w12_hi(uint32_t x, uint32_t cb) {
    return ((x & 0x07000700u) + cb) | ((x & 0x08000800u) << 4);
}

__device__ __forceinline__ bf16x8 w12_decode(uint32_t l0, uint32_t l1, uint32_t h, uint32_t cb) {
    u32x4 d;
    d.x = __builtin_amdgcn_perm(0u, l0, 0x0c010c00u) | w12_hi((h << 8) & 0x0f000f00u, cb);
    d.y = __builtin_amdgcn_perm(0u, l0, 0x0c030c02u) | w12_hi((h << 4) & 0x0f000f00u, cb);
    d.z = __builtin_amdgcn_perm(0u, l1, 0x0c010c00u) | w12_hi(h & 0x0f000f00u, cb);
    d.w = __builtin_amdgcn_perm(0u, l1, 0x0c030c02u) | w12_hi((h >> 4) & 0x0f000f00u, cb);
    return __builtin_bit_cast(bf16x8, d);
}

// An exception (pos = step * 512 + lane * 8 + j, bf16 bits) written over value j of its lane.
__device__ __forceinline__ bf16x8 w12_patch(bf16x8 a, int lane, int pos, int val) {
    u32x4 d = __builtin_bit_cast(u32x4, a);
    const int j = pos & 7;
    const bool me = lane == ((pos >> 3) & 63);
    const uint32_t sh = (uint32_t)(j & 1) * 16u;
    const uint32_t m = 0xffffu << sh, nv = ((uint32_t)val & 0xffffu) << sh;
    switch (j >> 1) {
        case 0: d.x = me ? ((d.x & ~m) | nv) : d.x; break;
        case 1: d.y = me ? ((d.y & ~m) | nv) : d.y; break;
        case 2: d.z = me ? ((d.z & ~m) | nv) : d.z; break;
        default: d.w = me ? ((d.w & ~m) | nv) : d.w; break;
    }
    return __builtin_bit_cast(bf16x8, d);
}

__device__ __forceinline__ uint32_t stream_load32(const uint32_t *p) { return __builtin_nontemporal_load(p); }

// A wave's window on one tile's exception list: lane l holds entry i + l (a sentinel past the
// tile's end), so the entries of a step are found with one compare and a ballot, without a load.
struct W12Cursor {
    int i, end, step;   // first entry of the window, end of the tile's entries, the next step
                        // with an entry (wave-uniform; INT_MAX or beyond any step: none)
    int x, y;           // this lane's entry: pos (step * 512 + lane * 8 + j) and bf16 bits
};

__device__ __forceinline__ int w12_step_of(const int2 *exc, int i, int end) {
    return i < end ? (exc[i].x >> 9) : 0x7fffffff;
}

// Place a cursor on the first of the tile's entries [i, end) at or after step s0. The wave's
// 64 lanes test 64 entries per round (one round unless the split starts more than 64 entries
// into the tile), instead of walking the list one dependent load at a time.
__device__ __forceinline__ int w12_first_at(const int2 *exc, int i, int end, int s0, int lane, int st) {
    while (true) {
        const unsigned long long m = __ballot(st >= s0);
        if (m != 0ull) return min(i + __ffsll((long long)m) - 1, end);
        i += 64;
        const int k = i + lane;
        st = k < end ? (exc[k].x >> 9) : 0x7fffffff;
    }
}

// Load the window at entry c.i and the step of its first entry.
__device__ __forceinline__ void w12_win_load(W12Cursor &c, const int2 *exc, int lane) {
    const int k = c.i + lane;
    const int2 e = k < c.end ? exc[k] : make_int2(0x7fffffff, 0);
    c.x = e.x;
    c.y = e.y;
    c.step = __builtin_amdgcn_readfirstlane(e.x) >> 9;
}

// Apply the tile's exceptions that fall on step su (wave-uniform, never decreasing from call to
// call; callers test su >= c.step first) to fragment a, and set c.step to the next step with an
// entry. Entries of other steps (the other waves' or earlier ones) are passed over in registers;
// the window moves on by 64 entries only once all of its entries lie at or before step su.
__device__ __forceinline__ bf16x8 w12_fixup(bf16x8 a, W12Cursor &c, const int2 *exc, int su, int lane) {
    while (true) {
        unsigned long long m = __ballot((c.x >> 9) == su);
        while (m != 0ull) {
            const int b = __builtin_ctzll(m);
            m &= m - 1ull;
            a = w12_patch(a, lane, __builtin_amdgcn_readlane(c.x, b), __builtin_amdgcn_readlane(c.y, b));
        }
        // entries sort by step: the first lane past su holds the next step (a sentinel: none)
        const unsigned long long after = __ballot((c.x >> 9) > su);
        if (after != 0ull) {
            c.step = __builtin_amdgcn_readlane(c.x, __builtin_ctzll(after)) >> 9;
            return a;
        }
        if (c.i + 64 < c.end) {
            c.i += 64;
            w12_win_load(c, exc, lane);
            continue;
        }
        c.step = 0x7fffffff;
        return a;
    }
}

// SwiGLU of four gate and up sums (each rounded to bf16 first), stored as bf16 at h + off.
__device__ __forceinline__ void swiglu_store4(bf16 *h, int64_t off, const floatx4 &g4, const floatx4 &u4) {
    float hv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float g = round_bf(g4[j]);
        const float u = round_bf(u4[j]);
        hv[j] = (g / (1.0f + expf(-g))) * u;
    }
    store4(h + off, hv[0], hv[1], hv[2], hv[3]);
}

// The last arriver of a balanced launch: the sum of parts slot0 .. slot0 + Q - 1 (index order:
// part 0, then + part 1, ...) of NV floatx4 values per lane, each part's values at scratch slot
// ((slot * NV + v) * 64 + lane) as two 64-bit halves, read with agent-scope loads. QC parts'
// loads go out together (Q a multiple of QC), so Q parts take Q / QC round trips, not Q.
template <int NV, int QC>
__device__ __forceinline__ void bal_add_parts(floatx4 (&sum)[NV], const uint64_t *scr, int slot0, int Q, int lane) {
    for (int q0 = 0; q0 < Q; q0 += QC) {
        uint64_t a[QC][NV], b[QC][NV];
#pragma unroll
        for (int j = 0; j < QC; ++j)
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const uint64_t *sp = scr + (((int64_t)(slot0 + q0 + j) * NV + v) * 64 + lane) * 2;
                a[j][v] = __hip_atomic_load(const_cast<uint64_t *>(sp), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                b[j][v] = __hip_atomic_load(const_cast<uint64_t *>(sp + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
        for (int j = 0; j < QC; ++j)
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const floatx4 x = {__uint_as_float((uint32_t)a[j][v]), __uint_as_float((uint32_t)(a[j][v] >> 32)),
                                   __uint_as_float((uint32_t)b[j][v]), __uint_as_float((uint32_t)(b[j][v] >> 32))};
                sum[v] = q0 + j == 0 ? x : sum[v] + x;
            }
    }
}

// Q is a power of two (a divisor of the launch's workgroup count): whole batches of up to 64
// registers of loads.
template <int NV>
__device__ __forceinline__ void bal_sum(floatx4 (&sum)[NV], const uint64_t *scr, int slot0, int Q, int lane) {
    constexpr int QC = 16 / NV > 1 ? 16 / NV : 1;
    if (Q % QC == 0) bal_add_parts<NV, QC>(sum, scr, slot0, Q, lane);
    else bal_add_parts<NV, 1>(sum, scr, slot0, Q, lane);
}

template <int NT, int MT>
struct Acc {
    floatx4 v[NT][MT];
};

// BAL (SwiGLU over one block of rows, GemmShape::bal_q = Q, bal_wg workgroups, two per compute
// unit): workgroup b runs group b over all of K on its W waves as above and, on one more wave,
// part b % Q of the K range of leftover gate/up pair (NT / 2) * n_groups + b / Q. The part's sums
// go to scratch (ep.y); the last of the pair's Q workgroups to arrive (ep.ctr) adds the parts in
// index order, applies SwiGLU and resets the counter. The part wave's loads and hand-off overlap
// the group's stream. Nothing waits on another workgroup.
template <int NT, int MT, int W, int EPI, bool W12, bool BAL = false>
__global__ __launch_bounds__(64 * (W + (BAL ? 1 : 0))) void gemm_kernel(GemmIn in, const bf16 *__restrict__ Wp,
                                                      W12Ref w12, int N, int Kd, int n_groups,
                                                      int ksteps, GemmEpi ep) {
    static_assert(!BAL || (EPI == EPI_SWIGLU && MT == 1), "balanced launch: SwiGLU over one block of rows");
    __shared__ floatx4 red[(W - 1) * NT * MT * 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, grp = lane >> 4;
    const int ng = blockIdx.x % n_groups;
    const int split = blockIdx.x / n_groups;
    const int S = Kd >> 5;
    const int s_begin = split * ksteps;
    const int s_end = min(s_begin + ksteps, S);
    const int M = in.M;            // rows in this launch (a chunk of at most 64)
    const int m0 = in.m0;          // first global row of the chunk

    const bf16 *wp[NT];
    const uint32_t *qp[NT];          // W12: lane's 12 bytes in the tile's first fragment
    W12Cursor cur[NT];
    uint32_t cb = 0;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    if constexpr (W12) cb = (uint32_t)(w12.plan[0] >> 1) * 0x01000100u;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int tile = tile_col<NT, EPI>(ng, t, EPI == EPI_QKV ? ep.D : ep.F) >> 4;
        if constexpr (W12) {
            qp[t] = w12.planes + ((int64_t)tile * S) * 192 + 3 * lane;
            cur[t].i = w12.plan[2 + tile];
            cur[t].end = w12.plan[3 + tile];
        } else {
            wp[t] = Wp + (((int64_t)tile * S) * 64 + lane) * 8;
        }
    }
    if constexpr (W12) {
        // cursors at the wave's first step: every tile's first 64 entries are tested at once
        int st[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int k = cur[t].i + lane;
            st[t] = k < cur[t].end ? (w12.exc[k].x >> 9) : 0x7fffffff;
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            cur[t].i = w12_first_at(w12.exc, cur[t].i, cur[t].end, s_begin + wv, lane, st[t]);
            w12_win_load(cur[t], w12.exc, lane);
        }
    }
    // activation blocks of this chunk; blocks past the last one (MT rounds the chunk up) re-read
    // it, and their columns are never stored
    const int nblk = (in.M_total + 15) >> 4;
    const bf16 *xp[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int blk = min((m0 >> 4) + mt, nblk - 1);
        xp[mt] = in.Xp + (((int64_t)blk * S) * 64 + lane) * 8;
    }

    if constexpr (BAL) {
        if (wv == W) {
            // the part wave: the leftover pair's steps sq0 .. sq0 + Sq - 1 in one chain, XB at a
            // time, then the hand-off; it meets the streaming waves at their one barrier
            constexpr int XB = 5;
            const int Q = ep.bal_q;
            const int lx = (int)blockIdx.x / Q, qi = (int)blockIdx.x % Q;
            const int pair = n_groups * (NT / 2) + lx;
            const int Sq = S / Q, sq0 = qi * Sq;
            const int tl[2] = {pair, ep.F / 16 + pair};
            const bf16 *xw[2];
            const uint32_t *xq[2];
            W12Cursor xc[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                if constexpr (W12) {
                    xq[t] = w12.planes + ((int64_t)tl[t] * S) * 192 + 3 * lane;
                    xc[t].i = w12.plan[2 + tl[t]];
                    xc[t].end = w12.plan[3 + tl[t]];
                } else {
                    xw[t] = Wp + (((int64_t)tl[t] * S) * 64 + lane) * 8;
                }
            }
            if constexpr (W12) {
                int st0[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int k = xc[t].i + lane;
                    st0[t] = k < xc[t].end ? (w12.exc[k].x >> 9) : 0x7fffffff;
                }
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    xc[t].i = w12_first_at(w12.exc, xc[t].i, xc[t].end, sq0, lane, st0[t]);
                    w12_win_load(xc[t], w12.exc, lane);
                }
            }
            floatx4 ex[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
            auto step = [&](const bf16x8 &xv, const bf16x8 (&f)[2], const uint32_t (&r0)[2],
                            const uint32_t (&r1)[2], const uint32_t (&rh)[2], int su) __attribute__((always_inline)) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    bf16x8 w;
                    if constexpr (W12) {
                        w = w12_decode(r0[t], r1[t], rh[t], cb);
                        if (su >= xc[t].step) w = w12_fixup(w, xc[t], w12.exc, su, lane);
                    } else {
                        w = f[t];
                    }
                    ex[t] = mfma16x16x32(w, xv, ex[t]);
                }
            };
            auto load = [&](bf16x8 &xv, bf16x8 (&f)[2], uint32_t (&r0)[2], uint32_t (&r1)[2], uint32_t (&rh)[2],
                            int su) __attribute__((always_inline)) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    if constexpr (W12) {
                        const uint32_t *fp = xq[t] + (int64_t)su * 192;
                        r0[t] = stream_load32(fp);
                        r1[t] = stream_load32(fp + 1);
                        rh[t] = stream_load32(fp + 2);
                    } else {
                        f[t] = stream_load((const bf16x8 *)(xw[t] + (int64_t)su * 512));
                    }
                }
                xv = *(const bf16x8 *)(xp[0] + (int64_t)su * 512);
            };
            // whole batches of XB steps: every load is used unconditionally, so all of a batch's
            // loads go out before its first product; then the steps left over one at a time
            int i0 = 0;
            for (; i0 + XB <= Sq; i0 += XB) {
                bf16x8 f[XB][2], xb[XB];
                uint32_t q0[XB][2], q1[XB][2], qh[XB][2];
#pragma unroll
                for (int u = 0; u < XB; ++u) load(xb[u], f[u], q0[u], q1[u], qh[u], sq0 + i0 + u);
#pragma unroll
                for (int u = 0; u < XB; ++u) step(xb[u], f[u], q0[u], q1[u], qh[u], sq0 + i0 + u);
            }
            for (; i0 < Sq; ++i0) {
                bf16x8 f[2], xv;
                uint32_t q0[2], q1[2], qh[2];
                load(xv, f, q0, q1, qh, sq0 + i0);
                step(xv, f, q0, q1, qh, sq0 + i0);
            }
            // Into scratch slot blockIdx.x, written through to device scope (64-bit agent-scope
            // stores); the wave waits for the stores to complete, then counts itself in, and the
            // last arriver reads the parts with agent-scope loads. No fence: this die's L2 is
            // neither written back nor invalidated.
            uint64_t *scr = reinterpret_cast<uint64_t *>(ep.y);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const floatx4 v = ex[t];
                uint64_t *d = scr + (((int64_t)blockIdx.x * 2 + t) * 64 + lane) * 2;
                __hip_atomic_store(d, (uint64_t)__float_as_uint(v[0]) | ((uint64_t)__float_as_uint(v[1]) << 32),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(d + 1, (uint64_t)__float_as_uint(v[2]) | ((uint64_t)__float_as_uint(v[3]) << 32),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_s_waitcnt(0);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            int prev = 0;
            if (lane == 0) prev = (int)__hip_atomic_fetch_add(ep.ctr + lx, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            prev = __shfl(prev, 0, 64);
            if (prev == Q - 1) {
                // every part is written: add them in index order and finish the pair
                floatx4 sum[2];
                bal_sum<2>(sum, scr, lx * Q, Q, lane);
                if (r16 < M) swiglu_store4(ep.h, frag_off(m0 + r16, pair * 16 + 4 * grp, ep.F), sum[0], sum[1]);
                if (lane == 0) __hip_atomic_store(ep.ctr + lx, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();               // the streaming waves' one barrier (before their sums)
            return;
        }
    }

    Acc<NT, MT> acc;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc.v[t][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

    // K steps per batch; W12 fragments are 3/4 the bytes and need a deeper batch for the same
    // bytes in flight per wave
    constexpr int U16 = (NT * MT >= 8 || (W == 8 && NT * MT == 4)) ? 2 : 4;
    constexpr int U = W12 ? (NT * MT >= 8 ? 2 : (EPI == EPI_PARTIAL ? SV_W12_U : SV_W12_U_WHOLE)) : U16;
    int s = s_begin + wv;
    for (; s + W * (U - 1) < s_end; s += W * U) {
        bf16x8 a[U][NT], b[U][MT];
        uint32_t r0[U][NT], r1[U][NT], rh[U][NT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if constexpr (W12) {
                    const uint32_t *f = qp[t] + (int64_t)(s + W * u) * 192;
                    r0[u][t] = stream_load32(f);
                    r1[u][t] = stream_load32(f + 1);
                    rh[u][t] = stream_load32(f + 2);
                } else {
                    a[u][t] = stream_load((const bf16x8 *)(wp[t] + (int64_t)(s + W * u) * 512));
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) b[u][mt] = *(const bf16x8 *)(xp[mt] + (int64_t)(s + W * u) * 512);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if constexpr (W12) {
                    a[u][t] = w12_decode(r0[u][t], r1[u][t], rh[u][t], cb);
                    if (s + W * u >= cur[t].step) a[u][t] = w12_fixup(a[u][t], cur[t], w12.exc, s + W * u, lane);
                }
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc.v[t][mt] = mfma16x16x32(a[u][t], b[u][mt], acc.v[t][mt]);
            }
    }
    for (; s < s_end; s += W) {
        bf16x8 a[NT], b[MT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if constexpr (W12) {
                const uint32_t *f = qp[t] + (int64_t)s * 192;
                a[t] = w12_decode(stream_load32(f), stream_load32(f + 1), stream_load32(f + 2), cb);
                if (s >= cur[t].step) a[t] = w12_fixup(a[t], cur[t], w12.exc, s, lane);
            } else {
                a[t] = stream_load((const bf16x8 *)(wp[t] + (int64_t)s * 512));
            }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) b[mt] = *(const bf16x8 *)(xp[mt] + (int64_t)s * 512);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc.v[t][mt] = mfma16x16x32(a[t], b[mt], acc.v[t][mt]);
    }

    // ---- the waves' sums, in wave order ------------------------------------------------------
    if (wave > 0) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) red[((wave - 1) * NT * MT + t * MT + mt) * 64 + lane] = acc.v[t][mt];
    }
    __syncthreads();
    if (wave != 0) return;
    for (int w = 0; w < W - 1; ++w)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc.v[t][mt] += red[(w * NT * MT + t * MT + mt) * 64 + lane];

    int col[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) col[t] = tile_col<NT, EPI>(ng, t, EPI == EPI_QKV ? ep.D : ep.F) + 4 * grp;

    // ---- epilogues ------------------------------------------------------------------------------
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = 16 * mt + r16;
        const bool live = m < M;
        const int row = m0 + m;
        if constexpr (EPI == EPI_PARTIAL) {
            if (live) {
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    *(floatx4 *)(ep.y + ((int64_t)split * in.M_total + row) * N + col[t]) = acc.v[t][mt];
            }
        } else if constexpr (EPI == EPI_SWIGLU) {
            if (!live) continue;
#pragma unroll
            for (int t = 0; t < NT / 2; ++t) {
                // h in fragment order: the down projection's activation operand
                float hv[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float g = round_bf(acc.v[t][mt][j]);
                    const float u = round_bf(acc.v[t + NT / 2][mt][j]);
                    hv[j] = (g / (1.0f + expf(-g))) * u;
                }
                store4(ep.h + frag_off(row, col[t], ep.F), hv[0], hv[1], hv[2], hv[3]);
            }
        } else if constexpr (EPI == EPI_QKV) {
            // the sums rounded to bf16, q and k rotated, q stored, the draft K/V rows written into
            // the request's cache slot ctx_len + node
            if (!live) continue;
            const int D = ep.D, half = D / 2;
            const int hd = col[0] / D, i0 = col[0] % D;        // head; dims i0..i0+3 and + D/2
            bf16 lo[4], hi[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float a = round_bf(acc.v[0][mt][j]), c = round_bf(acc.v[1][mt][j]);
                if (hd < ep.nq + ep.nkv) {
                    rope_pair(a, c, ep.rope[(int64_t)row * half + i0 + j], lo[j], hi[j]);
                } else {
                    lo[j] = (bf16)a;
                    hi[j] = (bf16)c;
                }
            }
            if (hd < ep.nq) {
                bf16 *qh = ep.q + ((int64_t)row * ep.nq + hd) * D;
                *(bf16x4 *)(qh + i0) = bf16x4{lo[0], lo[1], lo[2], lo[3]};
                *(bf16x4 *)(qh + i0 + half) = bf16x4{hi[0], hi[1], hi[2], hi[3]};
                continue;
            }
            const int b = row / ep.K, il = row % ep.K;
            if (ep.status[b] != 0) continue;
            const int pos = ep.ctx_len[b] + il;
            const int64_t page = page_of(ep.block_table, ep.max_pages, b, pos);
            const int slot = pos & 15;
            if (hd < ep.nq + ep.nkv) {
                bf16 *kr = ep.k_pool + ((page * ep.nkv + (hd - ep.nq)) * 16 + slot) * D;
                *(bf16x4 *)(kr + i0) = bf16x4{lo[0], lo[1], lo[2], lo[3]};
                *(bf16x4 *)(kr + i0 + half) = bf16x4{hi[0], hi[1], hi[2], hi[3]};
            } else {
                bf16 *vr = ep.v_pool + ((page * ep.nkv + (hd - ep.nq - ep.nkv)) * D) * 16 + slot;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    vr[(i0 + j) * 16] = lo[j];
                    vr[(i0 + half + j) * 16] = hi[j];
                }
            }
        } else if constexpr (EPI == EPI_ARGMAX) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if (ep.logits != nullptr && live) *(floatx4 *)(ep.logits + (int64_t)row * N + col[t]) = acc.v[t][mt];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (better(acc.v[t][mt][j], col[t] + j, bv, bi)) { bv = acc.v[t][mt][j]; bi = col[t] + j; }
            }
#pragma unroll
            for (int o = 16; o < 64; o <<= 1) {
                const float ov = __shfl_xor(bv, o, 64);
                const int oi = __shfl_xor(bi, o, 64);
                if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
            }
            if (grp == 0 && live) {
                ep.amax_val[(int64_t)ng * in.M_total + row] = bv;
                ep.amax_idx[(int64_t)ng * in.M_total + row] = bi;
            }
        }
    }
}

// ---- wide variant (more than 16 rows): waves split the weight tiles, activations via LDS ---------
// With 32..64 rows each weight fragment meets up to four activation fragments, and reading those
// from L2 per wave would cost more than the weights themselves. Here the workgroup's 4 waves each
// own TN = 2 weight tiles over the whole K range of the workgroup, and the activation rows pass
// through LDS once per workgroup in slabs of KS K-steps (double-buffered), one barrier per slab.
// Each compute unit streams at a capped rate, so a launch lasts as long as its busiest unit: the
// plans keep one workgroup per unit, and the split-K and balanced launches run a slab loop
// without branches, which fetches the weight fragments one slab and the activation slabs two
// slabs ahead of their products.
#ifndef SV_SKINNY_TARGET
#define SV_SKINNY_TARGET 640                            // workgroups a split skinny launch aims at
#endif
#ifndef SV_TC_TARGET
#define SV_TC_TARGET 512                                // workgroups a split tile launch aims at
#endif
constexpr int kPlanCUs = 256;                           // compute units of the target (MI355X)
#ifndef SV_WIDE_PER_CU
#define SV_WIDE_PER_CU 1
#endif
#ifndef SV_WIDE_KS
#define SV_WIDE_KS 4
#endif
#ifndef SV_WIDE_TARGET
#define SV_WIDE_TARGET 320
#endif
#ifndef SV_WIDE_BAL
#define SV_WIDE_BAL 1
#endif
#ifndef SV_SKINNY_BAL
#define SV_SKINNY_BAL 1                                 // one-block gate/up balanced (plan_gemm_swiglu)
#endif
#ifndef SV_SKINNY_BAL_NT
#define SV_SKINNY_BAL_NT 4                              // tiles per group of a balanced launch
#endif
#ifndef SV_SKINNY_W8_MAX
#define SV_SKINNY_W8_MAX 1200                           // eight waves below this many skinny workgroups
#endif
#ifndef SV_SKINNY_BAL_PAD
#define SV_SKINNY_BAL_PAD 55                            // KB of LDS a balanced workgroup claims
#endif
#ifndef SV_SKINNY_BAL_PER_CU
#define SV_SKINNY_BAL_PER_CU 2                          // its workgroups per compute unit
#endif
#ifndef SV_WIDE_PIPE_PARTIAL
#define SV_WIDE_PIPE_PARTIAL 1                          // split-K launches on the branch-free loop
#endif
constexpr int kWideWaves = 4, kWideTN = 2, kWideKS = SV_WIDE_KS;

// output column of tile t (0..TN-1) of wave w in group ng: SwiGLU pairs gate and up columns in the
// same wave and lane
template <int EPI>
__device__ __forceinline__ int wide_col(int ng, int w, int t, int F) {
    if constexpr (EPI == EPI_SWIGLU) {
        return (t == 0 ? 0 : F) + (ng * kWideWaves + w) * 16;
    } else {
        return ((ng * kWideWaves + w) * kWideTN + t) * 16;
    }
}

// A weight fragment as loaded: bf16 operand, or a lane's 12 W12 bytes (decoded at use).
struct W12Raw {
    uint32_t a, b, c;
};

// BAL (SwiGLU over exactly one workgroup per compute unit, GemmShape::bal_q = Q): workgroup b runs
// group b's four pairs over all of K and, first, part b % Q of the K range of leftover pair
// 4 * n_groups + b / Q, its four waves taking every fourth step of that part. The part's sums go
// to scratch (ep.y); the last of the pair's Q workgroups to arrive (ep.ctr) adds the parts in
// index order, applies SwiGLU and resets the counter. Nothing waits on another workgroup.
template <int TM, int EPI, bool W12, bool BAL>
__global__ __launch_bounds__(64 * kWideWaves) void gemm_wide_kernel(GemmIn in, const bf16 *__restrict__ Wp,
                                                                     W12Ref w12, int N, int Kd, int n_groups,
                                                                     int ksteps, GemmEpi ep) {
    using Frag = typename std::conditional<W12, W12Raw, bf16x8>::type;
    constexpr int NW = kWideWaves, TN = kWideTN, KS = kWideKS;
    constexpr int SLOTS = KS * TM * 64;                 // 16-byte slots per slab
    constexpr int PER = SLOTS / (64 * NW);              // slots staged per thread
    static_assert(SLOTS % (64 * NW) == 0, "slab must split evenly over the threads");
    static_assert((NW - 1) * 2 <= 2 * KS, "the leftover part's wave sums must fit the staging buffers");
    __shared__ bf16x8 xs[2][SLOTS];                     // [buffer][(step * TM + block) * 64 + lane]
    __shared__ float red_v[NW][64];
    __shared__ int red_i[NW][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, grp = lane >> 4;
    const int ng = blockIdx.x % n_groups;
    const int split = blockIdx.x / n_groups;
    const int S = Kd >> 5;
    const int s_begin = split * ksteps;
    const int s_end = min(s_begin + ksteps, S);
    const int nsteps = s_end > s_begin ? s_end - s_begin : 0;
    const int nslabs = (nsteps + KS - 1) / KS;
    const int M = in.M, m0 = in.m0;
    const int nblk = (in.M_total + 15) >> 4;

    const bf16 *wp[TN];
    const uint32_t *qp[TN];          // W12: lane's 12 bytes in the tile's fragment at s_begin
    W12Cursor cur[TN];
    uint32_t cb = 0;
    if constexpr (W12) cb = (uint32_t)(w12.plan[0] >> 1) * 0x01000100u;
#pragma unroll
    for (int t = 0; t < TN; ++t) {
        const int tile = wide_col<EPI>(ng, wave, t, ep.F) >> 4;
        if constexpr (W12) {
            qp[t] = w12.planes + ((int64_t)tile * S + s_begin) * 192 + 3 * lane;
            cur[t].i = w12.plan[2 + tile];
            cur[t].end = w12.plan[3 + tile];
        } else {
            wp[t] = Wp + ((((int64_t)tile) * S + s_begin) * 64 + lane) * 8;
        }
    }
    if constexpr (W12) {
        int st[TN];
#pragma unroll
        for (int t = 0; t < TN; ++t) {
            const int k = cur[t].i + lane;
            st[t] = k < cur[t].end ? (w12.exc[k].x >> 9) : 0x7fffffff;
        }
#pragma unroll
        for (int t = 0; t < TN; ++t) {
            cur[t].i = w12_first_at(w12.exc, cur[t].i, cur[t].end, s_begin, lane, st[t]);
            w12_win_load(cur[t], w12.exc, lane);
        }
    }

    // staging: thread slot i = threadIdx.x + 256 r covers (step, block, lane) of the slab
    auto stage_load = [&](bf16x8 (&xr)[PER], int slab) {
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            const int i = threadIdx.x + r * 64 * NW;
            const int l = i & 63, mt = (i >> 6) % TM, k = (i >> 6) / TM;
            const int s = s_begin + slab * KS + k;
            const int blk = min((m0 >> 4) + mt, nblk - 1);
            xr[r] = s < s_end ? *(const bf16x8 *)(in.Xp + (((int64_t)blk * S + s) * 64 + l) * 8) : bf16x8{};
        }
    };
    auto stage_store = [&](const bf16x8 (&xr)[PER], int buf) {
#pragma unroll
        for (int r = 0; r < PER; ++r) xs[buf][threadIdx.x + r * 64 * NW] = xr[r];
    };
    auto w_load = [&](Frag (&a)[KS][TN], int slab) {
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            const int s = slab * KS + k;                 // relative to s_begin
#pragma unroll
            for (int t = 0; t < TN; ++t) {
                if constexpr (W12) {
                    const uint32_t *f = qp[t] + (int64_t)s * 192;
                    a[k][t] = s < nsteps ? W12Raw{stream_load32(f), stream_load32(f + 1), stream_load32(f + 2)}
                                         : W12Raw{0u, 0u, 0u};
                } else {
                    a[k][t] = s < nsteps ? stream_load((const bf16x8 *)(wp[t] + (int64_t)s * 512)) : bf16x8{};
                }
            }
        }
    };

    floatx4 acc[TN][TM];
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int mt = 0; mt < TM; ++mt) acc[t][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

    auto multiply = [&](const Frag (&a)[KS][TN], int buf, int slab) {
        const int kmax = min(KS, nsteps - slab * KS);
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            if (k < kmax) {
                bf16x8 b[TM];
#pragma unroll
                for (int mt = 0; mt < TM; ++mt) b[mt] = xs[buf][(k * TM + mt) * 64 + lane];
#pragma unroll
                for (int t = 0; t < TN; ++t) {
                    bf16x8 w;
                    if constexpr (W12) {
                        const int su = s_begin + slab * KS + k;
                        w = w12_decode(a[k][t].a, a[k][t].b, a[k][t].c, cb);
                        if (su >= cur[t].step) w = w12_fixup(w, cur[t], w12.exc, su, lane);
                    } else {
                        w = a[k][t];
                    }
#pragma unroll
                    for (int mt = 0; mt < TM; ++mt) acc[t][mt] = mfma16x16x32(w, b[mt], acc[t][mt]);
                }
            }
        }
    };

    if constexpr (BAL && EPI == EPI_SWIGLU) {
        constexpr int XB = 5;                            // steps per load batch of the part
        const int Q = ep.bal_q;
        const int xp = (int)blockIdx.x / Q, qi = (int)blockIdx.x % Q;
        const int pair = n_groups * NW + xp;
        const int Sq = S / Q, sq0 = qi * Sq;
        const int tl[2] = {pair, ep.F / 16 + pair};
        floatx4 ex[2][TM];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int mt = 0; mt < TM; ++mt) ex[t][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
        const bf16 *xw[2];
        const uint32_t *xq[2];
        W12Cursor xc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if constexpr (W12) {
                xq[t] = w12.planes + ((int64_t)tl[t] * S) * 192 + 3 * lane;
                xc[t].i = w12.plan[2 + tl[t]];
                xc[t].end = w12.plan[3 + tl[t]];
            } else {
                xw[t] = Wp + (((int64_t)tl[t] * S) * 64 + lane) * 8;
            }
        }
        if constexpr (W12) {
            int st0[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int k = xc[t].i + lane;
                st0[t] = k < xc[t].end ? (w12.exc[k].x >> 9) : 0x7fffffff;
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                xc[t].i = w12_first_at(w12.exc, xc[t].i, xc[t].end, sq0 + wave, lane, st0[t]);
                w12_win_load(xc[t], w12.exc, lane);
            }
        }
        const bf16 *xa[TM];
#pragma unroll
        for (int mt = 0; mt < TM; ++mt) {
            const int blk = min((m0 >> 4) + mt, nblk - 1);
            xa[mt] = in.Xp + (((int64_t)blk * S) * 64 + lane) * 8;
        }
        // this wave's steps: sq0 + wave + NW i, i < nmine; loaded XB at a time
        const int nmine = (Sq - wave + NW - 1) / NW;
        for (int i0 = 0; i0 < nmine; i0 += XB) {
            Frag f[XB][2];
            bf16x8 xb[XB][TM];
#pragma unroll
            for (int u = 0; u < XB; ++u) {
                const int su = sq0 + wave + NW * min(i0 + u, nmine - 1);
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    if constexpr (W12) {
                        const uint32_t *fp = xq[t] + (int64_t)su * 192;
                        f[u][t] = W12Raw{stream_load32(fp), stream_load32(fp + 1), stream_load32(fp + 2)};
                    } else {
                        f[u][t] = stream_load((const bf16x8 *)(xw[t] + (int64_t)su * 512));
                    }
                }
#pragma unroll
                for (int mt = 0; mt < TM; ++mt) xb[u][mt] = *(const bf16x8 *)(xa[mt] + (int64_t)su * 512);
            }
#pragma unroll
            for (int u = 0; u < XB; ++u) {
                if (i0 + u >= nmine) break;
                const int su = sq0 + wave + NW * (i0 + u);
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    bf16x8 w;
                    if constexpr (W12) {
                        w = w12_decode(f[u][t].a, f[u][t].b, f[u][t].c, cb);
                        if (su >= xc[t].step) w = w12_fixup(w, xc[t], w12.exc, su, lane);
                    } else {
                        w = f[u][t];
                    }
#pragma unroll
                    for (int mt = 0; mt < TM; ++mt) ex[t][mt] = mfma16x16x32(w, xb[u][mt], ex[t][mt]);
                }
            }
        }
        // the part's sum over the waves, in wave order, into scratch slot (xp * Q + qi)
        floatx4 *red = reinterpret_cast<floatx4 *>(&xs[0][0]);
        if (wave > 0) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int mt = 0; mt < TM; ++mt) red[(((wave - 1) * 2 + t) * TM + mt) * 64 + lane] = ex[t][mt];
        }
        __syncthreads();
        if (wave == 0) {
            // The part's sums are written through to device scope (64-bit agent-scope stores), the
            // wave waits for them to complete and counts itself in; the last arriver reads the
            // parts with agent-scope loads. No fence: the L2 of this die is neither written back
            // nor invalidated under the other workgroups' weight streams.
            uint64_t *scr = reinterpret_cast<uint64_t *>(ep.y);
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int mt = 0; mt < TM; ++mt) {
                    floatx4 v = ex[t][mt];
                    for (int w = 1; w < NW; ++w) v += red[(((w - 1) * 2 + t) * TM + mt) * 64 + lane];
                    uint64_t *d = scr + ((((int64_t)blockIdx.x * 2 + t) * TM + mt) * 64 + lane) * 2;
                    __hip_atomic_store(d, (uint64_t)__float_as_uint(v[0]) | ((uint64_t)__float_as_uint(v[1]) << 32),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(d + 1, (uint64_t)__float_as_uint(v[2]) | ((uint64_t)__float_as_uint(v[3]) << 32),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_s_waitcnt(0);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            int prev = 0;
            if (lane == 0) prev = (int)__hip_atomic_fetch_add(ep.ctr + xp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            prev = __shfl(prev, 0, 64);
            if (prev == Q - 1) {
                // every part is written: add them in index order and finish the pair
                floatx4 sum[2 * TM];                      // [t * TM + mt]
                bal_sum<2 * TM>(sum, scr, xp * Q, Q, lane);
#pragma unroll
                for (int mt = 0; mt < TM; ++mt) {
                    const int m = 16 * mt + r16;
                    if (m < M) swiglu_store4(ep.h, frag_off(m0 + m, pair * 16 + 4 * grp, ep.F), sum[mt], sum[TM + mt]);
                }
                if (lane == 0) __hip_atomic_store(ep.ctr + xp, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __syncthreads();
    }

    if constexpr (BAL || (EPI == EPI_PARTIAL && SV_WIDE_PIPE_PARTIAL)) {
        // A loop body without branches (over W12 weights, only the rare exception patch), so that
        // each wait covers only the loads it needs. Weight fragments are requested one slab ahead
        // and activation slabs two ahead (two register sets), at the top of each half, before the
        // multiply. Slabs run in pairs; steps past the range re-read the last step's addresses
        // (cache hits) and their staged activations are zero, so they add nothing.
        if (nslabs > 0) {
            Frag wa[KS][TN], wb[KS][TN];
            bf16x8 xa[PER], xb[PER];
            auto xload = [&](bf16x8 (&xr)[PER], int slab) {
#pragma unroll
                for (int r = 0; r < PER; ++r) {
                    const int i = threadIdx.x + r * 64 * NW;
                    const int l = i & 63, mt = (i >> 6) % TM, k = (i >> 6) / TM;
                    const int sc = min(s_begin + slab * KS + k, s_end - 1);
                    const int blk = min((m0 >> 4) + mt, nblk - 1);
                    xr[r] = *(const bf16x8 *)(in.Xp + (((int64_t)blk * S + sc) * 64 + l) * 8);
                }
            };
            auto xstore = [&](const bf16x8 (&xr)[PER], int buf, int slab) {
#pragma unroll
                for (int r = 0; r < PER; ++r) {
                    const int i = threadIdx.x + r * 64 * NW;
                    const int k = (i >> 6) / TM;
                    xs[buf][i] = s_begin + slab * KS + k < s_end ? xr[r] : bf16x8{};
                }
            };
            auto wload = [&](Frag (&w)[KS][TN], int slab) {
#pragma unroll
                for (int k = 0; k < KS; ++k) {
                    const int sr = min(slab * KS + k, nsteps - 1);
#pragma unroll
                    for (int t = 0; t < TN; ++t) {
                        if constexpr (W12) {
                            const uint32_t *f = qp[t] + (int64_t)sr * 192;
                            w[k][t] = W12Raw{stream_load32(f), stream_load32(f + 1), stream_load32(f + 2)};
                        } else {
                            w[k][t] = stream_load((const bf16x8 *)(wp[t] + (int64_t)sr * 512));
                        }
                    }
                }
            };
            auto mul = [&](const Frag (&w)[KS][TN], int buf, int slab) {
#pragma unroll
                for (int k = 0; k < KS; ++k) {
                    bf16x8 bx[TM];
#pragma unroll
                    for (int mt = 0; mt < TM; ++mt) bx[mt] = xs[buf][(k * TM + mt) * 64 + lane];
#pragma unroll
                    for (int t = 0; t < TN; ++t) {
                        bf16x8 wf;
                        if constexpr (W12) {
                            const int su = s_begin + slab * KS + k;
                            wf = w12_decode(w[k][t].a, w[k][t].b, w[k][t].c, cb);
                            if (su >= cur[t].step && su < s_end) wf = w12_fixup(wf, cur[t], w12.exc, su, lane);
                        } else {
                            wf = w[k][t];
                        }
#pragma unroll
                        for (int mt = 0; mt < TM; ++mt) acc[t][mt] = mfma16x16x32(wf, bx[mt], acc[t][mt]);
                    }
                }
            };
            xload(xa, 0);
            wload(wa, 0);
            xload(xb, 1);
            xstore(xa, 0, 0);
            __syncthreads();
            const int npairs = (nslabs + 1) >> 1;
            for (int pi = 0; pi < npairs; ++pi) {
                const int j = 2 * pi;
                wload(wb, j + 1);
                xload(xa, j + 2);
                __builtin_amdgcn_sched_barrier(0);
                mul(wa, 0, j);
                xstore(xb, 1, j + 1);
                __syncthreads();
                wload(wa, j + 2);
                xload(xb, j + 3);
                __builtin_amdgcn_sched_barrier(0);
                mul(wb, 1, j + 1);
                xstore(xa, 0, j + 2);
                __syncthreads();
            }
        }
    } else if (nslabs > 0) {
        Frag wa[KS][TN], wb[KS][TN];
        bf16x8 xr[PER];
        stage_load(xr, 0);
        w_load(wa, 0);
        stage_store(xr, 0);
        __syncthreads();
        // two slabs per iteration so that the register buffers are named statically
        for (int j = 0; j < nslabs; j += 2) {
            if (j + 1 < nslabs) { stage_load(xr, j + 1); w_load(wb, j + 1); }
            multiply(wa, 0, j);
            if (j + 1 < nslabs) stage_store(xr, 1);
            __syncthreads();
            if (j + 1 >= nslabs) break;
            if (j + 2 < nslabs) { stage_load(xr, j + 2); w_load(wa, j + 2); }
            multiply(wb, 1, j + 1);
            if (j + 2 < nslabs) stage_store(xr, 0);
            __syncthreads();
        }
    }

    // ---- epilogues (each wave owns its tiles' whole sums) -------------------------------------
    int col[TN];
#pragma unroll
    for (int t = 0; t < TN; ++t) col[t] = wide_col<EPI>(ng, wave, t, ep.F) + 4 * grp;
    float bv_all[TM];
    int bi_all[TM];
#pragma unroll
    for (int mt = 0; mt < TM; ++mt) {
        const int m = 16 * mt + r16;
        const bool live = m < M;
        const int row = m0 + m;
        bv_all[mt] = -INFINITY;
        bi_all[mt] = 0x7fffffff;
        if constexpr (EPI == EPI_PARTIAL) {
            if (live) {
#pragma unroll
                for (int t = 0; t < TN; ++t)
                    *(floatx4 *)(ep.y + ((int64_t)split * in.M_total + row) * N + col[t]) = acc[t][mt];
            }
        } else if constexpr (EPI == EPI_SWIGLU) {
            if (live) swiglu_store4(ep.h, frag_off(row, col[0], ep.F), acc[0][mt], acc[1][mt]);
        } else if constexpr (EPI == EPI_ARGMAX) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
#pragma unroll
            for (int t = 0; t < TN; ++t) {
                if (ep.logits != nullptr && live) *(floatx4 *)(ep.logits + (int64_t)row * N + col[t]) = acc[t][mt];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (better(acc[t][mt][j], col[t] + j, bv, bi)) { bv = acc[t][mt][j]; bi = col[t] + j; }
            }
#pragma unroll
            for (int o = 16; o < 64; o <<= 1) {
                const float ov = __shfl_xor(bv, o, 64);
                const int oi = __shfl_xor(bi, o, 64);
                if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
            }
            bv_all[mt] = bv;
            bi_all[mt] = bi;
        }
    }
    if constexpr (EPI == EPI_ARGMAX) {
        // the group's best per row over its 4 waves, in wave order
#pragma unroll
        for (int mt = 0; mt < TM; ++mt) {
            if (grp == 0) { red_v[wave][r16 + 16 * (mt & 3)] = bv_all[mt]; red_i[wave][r16 + 16 * (mt & 3)] = bi_all[mt]; }
            if ((mt & 3) == 3 || mt == TM - 1) {
                __syncthreads();
                if (wave == 0 && lane < 16 * ((mt & 3) + 1)) {
                    float bv = red_v[0][lane];
                    int bi = red_i[0][lane];
                    for (int w = 1; w < NW; ++w)
                        if (better(red_v[w][lane], red_i[w][lane], bv, bi)) { bv = red_v[w][lane]; bi = red_i[w][lane]; }
                    const int m = 16 * (mt & ~3) + lane;
                    if (m < M) {
                        ep.amax_val[(int64_t)ng * in.M_total + m0 + m] = bv;
                        ep.amax_idx[(int64_t)ng * in.M_total + m0 + m] = bi;
                    }
                }
                __syncthreads();
            }
        }
    }
}

static int mt_for(int m) { return m <= 16 ? 1 : (m <= 32 ? 2 : 4); }

int gemm_groups(const GemmShape &g) { return g.N / (16 * g.nt); }

// A balanced launch keeps one part (two tiles, every row block) per workgroup and counts arrivals
// per leftover pair: the wide launch on kPlanCUs workgroups of four row blocks with four pairs per
// group, the skinny one on bal_wg workgroups of one row block with NT / 2 pairs per group.
size_t gemm_bal_scratch_bytes(const GemmShape &g) {
    if (g.bal_q <= 0) return 0;
    return g.wide ? (size_t)kPlanCUs * 2 * 4 * 64 * sizeof(floatx4) : (size_t)g.bal_wg * 2 * 64 * sizeof(floatx4);
}

int gemm_bal_counters(const GemmShape &g) {
    if (g.bal_q <= 0) return 0;
    return g.wide ? 4 * (gemm_groups(g) - kPlanCUs) : (g.nt / 2) * (gemm_groups(g) - g.bal_wg);
}

// The weights: bf16 fragments (Wp) or, when w12.planes is set, a W12 matrix.
template <int NT, int MT, int W, int EPI>
static hipError_t launch(const GemmShape &g, const GemmIn &in, const bf16 *Wp, const W12Ref &w12,
                         const GemmEpi &ep, hipStream_t st) {
    const int steps = g.Kd >> 5;
    if constexpr (EPI == EPI_SWIGLU && (NT == 2 || NT == 4) && MT == 1 && W == 8) {
        if (g.bal_q > 0 && g.bal_wg > 0 && ep.ctr != nullptr && ep.y != nullptr) {
            GemmEpi eb = ep;
            eb.bal_q = g.bal_q;
            // two workgroups per compute unit, never three: unused LDS up to 55 KB a workgroup
            // keeps a third off a unit (160 KB) whatever the register count
            constexpr size_t kRed = (size_t)(W - 1) * NT * MT * 64 * sizeof(floatx4);
            constexpr size_t kPad = SV_SKINNY_BAL_PAD * 1024 > kRed ? SV_SKINNY_BAL_PAD * 1024 - kRed : 0;
            if (w12.planes != nullptr)
                hipLaunchKernelGGL((gemm_kernel<NT, MT, W, EPI, true, true>), dim3(g.bal_wg), dim3(64 * (W + 1)), kPad, st,
                                   in, Wp, w12, g.N, g.Kd, g.bal_wg, steps, eb);
            else
                hipLaunchKernelGGL((gemm_kernel<NT, MT, W, EPI, false, true>), dim3(g.bal_wg), dim3(64 * (W + 1)), kPad, st,
                                   in, Wp, w12, g.N, g.Kd, g.bal_wg, steps, eb);
            return hipGetLastError();
        }
    }
    const int ks = (steps + g.splits - 1) / g.splits;
    if (w12.planes != nullptr)
        hipLaunchKernelGGL((gemm_kernel<NT, MT, W, EPI, true>), dim3(gemm_groups(g) * g.splits), dim3(64 * W),
                           0, st, in, Wp, w12, g.N, g.Kd, gemm_groups(g), ks, ep);
    else
        hipLaunchKernelGGL((gemm_kernel<NT, MT, W, EPI, false>), dim3(gemm_groups(g) * g.splits), dim3(64 * W),
                           0, st, in, Wp, w12, g.N, g.Kd, gemm_groups(g), ks, ep);
    return hipGetLastError();
}

// Eight waves per workgroup (512 threads) leave each wave 256 registers, enough for up to four
// 16x16 accumulator tiles without spilling; wider tiles stay at four waves.
template <int NT, int MT, int EPI>
static hipError_t by_waves(const GemmShape &g, const GemmIn &in, const bf16 *Wp, const W12Ref &w12,
                           const GemmEpi &ep, hipStream_t st) {
    switch (g.waves) {
        case 4: return launch<NT, MT, 4, EPI>(g, in, Wp, w12, ep, st);
        case 8:
            if constexpr (NT * MT <= 4) return launch<NT, MT, 8, EPI>(g, in, Wp, w12, ep, st);
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

template <int EPI>
static hipError_t by_tiles(const GemmShape &g, const GemmIn &in, const bf16 *Wp, const W12Ref &w12,
                           const GemmEpi &ep, hipStream_t st) {
    const int mt = mt_for(in.M);
    if constexpr (EPI == EPI_QKV) {
        // groups of a tile and its rotation partner, one block of rows
        if (g.nt != 2 || mt != 1) return hipErrorInvalidValue;
        return by_waves<2, 1, EPI>(g, in, Wp, w12, ep, st);
    } else {
        if (g.nt == 4) {
            if (mt == 1) return by_waves<4, 1, EPI>(g, in, Wp, w12, ep, st);
            if (mt == 2) return by_waves<4, 2, EPI>(g, in, Wp, w12, ep, st);
            return by_waves<4, 4, EPI>(g, in, Wp, w12, ep, st);
        }
        if (g.nt == 2) {
            if (mt == 1) return by_waves<2, 1, EPI>(g, in, Wp, w12, ep, st);
            if (mt == 2) return by_waves<2, 2, EPI>(g, in, Wp, w12, ep, st);
            return by_waves<2, 4, EPI>(g, in, Wp, w12, ep, st);
        }
        if constexpr (EPI == EPI_SWIGLU) {
            return hipErrorInvalidValue;   // paired epilogue needs two tiles per group
        } else {
            if (mt == 1) return by_waves<1, 1, EPI>(g, in, Wp, w12, ep, st);
            if (mt == 2) return by_waves<1, 2, EPI>(g, in, Wp, w12, ep, st);
            return by_waves<1, 4, EPI>(g, in, Wp, w12, ep, st);
        }
    }
}

template <int EPI, bool W12, bool BAL>
static void launch_wide_tm(const GemmShape &g, const GemmIn &in, const bf16 *Wp, const W12Ref &w12,
                           const GemmEpi &ep, dim3 grid, int n_groups, int ks, hipStream_t st) {
    const dim3 block(64 * kWideWaves);
    switch (mt_for(in.M)) {
        case 1: hipLaunchKernelGGL((gemm_wide_kernel<1, EPI, W12, BAL>), grid, block, 0, st, in, Wp, w12, g.N, g.Kd, n_groups, ks, ep); break;
        case 2: hipLaunchKernelGGL((gemm_wide_kernel<2, EPI, W12, BAL>), grid, block, 0, st, in, Wp, w12, g.N, g.Kd, n_groups, ks, ep); break;
        default: hipLaunchKernelGGL((gemm_wide_kernel<4, EPI, W12, BAL>), grid, block, 0, st, in, Wp, w12, g.N, g.Kd, n_groups, ks, ep); break;
    }
}

template <int EPI, bool W12>
static void launch_wide_as(const GemmShape &g, const GemmIn &in, const bf16 *Wp, const W12Ref &w12,
                           const GemmEpi &ep, hipStream_t st) {
    const int steps = g.Kd >> 5;
    if constexpr (EPI == EPI_SWIGLU) {
        if (g.bal_q > 0 && ep.ctr != nullptr && ep.y != nullptr) {
            GemmEpi eb = ep;
            eb.bal_q = g.bal_q;
            launch_wide_tm<EPI, W12, true>(g, in, Wp, w12, eb, dim3(kPlanCUs), kPlanCUs, steps, st);
            return;
        }
    }
    const int ks = (steps + g.splits - 1) / g.splits;
    launch_wide_tm<EPI, W12, false>(g, in, Wp, w12, ep, dim3(gemm_groups(g) * g.splits), gemm_groups(g), ks, st);
}

template <int EPI>
static hipError_t launch_wide(const GemmShape &g, const GemmIn &in, const bf16 *Wp, const W12Ref &w12,
                              const GemmEpi &ep, hipStream_t st) {
    if (w12.planes != nullptr) launch_wide_as<EPI, true>(g, in, Wp, w12, ep, st);
    else launch_wide_as<EPI, false>(g, in, Wp, w12, ep, st);
    return hipGetLastError();
}

// One 64-row chunk of a skinny or wide launch.
static hipError_t chunk(const GemmShape &g, int epi, const GemmIn &in, const bf16 *Wp, const W12Ref &w12,
                        const GemmEpi &ep, hipStream_t st) {
    if (g.wide) {
        switch (epi) {
            case EPI_PARTIAL: return launch_wide<EPI_PARTIAL>(g, in, Wp, w12, ep, st);
            case EPI_SWIGLU: return launch_wide<EPI_SWIGLU>(g, in, Wp, w12, ep, st);
            case EPI_ARGMAX: return launch_wide<EPI_ARGMAX>(g, in, Wp, w12, ep, st);
            default: return hipErrorInvalidValue;
        }
    }
    switch (epi) {
        case EPI_PARTIAL: return by_tiles<EPI_PARTIAL>(g, in, Wp, w12, ep, st);
        case EPI_SWIGLU: return by_tiles<EPI_SWIGLU>(g, in, Wp, w12, ep, st);
        case EPI_ARGMAX: return by_tiles<EPI_ARGMAX>(g, in, Wp, w12, ep, st);
        case EPI_QKV: return by_tiles<EPI_QKV>(g, in, Wp, w12, ep, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t gemm(const GemmShape &g, int epi, const GemmIn &in_all, const bf16 *Wp,
                const GemmEpi &ep, hipStream_t st) {
    if (g.tc) {
        GemmIn in = in_all;
        in.M_total = g.M;
        in.m0 = 0;
        in.M = g.M;
        return gemm_tc(g, epi, in, Wp, ep, st);
    }
    for (int m0 = 0; m0 < g.M; m0 += 64) {
        GemmIn in = in_all;
        in.M_total = g.M;
        in.m0 = m0;
        in.M = g.M - m0 < 64 ? g.M - m0 : 64;
        const hipError_t e = chunk(g, epi, in, Wp, W12Ref{}, ep, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t gemm_w12(const GemmShape &g, int epi, const GemmIn &in_all, const W12Ref &w,
                    const GemmEpi &ep, hipStream_t st) {
    if (g.tc || w.planes == nullptr) return hipErrorInvalidValue;
    for (int m0 = 0; m0 < g.M; m0 += 64) {
        GemmIn in = in_all;
        in.M_total = g.M;
        in.m0 = m0;
        in.M = g.M - m0 < 64 ? g.M - m0 : 64;
        const hipError_t e = chunk(g, epi, in, nullptr, w, ep, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Tiles per group, waves per workgroup and K splits for a projection of N outputs over Kd at M
// rows. Every workgroup reads the activation rows of its K range once, so a group of NT tiles
// costs 1/NT of its weight bytes again in activation reads: groups are four tiles wide where the
// register budget allows. Projections with few groups are split along K (partials, added by a
// separate pass): at one block of rows into at most one workgroup per compute unit, at more rows
// until about 640 workgroups stream. Projections with many groups run whole and finish their
// epilogue in place. Eight waves when there are few groups or K splits.
static GemmShape plan_skinny(int M, int N, int Kd, bool allow_split);

GemmShape plan_gemm(int M, int N, int Kd, bool allow_split, bool allow_tc) {
    GemmShape g;
    g.M = M;
    g.N = N;
    g.Kd = Kd;
    g.wide = false;
    g.tc = false;
    g.bal_q = 0;
    const int steps = Kd / 32;
    if (allow_tc && M >= 128 && N % gemm_tc_columns() == 0) {
        // hundreds of rows: the matrix-core tile kernel, one launch over all 256-row tiles;
        // narrow projections split K so that about SV_TC_TARGET workgroups stream (512, two per
        // compute unit, measured best at 512 rows: fewer splits leave fewer fp32 partials to
        // write and add; 768, 384 and 256 were 8, 5 and 10 % slower on the batched step)
        g.tc = true;
        g.nt = gemm_tc_columns() / 16;
        g.waves = 4;
        const int groups = N / gemm_tc_columns();
        const int mtiles = (M + 255) / 256;
        g.splits = 1;
        if (allow_split && groups * mtiles < SV_TC_TARGET / 2) {
            g.splits = SV_TC_TARGET / (groups * mtiles);
            if (g.splits > 16) g.splits = 16;
            while (g.splits > 1 && steps / g.splits < 8) --g.splits;
        }
        return g;
    }
    if (M > 16 && N % (16 * kWideWaves * kWideTN) == 0) {
        // wide variant: 8 tiles per workgroup; split K into as many parts as keep every compute
        // unit at SV_WIDE_PER_CU workgroups at most. Each unit streams at a capped rate, so the
        // launch lasts as long as its busiest unit: one workgroup per unit on the branch-free loop
        // measured best (64-node tree: 12.89 ms per step; two per unit 13.86, one per unit on the
        // slab loop that waits for all loads 14.26, two per unit on it 13.41)
        g.wide = true;
        g.nt = kWideWaves * kWideTN;
        g.waves = kWideWaves;
        const int groups = N / (16 * g.nt);
        g.splits = 1;
        if (SV_WIDE_BAL && !allow_split && groups > kPlanCUs && groups < 2 * kPlanCUs &&
            kPlanCUs % (4 * (groups - kPlanCUs)) == 0 && steps % (kPlanCUs / (4 * (groups - kPlanCUs))) == 0) {
            // whole-K projections with a few more groups than compute units (gate/up at 64 rows:
            // 272 groups): one workgroup per unit, each with one group and a K part of a leftover
            // pair (SwiGLU only; other epilogues ignore it)
            g.bal_q = kPlanCUs / (4 * (groups - kPlanCUs));
        }
        if (SV_WIDE_PER_CU > 0 && allow_split && groups < kPlanCUs * SV_WIDE_PER_CU) {
            g.splits = kPlanCUs * SV_WIDE_PER_CU / groups;
            if (g.splits > 32) g.splits = 32;
            while (g.splits > 1 && steps / g.splits < kWideKS) --g.splits;
        } else if (allow_split && groups < 256) {
            int best = 0;
            for (int sp = 2; sp <= 32 && sp <= steps; ++sp) {
                if (steps % sp != 0 || (steps / sp) % kWideKS != 0) continue;
                best = sp;
                if (groups * sp >= SV_WIDE_TARGET) break;
            }
            if (best == 0) {
                best = (SV_WIDE_TARGET + groups - 1) / groups;
                if (best > 32) best = 32;
                while (best > 1 && steps / best < kWideKS) --best;
            }
            g.splits = best;
        }
        return g;
    }
    return plan_skinny(M, N, Kd, allow_split);
}

// Over W12 weights the whole-K projections (gate/up, output head) may run a different wave count:
// their workgroups all fit at once, so the bytes in flight are set by waves x batch depth.
GemmShape plan_gemm_w12(int M, int N, int Kd, bool allow_split) {
    GemmShape g = plan_gemm(M, N, Kd, allow_split, false);
    if (!g.wide && !allow_split && g.waves == 8) g.waves = SV_W12_WHOLE_WAVES;
    return g;
}

// Gate/up (whole K, SwiGLU epilogue). At one block of rows with a few more four-tile groups than
// two per compute unit (27B shape: 544), the skinny launch runs balanced on exactly two workgroups
// per unit (BAL above): each unit streams the same bytes, where 1088 two-tile groups at two
// resident per unit leave a third round of 64 on a quarter of the units. Measured at the 27B
// shape: 57.4 us against 59.4 for the 1088 groups; two-tile groups balanced over 1024 workgroups
// (four per unit in two rounds) took 65.7, 1088 four-wave workgroups all resident 59.7.
GemmShape plan_gemm_swiglu(int M, int N, int Kd, bool w12) {
    GemmShape g = w12 ? plan_gemm_w12(M, N, Kd, false) : plan_gemm(M, N, Kd, false);
    constexpr int nt = SV_SKINNY_BAL_NT;
    if (SV_SKINNY_BAL && !g.wide && !g.tc && M <= 16 && N % (16 * nt) == 0) {
        const int groups = N / (16 * nt), nwg = SV_SKINNY_BAL_PER_CU * kPlanCUs, steps = Kd / 32;
        const int lp = nt / 2 * (groups - nwg);          // leftover pairs
        if (lp > 0 && nwg % lp == 0 && steps % (nwg / lp) == 0) {
            g.nt = nt;
            g.waves = 8;
            g.splits = 1;
            g.bal_q = nwg / lp;
            g.bal_wg = nwg;
        }
    }
    return g;
}

GemmShape plan_gemm_qkv(int M, int N, int Kd) {
    // whole K in two-tile groups (one group per 16 columns of a head and their rotation
    // partners): at the 27B shape 224 workgroups, like the split-K plan's, each streaming two
    // tiles over all of K instead of four over half of it
    GemmShape g = plan_skinny(M, N, Kd, false);
    g.nt = 2;
    g.splits = 1;
    const int steps = Kd / 32;
    g.waves = (N / 32 < 1200 && steps / 8 >= 2) ? 8 : 4;
    return g;
}

static GemmShape plan_skinny(int M, int N, int Kd, bool allow_split) {
    GemmShape g;
    g.M = M;
    g.N = N;
    g.Kd = Kd;
    g.wide = false;
    g.tc = false;
    const int steps = Kd / 32;
    const int mt = mt_for(M < 64 ? M : 64);
    g.nt = (N % 64 == 0) ? 4 : (N % 32 == 0 ? 2 : 1);
    if (mt == 4 && g.nt == 4) g.nt = 2;
    // one block of rows, whole K, many more groups than compute units (gate/up, the output head):
    // two-tile groups. Four times as many workgroups as units spread the stream more evenly than
    // four-tile groups (gate/up at the 27B shape: 2.1 per unit, an eighth of the units streaming
    // a workgroup more than the rest; 9.64 against 9.87 ms per block step)
    if (mt == 1 && !allow_split && N % 32 == 0 && N / 64 > kPlanCUs) g.nt = 2;
    const int groups = N / (16 * g.nt);
    g.splits = 1;
    if (allow_split && mt == 1 && groups < kPlanCUs) {
        // one block of rows: at most one workgroup per compute unit, as many as fit. A stream
        // split over up to one workgroup per unit runs at the full rate; a grid that leaves some
        // units one workgroup more than others waits for those (one 256 MB stream measured
        // 6.7 TB/s over 256 workgroups, 5.3 over 320, 5.7 over 544)
        g.splits = kPlanCUs / groups;
        if (g.splits > 16) g.splits = 16;
        while (g.splits > 1 && steps / g.splits < 16) --g.splits;
    } else if (allow_split && groups < 400) {
        g.splits = (SV_SKINNY_TARGET + groups / 2) / groups;
        if (g.splits > 16) g.splits = 16;
        while (g.splits > 1 && steps / g.splits < 16) --g.splits;
    }
    g.waves = 4;
    if (g.nt * mt <= 4 && (groups * g.splits < SV_SKINNY_W8_MAX) && steps / (8 * g.splits) >= 2) g.waves = 8;
    return g;
}

}  // namespace sv
