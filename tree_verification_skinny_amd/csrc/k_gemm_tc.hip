// k_gemm_tc.hip — the projections of a batched verify pass (hundreds of draft rows), where the
// matrix cores, not HBM, set the pace: one weight byte serves every row of the batch.
//
// Batching many requests into one pass is how the verify step amortises the weight read [SpecPilot
// digest, airadar.tv — summary paragraph]; at 512 rows the projections carry ~500 flops per
// weight byte, past what HBM alone can feed at matrix-core speed. Design:
//   * A workgroup of 4 waves (one per SIMD, so each has the whole register file) owns a
//     128-column x 256-row output tile: waves form a 2 x 2 grid, each wave 4 weight tiles
//     (64 columns) x 8 row blocks (128 rows), 32 accumulator tiles. A weight fragment serves 256
//     rows per read.
//   * Per 32-wide K step the workgroup's 8 weight fragments and 16 activation fragments (24 KB,
//     both already in MFMA fragment order, so every load is a contiguous 1 KB wave read) pass
//     through LDS; a wave reads 12 of them (4 + 8) for its 32 products.
//   * The fragments go from HBM / L2 straight into LDS (global_load_lds, no register staging),
//     one K step ahead of the products, into two LDS stages (48 KB, so that three workgroups
//     share a compute unit and cover each other's load latency); one wait and one barrier per
//     step. Without a register ring the loop body is a single copy and the 128 accumulator
//     registers stay where they are.
//   * One launch covers every 256-row tile; the tiles of one column group go to workgroups that
//     run back to back on the same XCD, so the weights come from HBM once and from L2 after.
//   * Epilogues as in the skinny kernel: fp32 split-K partials, SwiGLU (a wave holds gate tiles
//     and the matching up tiles), or the per-row greedy maximum of the output head.
#include "kernels.hpp"

namespace sv {

namespace {

constexpr int kWN = 2, kWM = 2;                // wave grid: columns x rows
constexpr int kTN = 4, kTM = 8;                // per wave: weight tiles x row blocks
constexpr int kNT = kWN * kTN;                 // weight tiles per workgroup (128 columns)
constexpr int kMB = kWM * kTM;                 // row blocks per workgroup (256 rows)
constexpr int kThreads = 64 * kWN * kWM;       // 256
constexpr int kSlots = (kNT + kMB) * 64;       // 16-byte slots per K step: 8 + 16 fragments
constexpr int kPer = kSlots / kThreads;        // slots staged per thread per step (6)
#ifndef SV_TC_STAGES
#define SV_TC_STAGES 2
#endif
constexpr int kStages = SV_TC_STAGES;          // LDS stages: K steps in flight + the one in use
static_assert(kSlots % kThreads == 0, "a K step must split evenly over the threads");

// s_waitcnt with vmcnt <= n (n < 64) and the other counters unconstrained
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00);
}

// packed weight tile of workgroup tile index t (0..7) in column group ng. SwiGLU: wave wn holds
// t = 4 wn + j, gate tiles for j = 0, 1 and the matching up tiles for j = 2, 3.
template <int EPI>
__device__ __forceinline__ int tc_col(int ng, int t, int F) {
    if constexpr (EPI == EPI_SWIGLU) {
        const int wn = t >> 2, j = t & 3;
        return (j < 2 ? 0 : F) + (ng * 4 + wn * 2 + (j & 1)) * 16;
    } else {
        return (ng * kNT + t) * 16;
    }
}

template <int EPI>
__global__ __launch_bounds__(kThreads, 2) void gemm_tc_kernel(GemmIn in, const bf16 *__restrict__ Wp,
                                                           int N, int Kd, int n_groups, int ksteps,
                                                           int n_units, int n_mt, GemmEpi ep) {
    __shared__ bf16x8 lds[kStages][kSlots];
    __shared__ float red_v[kWN][kMB * 16];
    __shared__ int red_i[kWN][kMB * 16];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave % kWN, wm = wave / kWN;
    const int r16 = lane & 15, grp = lane >> 4;
    // workgroup -> (row tile, column group, split). Consecutive workgroups land on consecutive
    // XCDs, so the row tiles of one (group, split) are given to workgroups 8 apart: they run back
    // to back on the same XCD and the second finds the weights in that XCD's L2.
    const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
    const int mtile = q % n_mt;
    const int unit = (q / n_mt) * 8 + xcd;
    if (unit >= n_units) return;                 // grid padding
    const int ng = unit % n_groups;
    const int split = unit / n_groups;
    const int S = Kd >> 5;
    const int s_begin = split * ksteps;
    const int s_end = min(s_begin + ksteps, S);
    const int nsteps = s_end > s_begin ? s_end - s_begin : 0;
    const int m0 = mtile * kMB * 16;
    const int M = min(in.M_total - m0, kMB * 16);
    const int nblk = (in.M_total + 15) >> 4;

    // the global source of each of this thread's slots (step 0 of the split): slot
    // i = tid + 256 r is fragment f = wave + 4 r (wave-uniform) at lane i % 64; fragments below 8
    // are weight tiles, the rest activation blocks
    const bf16 *src[kPer];
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
        const int f = wave + (kThreads / 64) * r;
        int64_t frag;
        if (f < kNT) {
            frag = (int64_t)(tc_col<EPI>(ng, f, ep.F) >> 4) * S + s_begin;
            src[r] = Wp + frag * 512;
        } else {
            frag = (int64_t)min((m0 >> 4) + f - kNT, nblk - 1) * S + s_begin;
            src[r] = in.Xp + frag * 512;
        }
    }
    // step s (relative to the split) into LDS stage st: slot i = tid + 256 r, so each wave writes
    // one contiguous 1 KB block per r, at a wave-uniform LDS address
    auto issue = [&](int s, int st) {
#pragma unroll
        for (int r = 0; r < kPer; ++r)
            __builtin_amdgcn_global_load_lds(
                (const void *)(src[r] + (int64_t)s * 512 + lane * 8),
                (__attribute__((address_space(3))) void *)&lds[st][(wave + (kThreads / 64) * r) * 64],
                16, 0, 0);
    };

    floatx4 acc[kTN][kTM];
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
        for (int mt = 0; mt < kTM; ++mt) acc[j][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

    auto multiply = [&](int buf) {
        bf16x8 a[kTN];
#pragma unroll
        for (int j = 0; j < kTN; ++j) a[j] = lds[buf][(wn * kTN + j) * 64 + lane];
        // activation fragments four at a time, to bound the live registers
#pragma unroll
        for (int h = 0; h < kTM / 4; ++h) {
            bf16x8 b[4];
#pragma unroll
            for (int mm = 0; mm < 4; ++mm) b[mm] = lds[buf][(kNT + wm * kTM + h * 4 + mm) * 64 + lane];
#pragma unroll
            for (int j = 0; j < kTN; ++j)
#pragma unroll
                for (int mm = 0; mm < 4; ++mm)
                    acc[j][h * 4 + mm] = mfma16x16x32(a[j], b[mm], acc[j][h * 4 + mm]);
        }
    };

    // prologue: steps 0 .. kStages-2 in flight
#pragma unroll
    for (int p = 0; p < kStages - 1; ++p)
        if (p < nsteps) issue(p, p);
    for (int s = 0; s < nsteps; ++s) {
        // step s has landed once at most the loads of the later steps already issued remain
        const int later = min(kStages - 2, nsteps - 1 - s);
        if (later >= 2) wait_vmcnt<2 * kPer>();
        else if (later == 1) wait_vmcnt<kPer>();
        else wait_vmcnt<0>();
        __syncthreads();                       // every wave's part of step s is in LDS, and step
                                               // s - 1 (the stage reused below) is consumed
        if (s + kStages - 1 < nsteps) issue(s + kStages - 1, (s + kStages - 1) % kStages);
        multiply(s % kStages);
    }

    // ---- epilogues ------------------------------------------------------------------------------
    int col[kTN];
#pragma unroll
    for (int j = 0; j < kTN; ++j) col[j] = tc_col<EPI>(ng, wn * kTN + j, ep.F) + 4 * grp;
#pragma unroll
    for (int mt = 0; mt < kTM; ++mt) {
        const int m = (wm * kTM + mt) * 16 + r16;     // row within the workgroup's rows
        const bool live = m < M;
        const int row = m0 + m;
        if constexpr (EPI == EPI_PARTIAL) {
            if (live) {
#pragma unroll
                for (int j = 0; j < kTN; ++j)
                    *(floatx4 *)(ep.y + ((int64_t)split * in.M_total + row) * N + col[j]) = acc[j][mt];
            }
        } else if constexpr (EPI == EPI_SWIGLU) {
            if (live) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    float hv[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float g = round_bf(acc[j][mt][e]);
                        const float u = round_bf(acc[j + 2][mt][e]);
                        hv[e] = (g / (1.0f + expf(-g))) * u;
                    }
                    store4(ep.h + frag_off(row, col[j], ep.F), hv[0], hv[1], hv[2], hv[3]);
                }
            }
        } else if constexpr (EPI == EPI_ARGMAX) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
#pragma unroll
            for (int j = 0; j < kTN; ++j) {
                if (ep.logits != nullptr && live) *(floatx4 *)(ep.logits + (int64_t)row * N + col[j]) = acc[j][mt];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (better(acc[j][mt][e], col[j] + e, bv, bi)) { bv = acc[j][mt][e]; bi = col[j] + e; }
            }
#pragma unroll
            for (int o = 16; o < 64; o <<= 1) {
                const float ov = __shfl_xor(bv, o, 64);
                const int oi = __shfl_xor(bi, o, 64);
                if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
            }
            if (grp == 0) {
                red_v[wn][m] = bv;
                red_i[wn][m] = bi;
            }
        }
    }
    if constexpr (EPI == EPI_ARGMAX) {
        // the group's best per row over its two column waves, in column order
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kMB * 16 / kThreads; ++k) {
            const int m = tid + k * kThreads;
            if (m < M) {
                float bv = red_v[0][m];
                int bi = red_i[0][m];
                if (better(red_v[1][m], red_i[1][m], bv, bi)) { bv = red_v[1][m]; bi = red_i[1][m]; }
                ep.amax_val[(int64_t)ng * in.M_total + m0 + m] = bv;
                ep.amax_idx[(int64_t)ng * in.M_total + m0 + m] = bi;
            }
        }
    }
}

}  // namespace

int gemm_tc_columns() { return kNT * 16; }

hipError_t gemm_tc(const GemmShape &g, int epi, const GemmIn &in, const bf16 *Wp, const GemmEpi &ep,
                   hipStream_t st) {
    const int steps = g.Kd >> 5;
    const int ks = (steps + g.splits - 1) / g.splits;
    const int groups = g.N / (kNT * 16);
    const int units = groups * g.splits;
    const int n_mt = (in.M_total + kMB * 16 - 1) / (kMB * 16);
    const dim3 grid((unsigned)((units + 7) / 8 * 8 * n_mt)), block(kThreads);
    switch (epi) {
        case EPI_PARTIAL: hipLaunchKernelGGL(gemm_tc_kernel<EPI_PARTIAL>, grid, block, 0, st, in, Wp, g.N, g.Kd, groups, ks, units, n_mt, ep); break;
        case EPI_SWIGLU: hipLaunchKernelGGL(gemm_tc_kernel<EPI_SWIGLU>, grid, block, 0, st, in, Wp, g.N, g.Kd, groups, ks, units, n_mt, ep); break;
        case EPI_ARGMAX: hipLaunchKernelGGL(gemm_tc_kernel<EPI_ARGMAX>, grid, block, 0, st, in, Wp, g.N, g.Kd, groups, ks, units, n_mt, ep); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace sv
