// k_w12.hip — load-time conversion of a bf16 projection matrix into W12, the lossless 12-bit
// layout the skinny projection kernel can stream instead of bf16.
//
// The SpecPilot digest (airadar.tv — "Reasons") names a lossless 12-bit weight format: each bf16
// weight is split into three 4-bit planes that the GEMM reassembles bit for bit in registers,
// which cuts the weight bytes a batch-1 pass streams by a quarter. The pages give neither the
// planes' contents nor how values that do not fit are kept. This layout:
//   * one window of 16 exponent fields [b, b+15] per matrix, b even, chosen to leave the fewest
//     values outside (lowest b on ties);
//   * planes 0 and 1 are a value's low byte (mantissa and the exponent's lowest bit), stored as
//     is; plane 2 is the nibble (sign, (e - b) >> 1), which gives back the high byte with one add
//     of b / 2 because b is even;
//   * a value outside the window is an exception: its planes hold the low byte and a zero
//     nibble, and (position, 16-bit value) goes into a per-matrix list sorted by tile, then
//     position, which the GEMM applies in registers after decoding.
// Physical order follows the bf16 fragment order (16-row tiles, 32-column steps): fragment
// (tile t, step s) is 768 bytes at (t * S + s) * 768, 12 bytes per lane, so that one 12-byte
// load per lane reads a whole fragment. For lane l (row 16t + l%16, columns 32s + 8(l/16) .. +7,
// values v0..v7), at dword 3l of the fragment:
//   dword 3l     = low bytes of v0..v3 (byte j = v_j),
//   dword 3l + 1 = low bytes of v4..v7,
//   dword 3l + 2 = nibbles: v_{2i} at bits 4i..4i+3, v_{2i+1} at bits 16+4i..16+4i+3,
// so that one shift and mask put a pair's two nibbles under the high bytes of a bf16 pair.
// An exception entry is (s * 512 + l * 8 + j, bf16 bits).
//
// Plan (int32): [0] b, [1] total exceptions, [2 .. 2 + T] exception offsets per tile (T + 1
// entries, exclusive prefix), then a 256-bin exponent histogram (scratch).
#include "kernels.hpp"

namespace sv {

static __device__ __forceinline__ int w12_field(uint16_t v) { return (v >> 7) & 0xff; }

// A small fill kernel (not hipMemsetAsync, which misbehaves inside captured graphs).
__global__ void zero_ints_kernel(int *__restrict__ p, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

// Exponent-field histogram of the whole matrix (row-major [n][kd]).
__global__ __launch_bounds__(256) void w12_hist_kernel(const uint16_t *__restrict__ w, int64_t total,
                                                       int *__restrict__ hist) {
    __shared__ int h[256];
    h[threadIdx.x] = 0;
    __syncthreads();
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256)
        atomicAdd(&h[w12_field(w[i])], 1);
    __syncthreads();
    if (h[threadIdx.x] != 0) atomicAdd(&hist[threadIdx.x], h[threadIdx.x]);
}

// One thread: the window with the most values inside (lowest base on ties).
__global__ void w12_base_kernel(int32_t *__restrict__ plan, const int *__restrict__ hist) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    long long best = -1;
    int best_b = 0;
    for (int b = 0; b <= 240; b += 2) {
        long long c = 0;
        for (int e = b; e <= b + 15; ++e) c += hist[e];
        if (c > best) {
            best = c;
            best_b = b;
        }
    }
    plan[0] = best_b;
}

// Exceptions per tile: one workgroup per tile.
__global__ __launch_bounds__(256) void w12_count_kernel(const uint16_t *__restrict__ w, int kd,
                                                        int32_t *__restrict__ plan) {
    __shared__ float red[4];
    const int tile = blockIdx.x;
    const int b = plan[0];
    int c = 0;
    const int64_t base = (int64_t)tile * 16 * kd;
    for (int i = threadIdx.x; i < 16 * kd; i += 256) {
        const int e = w12_field(w[base + i]);
        c += (e < b || e > b + 15) ? 1 : 0;
    }
    const float tot = block_sum_256((float)c, red);   // exact: counts stay far below 2^24
    if (threadIdx.x == 0) plan[2 + tile] = (int32_t)tot;
}

// Exclusive prefix over the tiles' counts, in place (one workgroup); plan[1] = total.
__global__ __launch_bounds__(256) void w12_scan_kernel(int32_t *__restrict__ plan, int tiles) {
    __shared__ int32_t part[256];
    int32_t *cnt = plan + 2;
    const int per = (tiles + 255) / 256;
    const int t0 = threadIdx.x * per;
    const int t1 = min(t0 + per, tiles);
    int32_t s = 0;
    for (int t = t0; t < t1; ++t) s += cnt[t];
    part[threadIdx.x] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t run = 0;
        for (int i = 0; i < 256; ++i) {
            const int32_t v = part[i];
            part[i] = run;
            run += v;
        }
        plan[1] = run;
        cnt[tiles] = run;
    }
    __syncthreads();
    int32_t run = part[threadIdx.x];
    for (int t = t0; t < t1; ++t) {
        const int32_t v = cnt[t];
        cnt[t] = run;
        run += v;
    }
}

// Planes and exception entries: one wave per tile, walking its steps in order; lanes take
// their exception slots by an in-wave exclusive prefix so the list is sorted by position.
__global__ __launch_bounds__(64) void w12_pack_kernel(const uint16_t *__restrict__ w, int kd,
                                                      const int32_t *__restrict__ plan,
                                                      uint32_t *__restrict__ planes,
                                                      int2 *__restrict__ exc) {
    const int tile = blockIdx.x;
    const int lane = threadIdx.x;
    const int b = plan[0];
    const int S = kd >> 5;
    int32_t next = plan[2 + tile];
    const int64_t row = (int64_t)tile * 16 + (lane & 15);
    for (int s = 0; s < S; ++s) {
        const int col = 32 * s + 8 * (lane >> 4);
        const uint4 raw = *(const uint4 *)(w + row * kd + col);
        const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
        uint32_t lo0 = 0, lo1 = 0, nib = 0;
        int esc_mask = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t v = (rw[j >> 1] >> (16 * (j & 1))) & 0xffffu;
            const int e = (int)((v >> 7) & 0xff);
            const bool fits = e >= b && e <= b + 15;
            const uint32_t n4 = fits ? (((v >> 15) << 3) | (uint32_t)((e - b) >> 1)) : 0u;
            if (j < 4) lo0 |= (v & 0xffu) << (8 * j);
            else lo1 |= (v & 0xffu) << (8 * (j - 4));
            nib |= n4 << ((j & 1) ? 16 + 4 * (j >> 1) : 4 * (j >> 1));
            if (!fits) esc_mask |= 1 << j;
        }
        uint32_t *f = planes + ((int64_t)tile * S + s) * 192 + 3 * lane;
        f[0] = lo0;
        f[1] = lo1;
        f[2] = nib;
        const int cnt = __popc(esc_mask);
        // in-wave exclusive prefix of the counts
        int incl = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o, 64);
            if (lane >= o) incl += y;
        }
        const int total = __shfl(incl, 63, 64);
        if (cnt != 0) {
            int k = next + incl - cnt;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (esc_mask & (1 << j)) {
                    exc[k] = make_int2(s * 512 + lane * 8 + j, (int)((rw[j >> 1] >> (16 * (j & 1))) & 0xffffu));
                    ++k;
                }
            }
        }
        next += total;
    }
}

hipError_t zero_ints(int *p, int n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(zero_ints_kernel, dim3(1), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

int w12_plan_ints(int n) { return 2 + (n / 16 + 1) + 256; }

hipError_t w12_plan(const bf16 *w, int n, int kd, int32_t *plan, hipStream_t st) {
    const int tiles = n / 16;
    int *hist = plan + 2 + tiles + 1;
    hipLaunchKernelGGL(zero_ints_kernel, dim3(1), dim3(256), 0, st, hist, 256);
    const int64_t total = (int64_t)n * kd;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(w12_hist_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                       reinterpret_cast<const uint16_t *>(w), total, hist);
    hipLaunchKernelGGL(w12_base_kernel, dim3(1), dim3(64), 0, st, plan, hist);
    hipLaunchKernelGGL(w12_count_kernel, dim3(tiles), dim3(256), 0, st,
                       reinterpret_cast<const uint16_t *>(w), kd, plan);
    hipLaunchKernelGGL(w12_scan_kernel, dim3(1), dim3(256), 0, st, plan, tiles);
    return hipGetLastError();
}

hipError_t w12_pack(const bf16 *w, int n, int kd, const int32_t *plan, uint32_t *planes, int2 *exc,
                    hipStream_t st) {
    hipLaunchKernelGGL(w12_pack_kernel, dim3(n / 16), dim3(64), 0, st,
                       reinterpret_cast<const uint16_t *>(w), kd, plan, planes, exc);
    return hipGetLastError();
}

}  // namespace sv
