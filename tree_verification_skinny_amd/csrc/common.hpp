// common.hpp — device types and helpers shared by the gfx950 kernels of the verify step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;

namespace sv {

constexpr int kWave = 64;
constexpr int kPage = 16;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float to_f(bf16 v) { return (float)v; }
// fp32 -> bf16, round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ bf16 to_bf(float v) { return (bf16)v; }
__device__ __forceinline__ float round_bf(float v) { return (float)(bf16)v; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// Sum over a 256-thread block; every thread gets the total. `red` holds >= 4 floats.
__device__ __forceinline__ float block_sum_256(float v, float *red) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

// (value, index) pair order for the greedy choice: larger value first, then lower index.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

// A 16-byte load marked non-temporal: data read once per pass (weights, the KV cache), which
// should not displace what is reused.
__device__ __forceinline__ bf16x8 stream_load(const bf16x8 *p) { return __builtin_nontemporal_load(p); }

__device__ __forceinline__ floatx4 mfma16x16x32(bf16x8 a, bf16x8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Fragment order of a bf16 matrix A [rows][cols] (cols % 32 == 0), the order the projection
// kernels stream both operands in: blocks of 16 rows; in each block, steps of 32 columns; in each
// step, 64 slots of 8 consecutive elements, slot l = A[16 block + l % 16][32 step + 8 (l / 16) ..].
// Element offset of A[r][c]; the 4-aligned groups c..c+3 stay contiguous.
__device__ __forceinline__ int64_t frag_off(int64_t r, int c, int cols) {
    return (((r >> 4) * (cols >> 5) + (c >> 5)) * 64 + (r & 15) + 16 * ((c >> 3) & 3)) * 8 + (c & 7);
}

// Four bf16 values to one 8-byte store.
__device__ __forceinline__ void store4(bf16 *dst, float a, float b, float c, float d) {
    bf16 v[4] = {to_bf(a), to_bf(b), to_bf(c), to_bf(d)};
    *reinterpret_cast<uint2 *>(dst) = *reinterpret_cast<const uint2 *>(v);
}

// Position p of request b -> (page id, slot). Caller guarantees p is inside the request's pages.
__device__ __forceinline__ int page_of(const int32_t *block_table, int max_pages, int b, int p) {
    return block_table[(int64_t)b * max_pages + (p >> 4)];
}

}  // namespace sv
