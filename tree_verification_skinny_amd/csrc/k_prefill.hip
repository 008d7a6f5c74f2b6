// k_prefill.hip — bookkeeping kernels of the prompt prefill. The pass itself is the verify pass
// run over consecutive chunks of the prompt as linear blocks: a drafted block is scored in one
// target pass [SpecPilot news piece, wireai.ir — "The main challenge"], and a prompt chunk is a
// block that is accepted whole, its K/V committed before the next chunk (see spec_prefill).
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

// After a chunk's pass: a request the pass marked bad (accepted_len < 0) fails for good; the
// others advance their committed context by the chunk. After the last chunk, the greedy token
// of the prompt's last position (or -1) goes to next_token.
__global__ void prefill_advance_kernel(const int32_t *__restrict__ acc, const int32_t *__restrict__ greedy,
                                       int n, int B, int last, int32_t *__restrict__ failed,
                                       int32_t *__restrict__ ctx_len, int32_t *__restrict__ next_token) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    if (acc[b] < 0) failed[b] = 1;
    if (!failed[b]) ctx_len[b] += n;
    if (last) next_token[b] = failed[b] ? -1 : greedy[b * n + n - 1];
}

// Row b*n + n - 1 of the chunk's fp32 logits [B*n][V] into out [B][V].
__global__ void prefill_last_logits_kernel(const float *__restrict__ logits, int n, int V,
                                           float *__restrict__ out) {
    const int b = blockIdx.y;
    const float *src = logits + ((int64_t)b * n + n - 1) * V;
    for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < V; j += gridDim.x * blockDim.x)
        out[(int64_t)b * V + j] = src[j];
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

hipError_t prefill_advance(const int32_t *acc, const int32_t *greedy, int n, int B, bool last,
                           int32_t *failed, int32_t *ctx_len, int32_t *next_token, hipStream_t st) {
    hipLaunchKernelGGL(prefill_advance_kernel, dim3((B + 255) / 256), dim3(256), 0, st, acc, greedy, n, B,
                       last ? 1 : 0, failed, ctx_len, next_token);
    return hipGetLastError();
}

hipError_t prefill_last_logits(const float *logits, int n, int B, int V, float *out, hipStream_t st) {
    hipLaunchKernelGGL(prefill_last_logits_kernel, dim3((V + 255) / 256 < 64 ? (V + 255) / 256 : 64, B),
                       dim3(256), 0, st, logits, n, V, out);
    return hipGetLastError();
}

}  // namespace sv
