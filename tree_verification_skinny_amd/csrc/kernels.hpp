// kernels.hpp — host-side launchers of the gfx950 kernels (internal to libspecverify).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace sv {

// ---- skinny GEMM: Y = X . W^T with X [M][Kd] bf16 (row stride ldx), W [N][Kd] bf16 ----------

struct GemmShape {
    int M, N, Kd, ldx;
    int nt;         // 16-row weight tiles per wave (2 or 4)
    int splits;     // K splits (partials)
};

// Number of workgroups (weight tile groups x splits) a partial GEMM launches per 64-row chunk.
int gemm_groups(const GemmShape &g);
// Partials P[s][m][n] = sum over the split's K range, s = 0..splits-1.
hipError_t gemm_partials(const GemmShape &g, const bf16 *X, const bf16 *W, float *P, hipStream_t st);
// Output head: per (group of 16*nt columns, row) the greedy (max, lowest index) into
// amax_val/amax_idx [n_groups][M]; optionally the fp32 logits [M][N]. splits must be 1.
hipError_t gemm_argmax(const GemmShape &g, const bf16 *X, const bf16 *W, float *logits,
                       float *amax_val, int *amax_idx, hipStream_t st);

// ---- attention ------------------------------------------------------------------------------

constexpr int kAttnChunk = 128;  // keys per attention workgroup

struct AttnArgs {
    const bf16 *q;               // [B*K][nq][D]
    const bf16 *k_pool, *v_pool; // this layer
    const int32_t *block_table;
    int max_pages, n_pages;
    const int32_t *ctx_len;
    const uint64_t *anc;         // [B*K]
    const int32_t *status;       // [B]
    int B, K, nq, nkv, D;
    int n_chunks;                // per request (grid), >= ceil((ctx + K) / kAttnChunk)
    float *part_o;               // [B][nkv][n_chunks][group*K][D]
    float2 *part_ml;             // [B][nkv][n_chunks][group*K]
    bf16 *out;                   // [B*K][nq*D]
};
hipError_t attention(const AttnArgs &a, hipStream_t st);

// ---- elementwise / bookkeeping --------------------------------------------------------------

struct NodeInfo {
    int32_t *depth, *pos, *status;
    uint64_t *anc;
    float2 *rope;                // [B*K][D/2] (cos, sin) at each node's position
};

hipError_t tree_prep(const int32_t *tokens, const int32_t *parent, const int32_t *ctx_len,
                     const int32_t *block_table, int max_pages, int n_pages, int B, int K,
                     int vocab, const NodeInfo &ni, hipStream_t st);
hipError_t rope_table(const NodeInfo &ni, int M, int D, double theta, hipStream_t st);
hipError_t embed_norm(const int32_t *tokens, const bf16 *embed, const bf16 *gain, int M, int H,
                      int vocab, float eps, bf16 *x, bf16 *u, bf16 *trace, hipStream_t st);
hipError_t qkv_rope_store(const float *P, int splits, const NodeInfo &ni, const int32_t *ctx_len,
                          const int32_t *block_table, int max_pages, int B, int K, int nq,
                          int nkv, int D, bf16 *q, bf16 *k_pool, bf16 *v_pool, hipStream_t st);
hipError_t residual_norm(const float *P, int splits, int M, int H, const bf16 *gain, float eps,
                         bf16 *x, bf16 *u, bf16 *trace, hipStream_t st);
hipError_t swiglu(const float *P, int splits, int M, int F, bf16 *h, hipStream_t st);
hipError_t argmax_partials(const float *logits, int M, int V, float *amax_val, int *amax_idx,
                           int n_chunks, hipStream_t st);
hipError_t argmax_accept(const float *amax_val, const int *amax_idx, int n_groups,
                         const int32_t *tokens, const int32_t *parent, const NodeInfo &ni, int B,
                         int K, int32_t *greedy, int32_t *accepted_len, int32_t *bonus,
                         int32_t *path, hipStream_t st);
hipError_t commit_kv(const int32_t *accepted_len, const int32_t *path, const int32_t *ctx_len,
                     const int32_t *block_table, int max_pages, int n_pages, int L, int B, int K,
                     int nkv, int D, bf16 *k_pool, bf16 *v_pool, hipStream_t st);
hipError_t commit_ctx(const int32_t *accepted_len, int32_t *ctx_len, int B, hipStream_t st);

}  // namespace sv
