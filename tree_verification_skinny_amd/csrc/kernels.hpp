// kernels.hpp — host-side launchers of the gfx950 kernels (internal to libspecverify).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace sv {

// ---- skinny GEMM: Y = X . W^T with X [M][Kd] bf16, W [N][Kd] bf16 packed in fragment order ----

struct GemmShape {
    int M, N, Kd;
    int nt;         // 16-row weight tiles per workgroup (1, 2 or 4; 8 for the wide variant)
    int waves;      // waves per workgroup (splitting K, or the tiles in the wide variant)
    int splits;     // K splits across workgroups (fp32 partials when > 1)
    bool wide;      // more than 16 rows: waves split the tiles, activations staged in LDS
    bool tc;        // a batch of hundreds of rows: the matrix-core-bound tile kernel
    int bal_q = 0;  // SwiGLU balanced over the compute units: 0 (off), or the K parts Q of each
                    // leftover gate/up pair (gemm_wide_kernel; gemm_kernel at one row block)
    int bal_wg = 0; // workgroups of a balanced skinny launch (two per compute unit)
};

// What a workgroup does with its finished tiles: partial sums of its K split, or (whole K)
// SwiGLU or the output head's per-group greedy maximum.
enum { EPI_PARTIAL = 0, EPI_SWIGLU = 1, EPI_ARGMAX = 2, EPI_QKV = 3 };

// The B operand: activations X [M_total][Kd] in fragment order (frag_off), rows padded to a
// multiple of 16.
struct GemmIn {
    const bf16 *Xp;
    int M, M_total, m0;          // filled per 64-row chunk by gemm()
};

struct GemmEpi {
    int F;                       // ffn (SwiGLU pairing)
    // PARTIAL: fp32 y [splits][M][N]
    float *y;
    // SWIGLU: h [M][F] in fragment order
    bf16 *h;
    // ARGMAX: per tile group (max, lowest index) [n_groups][M]; optional fp32 logits [M][N]
    float *logits, *amax_val;
    int *amax_idx;
    // QKV (whole K, groups of the two rotation halves of one head): bf16 rounding, RoPE with the
    // (cos, sin) table [M][D/2], q [M][nq][D], and the draft K/V rows into cache slots
    // ctx_len + node of requests whose status is 0
    const float2 *rope;
    const int32_t *status, *ctx_len, *block_table;
    int max_pages, K, nq, nkv, D;
    bf16 *q, *k_pool, *v_pool;
    // SWIGLU balanced over the compute units (GemmShape::bal_q): the leftover pairs' K-part sums go
    // to y (gemm_bal_scratch_bytes) and ctr holds one arrival counter per leftover pair
    // (gemm_bal_counters ints), zero before the launch and left zero by it
    int *ctr;
    int bal_q;
};

// A projection matrix in W12 form (k_w12.hip): three 4-bit planes per value in fragment order,
// the plan (window base, per-tile exception offsets) and the exception list.
struct W12Ref {
    const uint32_t *planes;
    const int32_t *plan;
    const int2 *exc;
};
int w12_plan_ints(int n);
hipError_t w12_plan(const bf16 *w, int n, int kd, int32_t *plan, hipStream_t st);
hipError_t w12_pack(const bf16 *w, int n, int kd, const int32_t *plan, uint32_t *planes, int2 *exc,
                    hipStream_t st);

int gemm_groups(const GemmShape &g);
// Scratch (bytes) and counters (ints) a balanced wide SwiGLU launch needs (0 when not balanced).
size_t gemm_bal_scratch_bytes(const GemmShape &g);
int gemm_bal_counters(const GemmShape &g);
hipError_t zero_ints(int *p, int n, hipStream_t st);
GemmShape plan_gemm(int M, int N, int Kd, bool allow_split, bool allow_tc = true);
GemmShape plan_gemm_swiglu(int M, int N, int Kd, bool w12);
hipError_t gemm(const GemmShape &g, int epi, const GemmIn &in, const bf16 *Wp, const GemmEpi &ep,
                hipStream_t st);
// The projection over a W12 matrix: the skinny or wide variant (never the tile kernel) as
// plan_gemm_w12 picks, bit-identical to gemm() over the same matrix in bf16 whenever the plans
// agree (every shape below 128 rows).
GemmShape plan_gemm_w12(int M, int N, int Kd, bool allow_split);
// The QKV projection with its RoPE epilogue (EPI_QKV): the skinny kernel, whole K, two-tile groups
// (the rotation halves of one head); for passes of at most 16 rows.
GemmShape plan_gemm_qkv(int M, int N, int Kd);
hipError_t gemm_w12(const GemmShape &g, int epi, const GemmIn &in, const W12Ref &w, const GemmEpi &ep,
                    hipStream_t st);
// Row-major [n][kd] -> fragment order; rows up to the next multiple of 16 are zero.
hipError_t pack_weight(const bf16 *w, int n, int kd, bf16 *out, hipStream_t st);
// The tile kernel for hundreds of rows (k_gemm_tc.hip): one launch covers all in.M_total rows,
// gemm_tc_columns() columns per workgroup.
hipError_t gemm_tc(const GemmShape &g, int epi, const GemmIn &in, const bf16 *Wp, const GemmEpi &ep,
                   hipStream_t st);
int gemm_tc_columns();

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
    bf16 *out;                   // [B*K][nq*D] in fragment order (the O projection's operand)
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
// x = embedding rows, u = RMSNorm(x) * gain (u in fragment order).
hipError_t embed_norm(const int32_t *tokens, const bf16 *table, const bf16 *gain, int M, int H,
                      int vocab, float eps, bf16 *x, bf16 *u, bf16 *trace, hipStream_t st);
// Add the split-K partials of the QKV projection (split order), round to bf16, rotate q and k,
// store q [M][nq][D] and the keys and values into the cache slots of the draft nodes.
hipError_t reduce_qkv(const float *P, int splits, const NodeInfo &ni, const int32_t *ctx_len,
                      const int32_t *block_table, int max_pages, int B, int K, int nq, int nkv,
                      int D, bf16 *q, bf16 *k_pool, bf16 *v_pool, hipStream_t st);
// Add the split-K partials of a projection into the residual stream, x = bf16(x + bf16(sum)),
// then u = RMSNorm(x) * gain for the next projection (u in fragment order).
hipError_t reduce_resid_norm(const float *P, int splits, int M, int H, const bf16 *gain, float eps,
                             bf16 *x, bf16 *u, bf16 *trace, hipStream_t st);
hipError_t argmax_partials(const float *logits, int M, int V, float *amax_val, int *amax_idx,
                           int n_chunks, hipStream_t st);
int argmax_chunks(int V);
// err (device, may be NULL): when set, every request is reported failed.
hipError_t argmax_accept(const float *amax_val, const int *amax_idx, int n_groups,
                         const int32_t *tokens, const int32_t *parent, const NodeInfo &ni, int B,
                         int K, int32_t *greedy, int32_t *accepted_len, int32_t *bonus,
                         int32_t *path, hipStream_t st, const uint32_t *err = nullptr);
hipError_t commit_kv(const int32_t *accepted_len, const int32_t *path, const int32_t *ctx_len,
                     const int32_t *block_table, int max_pages, int n_pages, int L, int B, int K,
                     int nkv, int D, bf16 *k_pool, bf16 *v_pool, hipStream_t st);
// ctx_len += accepted_len + 1 where commit_kv applies (the same all-or-nothing rule).
hipError_t commit_ctx(const int32_t *accepted_len, const int32_t *path, const int32_t *block_table,
                      int max_pages, int n_pages, int K, int32_t *ctx_len, int B, hipStream_t st);
// Prompt prefill bookkeeping (k_prefill.hip).
hipError_t prefill_init(int32_t *failed, int B, hipStream_t st);
hipError_t prefill_gather(const int32_t *prompt, int p, int c0, int n, int B, int32_t *out, hipStream_t st);

// Chunked prefill (k_prefill.hip): positions and per-request status of a chunk of n rows per
// request; causal attention of the chunk over the cache into the O operand; each request's last
// row into the output head's operand; the head's per-group maxima merged into the next tokens,
// and the committed context advanced.
hipError_t prefill_prep(const int32_t *tokens, int n, int B, int vocab, const int32_t *ctx_len,
                        const int32_t *block_table, int max_pages, int n_pages, const int32_t *failed,
                        int32_t *pos, int32_t *status, hipStream_t st);
hipError_t prefill_attention(const bf16 *q, const bf16 *k_pool, const bf16 *v_pool, const int32_t *block_table,
                             int max_pages, const int32_t *ctx_len, const int32_t *status, int B, int n, int nq,
                             int nkv, int D, bf16 *out, hipStream_t st);
hipError_t prefill_last_rows(const bf16 *u, int n, int B, int H, bf16 *out, hipStream_t st);
hipError_t prefill_finish(const float *amv, const int *ami, int groups, int B, int n, bool last,
                          const int32_t *status, int32_t *failed, int32_t *ctx_len, int32_t *next_token,
                          hipStream_t st);
// Recurrent layers of a hybrid target: the tree pass over the committed state (k_recurrent.hip)
// and the accepted node's state written in place (k_rec_commit.hip). D = dk = dv, 64 or 128;
// K <= kRecMaxK.
constexpr int kRecMaxK = 64;
hipError_t rec_tree(const float *state, const bf16 *q, const bf16 *k, const bf16 *v,
                    const float *log_gate, const int32_t *tree_parent, int B, int K, int H, int D,
                    float *out, int32_t *status, hipStream_t st);
hipError_t rec_commit(float *state, const bf16 *k, const bf16 *v, const float *log_gate,
                      const int32_t *accepted_len, const int32_t *accepted_path, int B, int K, int H,
                      int D, hipStream_t st);
// A recurrent layer inside the verify pass: its projection's split-K partials [splits][M][N]
// (N >= 3 H D + H: q, k, v heads, then the gate inputs) to q, k, v bf16 [M][H][D] and the
// log-gates g = -softplus(bf16(a)) fp32 [M][H]; the tree pass's fp32 output [M][W] to the O
// projection's bf16 operand in fragment order.
hipError_t reduce_rec(const float *P, int splits, int M, int N, int H, int D, bf16 *q, bf16 *k, bf16 *v,
                      float *g, hipStream_t st);
hipError_t rec_operand(const float *out, int M, int W, bf16 *x, hipStream_t st);
// ---- the persistent pass over the layers for at most 16 rows (k_fused.hip) ------------------------
constexpr int kFusedMaxLayers = 16;    // layers per launch (their weights ride in the arguments)
// Phase timestamps per (layer, workgroup): QKV wait begin, inputs ready, loop end, done (0-3),
// attention items done (4), merges done (5), O (6-9), gate/up (10-13), down (14-17); inside the
// (last) attention item of the workgroup: inputs ready (18), keys and values in LDS (19), products
// done (20); inside its (last) merge task: inputs ready (21), output written (22).
constexpr int kFusedTraceEvents = 24;
enum { FUSED_QKV = 0, FUSED_O = 1, FUSED_GU = 2, FUSED_DOWN = 3 };

// One projection, split evenly over g_eff workgroups as ranges of (64-column group, 32-wide K
// step) units; the same split every layer.
struct FusedPhase {
    int S;            // K steps
    int groups;       // 64-column groups
    int units;        // groups * S
    int g_eff;        // workgroups with units: min(G, units)
    int max_parts;    // most workgroups sharing a group
    float *part;      // [groups][max_parts][1024] fp32 partial sums
    uint32_t *cnt;    // [groups] arrivals (every layer adds the group's part count)
    uint32_t *flag;   // [groups] epoch (global layer + 1) of the finished group
};

struct FusedArgs {
    int L0, nl, Lt;                  // first layer and layer count of this launch; all layers
    int H, nq, nkv, D, F, B, K, M;   // M = B * K <= 16
    int G;                           // persistent workgroups (one per compute unit)
    float eps, scale_log2;
    const bf16 *w[kFusedMaxLayers][4];          // packed weights: qkv, o, gate/up, down
    const bf16 *g_attn[kFusedMaxLayers], *g_mlp[kFusedMaxLayers], *g_final;
    bf16 *k_pool, *v_pool;
    int64_t layer_stride;
    const int32_t *block_table;
    int max_pages;
    const int32_t *ctx_len, *status;
    const uint64_t *anc;
    const float2 *rope;
    // Operands read with plain (cached) loads have one slot per layer of a launch, written once
    // in it: the residual stream after O and after down ([16][H] fragment order; the input of
    // the launch's first layer is the last down slot, which the embedding fills before layer 0),
    // q ([M][nq][D]), the attention output ([16][nq*D] fragment order, O's operand) and the
    // SwiGLU output ([16][F] fragment order, down's operand).
    bf16 *x_o, *x_d;                 // [kFusedMaxLayers][16][H]
    float *ssq_o, *ssq_d;            // [H/64][16] groups' sums of squares after O, after down
    bf16 *q;                         // [kFusedMaxLayers][M][nq][D]
    bf16 *ao;                        // [kFusedMaxLayers][16][nq*D]
    bf16 *h;                         // [kFusedMaxLayers][16][F]
    bf16 *u_head;                    // [16][H] fragment order, the output head's operand
    bf16 *trace;                     // optional [Lt + 1][M][H] residual stream
    FusedPhase ph[4];
    int CH, n_chunks, n_items, n_tasks;   // keys per attention item, chunks per request, items, merges
    float *att_o;                    // [n_items][tiles][16][D]
    uint64_t *att_ml;                // [n_items][tiles][16] (max, sum) pairs
    uint32_t *f_att, *f_comb;        // epochs of the items and the merge tasks
    uint32_t *err;                   // set when a wait timed out
    uint64_t *trace_t;               // optional [Lt][G][kFusedTraceEvents] phase timestamps
};
// Workgroups of fused_layers that fit on one compute unit (0 when it cannot run).
int fused_occupancy(int D);
// Before the first launch: clears the sync words and the attention and SwiGLU operands, and
// writes x (embedding rows, zero past M), its per-group sums of squares and the trace's first row.
hipError_t fused_prep(const FusedArgs &a, const int32_t *tokens, const bf16 *embed, int vocab,
                      uint32_t *sync_words, int n_sync, hipStream_t st);
hipError_t fused_layers(const FusedArgs &a, hipStream_t st);

// Reads bytes (a multiple of 16, 16-byte aligned) once as a grid-stride stream.
hipError_t read_probe(const void *buf, int64_t bytes, uint32_t *out, hipStream_t st);

}  // namespace sv
