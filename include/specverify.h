/*
 * specverify.h — C ABI of the MI355X (gfx950) verification step of lossless greedy speculative
 * decoding.
 *
 * The operation. A drafter proposes several tokens per step and the target model checks all of
 * them in one forward pass [JetSpec article, seventnews.com — opening section]. Parallel
 * drafters propose a whole block [SpecPilot news piece, wireai.ir — "The main challenge"]; tree
 * drafters propose a tree in which every token is conditioned on the path leading to it
 * [JetSpec article — "Technical architecture"]. Verification is lossless in the greedy sense:
 * every emitted token is the target's greedy choice [SpecPilot digest, airadar.tv — "Risks"].
 * So one call scores a draft tree of k nodes per request against the request's KV cache and
 * accepts the deepest root path whose every token equals the target's argmax given that path.
 * At batch 1 that pass reads all target weights for a few tokens, and per-request overhead is
 * what erodes batched speedups [SpecPilot digest — summary paragraph]: the library therefore
 * runs every request of a batch in the same kernels, with no per-request launches and no host
 * synchronisation.
 *
 * Target model (the pages fix none): pre-norm decoder, RMSNorm, rotate-half RoPE, grouped-query
 * attention, SwiGLU MLP, untied embedding and output head, bf16 weights, fp32 accumulation.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked HOST. Every call only enqueues work on
 *     `stream` and returns; outputs are valid once the stream work has completed.
 *   - The library never allocates or frees device memory; the caller owns every buffer and must
 *     keep it alive until the enqueued work completes. Scratch comes from `workspace`.
 *   - Problems visible on the host (NULL pointer, unsupported shape, small workspace) return a
 *     negative SPEC_E* code and enqueue nothing. Problems visible only in device data (a token
 *     outside the vocabulary, a malformed tree, a context that does not fit the request's
 *     pages) mark that request alone: its accepted_len and bonus_token become -1, its path all
 *     -1, its KV cache is not written; other requests in the batch proceed normally.
 *   - Calls on different streams with disjoint outputs and workspaces may run concurrently; the
 *     library keeps no global state.
 *   - bf16 = IEEE binary32 truncated to its upper 16 bits (storage), rounded to nearest even.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define SPEC_OK 0
#define SPEC_EINVAL (-1)        /* NULL pointer, negative size, malformed argument */
#define SPEC_EUNSUPPORTED (-2)  /* a shape this build does not implement (see spec_verify) */
#define SPEC_EWORKSPACE (-3)    /* workspace smaller than the *_workspace_bytes answer */
#define SPEC_EHIP (-4)          /* a HIP launch or runtime call failed */
#define SPEC_ESCRATCH (-5)      /* larger than the fixed scratch of spec_accept_noalloc */

#define SPEC_PAGE_SIZE 16       /* tokens per KV page */
#define SPEC_MAX_K 64           /* draft nodes per request (one 64-bit ancestor mask per node) */

/* Model shape. Supported: head_dim in {64, 128}; n_q_heads a multiple of n_kv_heads;
 * hidden a multiple of 64 and <= 16384; n_q_heads*head_dim and ffn multiples of 32; vocab a
 * multiple of 64. The workspace must be 256-byte aligned. */
typedef struct {
    int n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
    float rms_eps;              /* RMSNorm epsilon, added to mean(x^2) */
    double rope_theta;          /* RoPE base: pair j of a head turns by pos * theta^(-2j/d) */
} spec_model_cfg;

/* One decoder layer, all bf16 (DEVICE pointers). Logical shapes, [out][in]:
 *   attn_norm [H]; w_qkv [(nq + 2 nkv) d][H] rows = q heads, then k heads, then v heads;
 *   w_o [H][nq d]; mlp_norm [H]; w_gate_up [2F][H] rows = F gate rows, then F up rows;
 *   w_down [H][F].
 * The four projection matrices (and spec_weights.lm_head) are passed PACKED: converted once,
 * at load time, from row-major [out][in] by spec_pack_weight. The norms and the embedding table
 * stay row-major. */
typedef struct {
    const void *attn_norm, *w_qkv, *w_o, *mlp_norm, *w_gate_up, *w_down;
} spec_layer_weights;

/* One projection matrix [n][kd] in W12, the lossless 12-bit layout built by spec_w12_plan and
 * spec_w12_pack (DEVICE pointers): planes (n*kd*3/2 bytes), plan (spec_w12_plan_ints ints),
 * exc (2 ints per exception). */
typedef struct {
    const void *planes;
    const int32_t *plan;
    const int32_t *exc;
} spec_w12_matrix;

typedef struct {
    spec_w12_matrix w_qkv, w_o, w_gate_up, w_down;
} spec_w12_layer;

typedef struct {
    spec_model_cfg cfg;
    const spec_layer_weights *layers;   /* HOST array of cfg.n_layers entries */
    const void *embed;                  /* bf16 [V][H], row-major */
    const void *final_norm;             /* bf16 [H] */
    const void *lm_head;                /* bf16 [V][H], packed (spec_pack_weight); may be NULL
                                           when w12_lm_head.planes is set */
    /* Optional W12 projections. w12_layers: HOST array of cfg.n_layers entries or NULL; when
     * set, the four projections of every layer are streamed from it and the w_qkv, w_o,
     * w_gate_up and w_down members of `layers` are ignored (they may be NULL). w12_lm_head:
     * used when its planes member is set. W12 needs batch * k <= 64 (SPEC_EUNSUPPORTED
     * otherwise). The results are bit-identical to the bf16 pass over the same weights. */
    const spec_w12_layer *w12_layers;
    spec_w12_matrix w12_lm_head;
    /* Hybrid targets: HOST array of cfg.n_layers entries, or NULL (every layer attention).
     * SPEC_LAYER_RECURRENT marks a layer whose attention mixer is replaced by the gated linear
     * recurrence of spec_rec_tree_verify (the reading below, "Recurrent layers"): its w_qkv is
     * [R][H] packed, R = 3 nq d + nq rounded up to a multiple of 16, rows = q heads, k heads,
     * v heads (nq = n_q_heads each), one gate row per head, then zero rows; its w_o [H][nq d];
     * the other members as an attention layer's. Per head: g = -softplus(bf16(gate input)) in
     * fp32 (-a above a = 20), S <- e^g S + k v^T along each node's root path from the committed
     * state, o = S^T q rounded to bf16, x += o . W_o^T. No RoPE, no cache rows. Recurrent layers
     * need bf16 weights (no W12) and the per-step plan. */
    const int32_t *layer_kind;
} spec_weights;

#define SPEC_LAYER_ATTENTION 0
#define SPEC_LAYER_RECURRENT 1

/* Paged KV cache, bf16. A page holds SPEC_PAGE_SIZE consecutive positions of one request.
 *   k_pool [n_layers][n_pages][n_kv_heads][16][head_dim]   (keys, one row per position)
 *   v_pool [n_layers][n_pages][n_kv_heads][head_dim][16]   (values, transposed in the page)
 *   block_table [batch][max_pages_per_req]: page ids; position p of request b lives in page
 *   block_table[b][p / 16], slot p % 16. Keys are stored after RoPE. */
typedef struct {
    void *k_pool;
    void *v_pool;
    const int32_t *block_table;
    int n_pages;
    int max_pages_per_req;
    /* Recurrent layers of a hybrid target (all NULL for a dense one):
     *   rec_state: HOST array of n_layers DEVICE pointers; for a recurrent layer l the committed
     *   state fp32 [batch][nq][d][d], each head's S stored transposed as spec_rec_tree_verify
     *   reads it; NULL for attention layers. spec_verify reads it; spec_commit_kv advances it.
     *   rec_k, rec_v (bf16) [n_layers][batch][k][nq][d] and rec_g (fp32) [n_layers][batch][k][nq]:
     *   written by spec_verify for each recurrent layer (that pass's keys, values and log-gates,
     *   node order), read by spec_commit_kv with the same batch and k. The page pools keep their
     *   n_layers layout; a recurrent layer's pages hold no rows. */
    float *const *rec_state;
    void *rec_k;
    void *rec_v;
    float *rec_g;
} spec_kv_cache;

/* Optional extra outputs of spec_verify (any member may be NULL; the struct pointer too). */
typedef struct {
    float *logits;          /* fp32 [batch*k][vocab]: the target's logits for every draft node */
    int32_t *greedy;        /* int32 [batch*k]: argmax of each node's logits (lowest index) */
    void *hidden;           /* bf16 [n_layers + 1][batch*k][hidden]: residual stream entering
                               each layer, then after the last layer (before the final norm) */
    hipEvent_t *gate_up_events;  /* HOST array of 2 * n_layers events or NULL: events[2l] is
                               recorded on `stream` right before layer l's gate/up projection
                               kernel and events[2l+1] right after it, for per-launch timing
                               of the pass's largest kernel. Time eager calls: events captured
                               into a HIP graph are not ordered against its kernels. Used by the
                               per-step path only. */
    int path;               /* SPEC_PATH_AUTO (0): the library's choice (currently the per-step
                               path); SPEC_PATH_STEPS: one kernel per step of each layer;
                               SPEC_PATH_PERSISTENT: SPEC_EUNSUPPORTED where it does not apply. */
    hipEvent_t *layer_events;   /* HOST array of 2 * ceil(n_layers / 16) events or NULL: recorded
                               on `stream` right before and right after each launch of the
                               persistent layers kernel (persistent path only; eager calls). */
    uint64_t *phase_trace;  /* device, persistent path only, or NULL: uint64 [n_layers][G][24]
                               with G = the device's compute units (at most 512), the
                               s_memrealtime ticks (100 MHz) at which workgroup w reached each
                               phase boundary of layer l: QKV wait begin, inputs ready, main loop
                               end, done (0-3); attention items done (4); merges done (5); the same
                               four for O (6-9), gate/up (10-13) and down (14-17); inside the
                               workgroup's (last) attention item: inputs ready, keys and values
                               staged, products done (18-20); inside its (last) merge task:
                               inputs ready, output written (21-22); 23 unused. Entries of
                               workgroups without that work are left unwritten. */
} spec_verify_extras;

/* The two launch plans of spec_verify. Both compute the same pass with the same arithmetic;
 * only the order of some fp32 sums differs.
 *  - Per-step (SPEC_PATH_STEPS): every step of a layer (projection, split-K add with RoPE and
 *    the K/V write, attention and its merge, residual add with RMSNorm) is its own kernel.
 *  - Persistent (SPEC_PATH_PERSISTENT): for batch * k <= 16 rows (a block of up to 16 draft
 *    tokens, or a few small blocks or trees), head_dim 64 or 128 and at most 8 query heads per kv
 *    head, bf16 weights: one kernel per group of up to 16 layers, one workgroup per compute
 *    unit, whose steps hand data to each other through memory inside the kernel. It needs the
 *    whole GPU while it runs: if work on other streams holds compute units so that its
 *    workgroups cannot all be resident, its bounded waits expire after about one second and
 *    every request of the call is reported failed (accepted_len = bonus = -1). */
#define SPEC_PATH_AUTO 0
#define SPEC_PATH_STEPS 1
#define SPEC_PATH_PERSISTENT 2

/* Workspace bytes spec_verify needs for this shape, batch, k and cache page budget per request
 * (kv->max_pages_per_req of the calls it will serve). HOST out-pointer. The library never
 * allocates: a pass reads every weight for a handful of tokens at batch 1 and per-request
 * overhead erodes batched gains [SpecPilot digest, airadar.tv — summary paragraph], so all
 * scratch of a call (residual stream, split-K partials, attention partials sized by the page
 * budget) comes from this one caller buffer. */
int spec_workspace_bytes(const spec_model_cfg *cfg, int batch, int k, int max_pages_per_req,
                         size_t *bytes);

/* One verification pass.
 *   draft_tokens [batch][k]: node 0 of each request is the root, the last committed token
 *       (its K/V is not yet in the cache); nodes 1..k-1 are draft tokens.
 *   tree_parent  [batch][k] or NULL: parent[0] = -1 and 0 <= parent[i] < i (nodes in
 *       topological order, one root). NULL means a linear block (parent[i] = i - 1).
 *   ctx_len      [batch]: committed positions per request. Node i sits at position
 *       ctx_len + depth(i). The caller must provide pages for positions [0, ctx_len + k).
 * Effects: writes every node's rotated key and value into cache slots ctx_len .. ctx_len+k-1
 *   (node order) of every layer. Outputs per request:
 *   accepted_len [batch]: accepted draft tokens on the deepest accepted root path, 0..k-1 (the
 *       root is not counted); bonus_token [batch]: the target's greedy token after that path's
 *       last node; accepted_path [batch][k]: node ids of that path from the root, then -1.
 *   Equal-depth accepted nodes (possible only with duplicate sibling tokens) resolve to the
 *   lowest node id. Arithmetic: bf16 storage between steps, fp32 accumulation and softmax.
 * Hybrid targets (weights->layer_kind marks recurrent layers): each recurrent layer reads its
 *   committed state from kv->rec_state and writes the pass's keys, values and log-gates to
 *   kv->rec_k / rec_v / rec_g (no cache rows); SPEC_EINVAL when those are missing,
 *   SPEC_EUNSUPPORTED with W12 weights or the persistent plan.
 * Shapes: 1 <= k <= SPEC_MAX_K; batch >= 1. */
int spec_verify(const spec_weights *weights, const spec_kv_cache *kv,
                const int32_t *draft_tokens, const int32_t *tree_parent, const int32_t *ctx_len,
                int batch, int k,
                int32_t *accepted_len, int32_t *bonus_token, int32_t *accepted_path,
                const spec_verify_extras *extras /* HOST, may be NULL */,
                void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Commit the accepted path into the cache. Only the accepted root path becomes context: a draft
 * token is kept only if it and every earlier token of its path equal the target's greedy
 * choice [SpecPilot digest, airadar.tv — "Risks"], and a tree token's K/V row was computed for
 * its own root path [JetSpec article, seventnews.com — "Technical architecture"]. For every
 * layer, K and V, slot ctx_len + t receives the row of slot ctx_len + accepted_path[t],
 * t = 0..accepted_len (every source is read before any slot is written); then
 * ctx_len += accepted_len + 1, on the device.
 * A request's commit is all or nothing. It applies only when 0 <= accepted_len < k,
 * accepted_path[0] = 0 and t <= accepted_path[t] < k for t = 1..accepted_len (node ids are
 * topological, so the node at depth t has id >= t), ctx_len >= 0, ctx_len + k fits
 * max_pages_per_req pages, and the pages of positions ctx_len .. ctx_len + k - 1 are valid
 * ids. Any other request (e.g. accepted_len = -1 from a failed verify) keeps its rows and its
 * ctx_len. Device pointers: accepted_len [batch], accepted_path [batch][k], ctx_len [batch]
 * (in/out). Takes the outputs of spec_verify on the same stream; k and batch as given to it.
 * Hybrid targets (kv->rec_state set): each recurrent layer's state then becomes the state after
 * the accepted path, applied from the committed one with that pass's kv->rec_k, rec_v and rec_g
 * (spec_rec_commit's rule: 0 <= accepted_len < k and node ids in [0, k), else the state is
 * kept; a request that failed in spec_verify has accepted_len -1 and keeps both).
 * Host-side errors (NULL pointers, batch or k < 1, k > SPEC_MAX_K, a bad cfg, a recurrent
 * state without the pass's buffers) return before anything is enqueued. */
int spec_commit_kv(const spec_model_cfg *cfg, const spec_kv_cache *kv,
                   const int32_t *accepted_len, const int32_t *accepted_path, int32_t *ctx_len,
                   int batch, int k, hipStream_t stream);

/* Workspace bytes spec_accept needs. HOST out-pointer. */
int spec_accept_workspace_bytes(int batch, int k, int vocab, size_t *bytes);

/* The acceptance half of spec_verify on caller-supplied logits: per node the greedy token
 * (lowest index of the row maximum), then the accepted-path walk, with the same outputs and
 * conventions as spec_verify. A draft token is kept only while it and every earlier token of its
 * root path equal the target's greedy choice [SpecPilot digest, airadar.tv — "Risks"], each tree
 * node judged on its own path [JetSpec article, seventnews.com — "Technical architecture"].
 * logits: fp32 [batch*k][vocab]. */
int spec_accept(const float *logits, const int32_t *draft_tokens, const int32_t *tree_parent,
                int batch, int k, int vocab,
                int32_t *accepted_len, int32_t *bonus_token, int32_t *accepted_path,
                int32_t *greedy /* [batch*k] or NULL */,
                void *workspace, size_t workspace_bytes, hipStream_t stream);

/* spec_accept without a workspace argument and without any allocation, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same inputs, outputs, kernels and results as spec_accept; its scratch (the
 * per-node tree bookkeeping and the per-chunk greedy partials) is a static device array of the
 * library, SPEC_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends. Limits:
 * batch * k <= SPEC_NOALLOC_MAX_ROWS and vocab <= SPEC_NOALLOC_MAX_VOCAB, else SPEC_ESCRATCH
 * (returned before anything is enqueued). The current device must be the one `stream` belongs
 * to. Every call on one GPU shares that GPU's scratch and nothing in it needs to start at zero;
 * calls that overlap on one GPU (other streams, other threads) race and must be serialised by
 * the caller. Other errors as for spec_accept. */
#define SPEC_NOALLOC_MAX_ROWS 4096
#define SPEC_NOALLOC_MAX_VOCAB 262144
#define SPEC_NOALLOC_SCRATCH_BYTES ((size_t)4276224)
int spec_accept_noalloc(const float *logits, const int32_t *draft_tokens,
                        const int32_t *tree_parent, int batch, int k, int vocab,
                        int32_t *accepted_len, int32_t *bonus_token, int32_t *accepted_path,
                        int32_t *greedy /* [batch*k] or NULL */, hipStream_t stream);

/* Convert one projection matrix from row-major w [n][kd] bf16 into the packed layout the
 * verify kernels stream (same size, n*kd*2 bytes, at `packed`, which must not overlap `w`).
 * Packed order: for every tile of 16 rows (tile t = rows 16t..16t+15) and every step of 32
 * columns (s = columns 32s..32s+31), in that nesting, 64 slots of 8 consecutive bf16; slot l
 * holds w[16t + l%16][32s + 8(l/16) .. + 7]. One 128-bit load per lane of a 64-wide wavefront
 * then fetches one matrix-core operand as 1 KB of contiguous memory. Needs n % 16 == 0 and
 * kd % 32 == 0 (SPEC_EUNSUPPORTED otherwise) and 16-byte aligned w and packed (SPEC_EINVAL).
 * A one-time, load-time transform; enqueued on `stream`. */
int spec_pack_weight(const void *w, int n, int kd, void *packed, hipStream_t stream);

/* The weight-streaming projection spec_verify runs for every weight matrix, on its own:
 * partials[s][m][n] = sum, over split s's share of the reduction dimension, of x[m][j]*w[n][j]
 * (bf16 operands, fp32 sums), with the split count spec_verify picks for this shape; the
 * projection is the sum of the splits in index order. A single pass at batch 1 reads every
 * weight once for a few rows [SpecPilot digest, airadar.tv — summary paragraph], so this is the
 * kernel whose HBM bandwidth the pass lives on. For kernel-level tests and bandwidth
 * measurement.
 *   x: bf16 [m][kd] row-major; w: bf16 [n][kd] packed (spec_pack_weight); partials: a
 *   256-byte aligned buffer of spec_skinny_gemm_bytes() bytes, whose first splits*m*n floats
 *   receive the partial sums (the rest holds a fragment-order copy of x); *splits (HOST)
 *   receives the split count. Needs kd % 32 == 0, n % 16 == 0, m >= 1. */
int spec_skinny_gemm_bytes(int m, int n, int kd, size_t *bytes);
int spec_skinny_gemm(const void *x, int m, int kd, const void *w, int n, float *partials,
                     size_t partial_bytes, int *splits, hipStream_t stream);

/* Measurement aid: reads `bytes` of device memory once as a plain grid-stride stream of 16-byte
 * loads (the access pattern DRAM serves best) and folds them into a word that is written to
 * *out (a DEVICE uint32) only in the unlikely case that it equals a fixed constant, so the loads
 * cannot be dropped. Its rate is the streaming-read ceiling the projection kernels are compared
 * against. buf must be 16-byte aligned and bytes a multiple of 16; returns SPEC_EINVAL
 * otherwise. Enqueued on `stream`. */
int spec_read_probe(const void *buf, size_t bytes, uint32_t *out, hipStream_t stream);

/* ---- W12: lossless 12-bit weights -------------------------------------------------------------
 * The SpecPilot digest (airadar.tv — "Reasons") names a lossless 12-bit weight format: every
 * bf16 weight split into three 4-bit planes that the GEMM rebuilds bit for bit in registers, so
 * that a weight-bound batch-1 pass streams a quarter fewer bytes. The pages fix neither the
 * planes' contents nor what happens to values that do not fit; this library's layout:
 *   - one window of 16 exponent fields [b, b+15] per matrix, b even (0..240), the one that
 *     leaves the fewest values outside (lowest b on ties);
 *   - planes 0 and 1: the value's low byte (mantissa, lowest exponent bit), as is; plane 2: the
 *     nibble (sign, (e - b) >> 1);
 *   - a value outside the window is an exception: its planes hold its low byte and a zero
 *     nibble, and exc holds (position, bf16 bits) pairs sorted by tile, then position, where
 *     position = s * 512 + l * 8 + j for value j of slot l of step s (the slots of
 *     spec_pack_weight's order);
 *   - planes: fragment (tile t, step s) of spec_pack_weight's order is 768 bytes at
 *     (t * (kd/32) + s) * 768, 12 bytes per slot l at 12 l: a dword of the low bytes of values
 *     0..3 (byte j = value j), a dword of values 4..7, a dword of nibbles (value 2i at bits
 *     4i..4i+3, value 2i+1 at bits 16+4i..16+4i+3);
 *   - plan (int32): [0] b, [1] exception count E, [2 .. 2 + n/16] per-tile exception offsets
 *     (exclusive prefix, n/16 + 1 entries), then 256 ints of scratch.
 * The format pays where the window holds nearly every weight (about 1e-4 of N(0, 0.02) weights
 * are exceptions); read plan[1] after spec_w12_plan to decide, and to size exc (2*E ints).
 * Needs n % 16 == 0 and kd % 32 == 0 (SPEC_EUNSUPPORTED), a 16-byte aligned w, 16-byte aligned
 * planes and 8-byte aligned exc (SPEC_EINVAL). One-time, load-time transforms, enqueued on
 * `stream`. */
int spec_w12_plan_ints(int n, int kd, size_t *ints /* HOST */);
int spec_w12_plan(const void *w /* bf16 [n][kd] row-major */, int n, int kd, int32_t *plan,
                  hipStream_t stream);
int spec_w12_pack(const void *w /* bf16 [n][kd] row-major */, int n, int kd, const int32_t *plan,
                  void *planes, int32_t *exc, hipStream_t stream);

/* spec_skinny_gemm over a W12 matrix: the same partials, bit for bit, as spec_skinny_gemm over
 * the bf16 matrix it encodes for m < 128 (same kernels, tiles and splits). From 128 rows
 * spec_skinny_gemm switches to its matrix-core tile kernel while W12 keeps 64-row chunks; the
 * split count may then differ, and partial_bytes as spec_skinny_gemm_bytes gives covers both. */
int spec_skinny_gemm_w12(const void *x, int m, int kd, const spec_w12_matrix *w, int n,
                         float *partials, size_t partial_bytes, int *splits, hipStream_t stream);

/* ---- Prefill: a prompt's K/V ahead of the first verify step ----------------------------------
 * Appends p prompt tokens per request to its committed context: writes their rotated keys and
 * values into cache slots ctx_len .. ctx_len + p - 1 of every layer, returns the target's greedy
 * token after the last prompt token (the root of the first verify step) and sets
 * ctx_len += p on the device. Every prompt position is a node whose tokens are all given and all
 * kept: it attends to the committed context and the positions before it, as a fully accepted
 * linear block does in a verify pass [SpecPilot news piece, wireai.ir — "The main challenge"].
 * The prompt runs in chunks of up to 4096 positions per pass (over all requests: 4096 / batch
 * per request), each chunk's K/V written before its attention reads them; the projections run
 * on the matrix cores, attention is causal over the paged cache, and the output head runs only
 * for each request's last position.
 *   prompt [batch][p] int32; ctx_len [batch] in/out; next_token [batch] out (-1 for a request
 *   whose prompt holds a token outside the vocabulary or whose pages do not cover
 *   ctx_len + p: its ctx_len is left where its last good chunk ended and its cache rows past it
 *   are unspecified); last_logits [batch][vocab] fp32 or NULL: the last prompt position's
 *   logits. Weights as for spec_verify (bf16 or W12), attention layers only (SPEC_EUNSUPPORTED
 *   for a recurrent layer, or for more than 8 query heads per kv head).
 * spec_prefill_workspace_bytes: the workspace for `batch` requests whose prompts may reach
 *   max_pages_per_req * 16 positions; it does not depend on want_logits (the logits go straight
 *   to the caller's buffer). Errors as for spec_verify: SPEC_EINVAL for NULL pointers, a
 *   workspace that is not 256-byte aligned, batch or p below 1; SPEC_EWORKSPACE for a short
 *   workspace. weights and kv are host structs as for spec_verify; prompt, ctx_len, next_token,
 *   last_logits and workspace are device pointers. Async on stream; calls that overlap on one
 *   cache race. */
int spec_prefill_workspace_bytes(const spec_model_cfg *cfg, int batch, int max_pages_per_req,
                                 int want_logits, size_t *bytes /* HOST */);
int spec_prefill(const spec_weights *weights, const spec_kv_cache *kv, const int32_t *prompt,
                 int32_t *ctx_len, int batch, int p, int32_t *next_token, float *last_logits,
                 void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- Recurrent layers of a hybrid target ------------------------------------------------------
 * The SpecPilot digest (airadar.tv — "Reasons") names tree verification for targets that mix
 * recurrent layers in, without giving the recurrence. This library's reading: per head, a
 * scalar-gated linear recurrence over a state S [dk][dv] (fp32),
 *     S <- exp(g) S + k v^T, then o = S^T q, for each token,
 * where every node of a draft tree continues its parent's state and the root continues the
 * committed one (the tree is conditioned on paths as for attention [JetSpec article,
 * seventnews.com — "Technical architecture"]). dk = dv = head_dim, 64 or 128.
 *
 * spec_rec_tree_verify: one recurrent layer over a draft tree, reading the committed state once
 * and writing no per-node state.
 *   state: S stored transposed, [batch][n_heads][dv][dk] fp32 (element [c][r] holds S[r][c],
 *   so each value column's dk entries are contiguous; read only); q, k, v
 *   [batch][k][n_heads][head_dim] bf16; log_gate [batch][k][n_heads] fp32 (g, normally <= 0);
 *   tree_parent [batch][k] int32 as for spec_verify, or NULL for chains; out
 *   [batch][k][n_heads][head_dim] fp32; status [batch] int32 out: 0, or 1 for a malformed tree
 *   (that request's outputs are zero).
 * spec_rec_commit: the state of each request's accepted node, written over state in place (same
 *   transposed layout):
 *   the tokens accepted_path[b][0..accepted_len[b]] (node ids as spec_verify returns them)
 *   applied to the committed state. A request with accepted_len < 0, accepted_len >= k, or a
 *   node id outside [0, k) keeps its state. k, v, log_gate as passed to the verify call.
 * Both: device pointers, 16-byte aligned; async on stream; k <= 64 (SPEC_EUNSUPPORTED past it
 * or for another head_dim); SPEC_EINVAL for NULL pointers, misalignment or batch, k or n_heads
 * below 1. Calls that overlap on one state buffer race. */
int spec_rec_tree_verify(const float *state, const void *q, const void *k, const void *v,
                         const float *log_gate, const int32_t *tree_parent, int batch, int k_nodes,
                         int n_heads, int head_dim, float *out, int32_t *status, hipStream_t stream);
int spec_rec_commit(float *state, const void *k, const void *v, const float *log_gate,
                    const int32_t *accepted_len, const int32_t *accepted_path, int batch,
                    int k_nodes, int n_heads, int head_dim, hipStream_t stream);

/* Static text for a return code. */
const char *spec_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
