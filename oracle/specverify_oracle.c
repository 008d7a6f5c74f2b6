/*
 * specverify_oracle.c — plain, slow CPU oracle for the verification step of lossless greedy
 * speculative decoding.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark load this library. The product (the HIP library) never does, and the two share no
 * source, header, table or helper.
 *
 * What is computed, and where the pages say so:
 *   - A drafter proposes several tokens and the target checks all of them at once, in one pass
 *     [JetSpec article, seventnews.com — opening section]. Parallel drafters propose a whole
 *     block per step [SpecPilot news piece, wireai.ir — "The main challenge"]; tree drafters
 *     propose a tree in which every token is conditioned on the path that leads to it
 *     [JetSpec article — "Technical architecture"].
 *   - "Lossless" means every emitted token is the target's greedy choice, although a different
 *     order of computation in batched verification may flip near-ties
 *     [SpecPilot digest, airadar.tv — "Risks"].
 * Hence the plain definition this file writes out: the accepted path is the deepest root path
 * of the draft tree whose every token equals the target's greedy argmax given that path, which
 * is exactly what one-token-at-a-time greedy decoding would have emitted.
 *
 * The pages fix no model. The target is a pre-norm decoder (RMSNorm, rotate-half RoPE,
 * grouped-query attention, SwiGLU MLP, untied embedding and output head), stored in bf16.
 *
 * Precision (the reading used throughout): bf16 storage, round-to-nearest-even, at every tensor
 * boundary; products of bf16 values and their sums in fp32, summed in ascending index order;
 * softmax in fp32; logits in fp32, never rounded. Every output row depends only on its own
 * inputs and its ancestors, never on how many rows are processed together, so a block pass, a
 * chain-tree pass and one-token-at-a-time decoding give bit-identical results.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp (no fast-math). OpenMP splits work only over
 * independent output elements; every reduction stays in one thread, in index order.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------------ */
/* bf16 <-> fp32                                                                              */
/* ------------------------------------------------------------------------------------------ */

/* A bf16 value is the top 16 bits of an IEEE binary32. */
static float bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round a binary32 to the nearest bf16, ties to even; NaN stays a (quiet) NaN. */
static uint16_t f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

/* Threads the OpenMP loops below use. */
int orc_max_threads(void) { return omp_get_max_threads(); }

/* Threads of the following parallel loops (timing at one thread and at all cores). */
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

void orc_f32_to_bf16(const float *in, uint16_t *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16(in[i]);
}

void orc_bf16_to_f32(const uint16_t *in, float *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_to_f32(in[i]);
}

/* ------------------------------------------------------------------------------------------ */
/* Model description                                                                          */
/* ------------------------------------------------------------------------------------------ */

typedef struct {
    int n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
    float rms_eps;
    double rope_theta;
} orc_cfg;

/* One decoder layer. Row-major matrices, out-features x in-features:
 *   w_qkv     [(nq + 2 nkv) d][H]  rows: all q heads, then all k heads, then all v heads
 *   w_o       [H][nq d]
 *   w_gate_up [2F][H]              rows: F gate rows, then F up rows
 *   w_down    [H][F]
 * attn_norm, mlp_norm: [H] RMSNorm gains. */
typedef struct {
    const uint16_t *attn_norm, *w_qkv, *w_o, *mlp_norm, *w_gate_up, *w_down;
} orc_layer_w;

/* ------------------------------------------------------------------------------------------ */
/* Draft tree                                                                                 */
/* ------------------------------------------------------------------------------------------ */

/* Node 0 is the root (parent -1): the last committed token, whose K/V is not cached yet.
 * Every other node names an earlier node as parent (0 <= parent[i] < i), so one left-to-right
 * sweep gives the depths. Returns 0, or -1 for a malformed tree. A chain is parent[i] = i - 1. */
int orc_tree_depth(const int32_t *parent, int k, int32_t *depth) {
    if (k < 1 || parent[0] != -1) return -1;
    depth[0] = 0;
    for (int i = 1; i < k; ++i) {
        if (parent[i] < 0 || parent[i] >= i) return -1;
        depth[i] = depth[parent[i]] + 1;
    }
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Building blocks                                                                            */
/* ------------------------------------------------------------------------------------------ */

/* RMSNorm of each row: out = bf16((x / sqrt(mean(x^2) + eps)) * g). */
void orc_rmsnorm(const uint16_t *x, const uint16_t *g, int rows, int h, float eps, uint16_t *out) {
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r) {
        const uint16_t *xr = x + (int64_t)r * h;
        float ss = 0.0f;
        for (int j = 0; j < h; ++j) {
            float v = bf16_to_f32(xr[j]);
            ss += v * v;
        }
        float inv = 1.0f / sqrtf(ss / (float)h + eps);
        for (int j = 0; j < h; ++j)
            out[(int64_t)r * h + j] = f32_to_bf16((bf16_to_f32(xr[j]) * inv) * bf16_to_f32(g[j]));
    }
}

/* y[i][n] = sum_k x[i][k] * w[n][k], fp32, k ascending. x: [m][kd] bf16, w: [n][kd] bf16,
 * y: [m][n] fp32. Each of the m sums for weight row n runs in its own accumulator. */
void orc_linear(const uint16_t *x, int m, int kd, const uint16_t *w, int n, float *y) {
    float *xt = (float *)malloc(sizeof(float) * (size_t)kd * (size_t)m);
    for (int i = 0; i < m; ++i)
        for (int k = 0; k < kd; ++k) xt[(int64_t)k * m + i] = bf16_to_f32(x[(int64_t)i * kd + k]);
#pragma omp parallel
    {
        float *acc = (float *)malloc(sizeof(float) * (size_t)m);
#pragma omp for schedule(static)
        for (int r = 0; r < n; ++r) {
            const uint16_t *wr = w + (int64_t)r * kd;
            for (int i = 0; i < m; ++i) acc[i] = 0.0f;
            for (int k = 0; k < kd; ++k) {
                float wk = bf16_to_f32(wr[k]);
                const float *xk = xt + (int64_t)k * m;
                for (int i = 0; i < m; ++i) acc[i] += xk[i] * wk;
            }
            for (int i = 0; i < m; ++i) y[(int64_t)i * n + r] = acc[i];
        }
        free(acc);
    }
    free(xt);
}

/* Rotate-half rotary embedding, in place on t: [m][nh][d] bf16, token i at position pos[i].
 * Pair (j, j + d/2) of every head turns by angle pos * theta^(-2j/d); the angle, its cosine and
 * its sine are taken in double, then the rotation itself in fp32 and the result rounded. */
void orc_rope(uint16_t *t, const int32_t *pos, int m, int nh, int d, double theta) {
    int half = d / 2;
    for (int i = 0; i < m; ++i) {
        for (int j = 0; j < half; ++j) {
            double inv_freq = pow(theta, -2.0 * (double)j / (double)d);
            double ang = (double)pos[i] * inv_freq;
            float c = (float)cos(ang), s = (float)sin(ang);
            for (int h = 0; h < nh; ++h) {
                uint16_t *th = t + ((int64_t)i * nh + h) * d;
                float a = bf16_to_f32(th[j]), b = bf16_to_f32(th[j + half]);
                float ra = a * c - b * s;
                float rb = b * c + a * s;
                th[j] = f32_to_bf16(ra);
                th[j + half] = f32_to_bf16(rb);
            }
        }
    }
}

/* Attention of draft node i over the committed context plus its own root path.
 *   q:            [m][nq][d] bf16 (already rotated)
 *   k_ctx, v_ctx: [ctx][nkv][d] bf16, positions 0..ctx-1
 *   k_new, v_new: [m][nkv][d] bf16, the draft nodes' own keys and values (node order)
 *   parent:       [m] tree parents; node i sees the nodes on the path root..i
 *   o:            [m][nq][d] bf16 out
 * Query head h reads kv head h / (nq / nkv). Keys are visited in position order: the context,
 * then the path from the root down to i. s_j = (q . k_j) / sqrt(d) in fp32; p_j = exp(s_j - max);
 * o = (sum_j p_j v_j) / (sum_j p_j), rounded once. */
void orc_attention(const uint16_t *q, const uint16_t *k_ctx, const uint16_t *v_ctx, int ctx,
                   const uint16_t *k_new, const uint16_t *v_new, const int32_t *parent, int m,
                   int nq, int nkv, int d, uint16_t *o) {
    int group = nq / nkv;
    float scale = 1.0f / sqrtf((float)d);
#pragma omp parallel
    {
        int *path = (int *)malloc(sizeof(int) * (size_t)m);
        float *s = (float *)malloc(sizeof(float) * ((size_t)ctx + (size_t)m));
        float *acc = (float *)malloc(sizeof(float) * (size_t)d);
#pragma omp for schedule(static) collapse(2)
        for (int i = 0; i < m; ++i) {
            for (int h = 0; h < nq; ++h) {
                /* path root..i, by walking parents up from i and reversing */
                int len = 0;
                for (int node = i; node >= 0; node = parent[node]) path[len++] = node;
                for (int a = 0, b = len - 1; a < b; ++a, --b) {
                    int tmp = path[a]; path[a] = path[b]; path[b] = tmp;
                }
                int g = h / group;
                const uint16_t *qh = q + ((int64_t)i * nq + h) * d;
                int nkeys = ctx + len;
                for (int j = 0; j < nkeys; ++j) {
                    const uint16_t *kj = (j < ctx) ? k_ctx + ((int64_t)j * nkv + g) * d
                                                   : k_new + ((int64_t)path[j - ctx] * nkv + g) * d;
                    float dot = 0.0f;
                    for (int e = 0; e < d; ++e) dot += bf16_to_f32(qh[e]) * bf16_to_f32(kj[e]);
                    s[j] = dot * scale;
                }
                float mx = s[0];
                for (int j = 1; j < nkeys; ++j) if (s[j] > mx) mx = s[j];
                float z = 0.0f;
                for (int e = 0; e < d; ++e) acc[e] = 0.0f;
                for (int j = 0; j < nkeys; ++j) {
                    float p = expf(s[j] - mx);
                    z += p;
                    const uint16_t *vj = (j < ctx) ? v_ctx + ((int64_t)j * nkv + g) * d
                                                   : v_new + ((int64_t)path[j - ctx] * nkv + g) * d;
                    for (int e = 0; e < d; ++e) acc[e] += p * bf16_to_f32(vj[e]);
                }
                uint16_t *oh = o + ((int64_t)i * nq + h) * d;
                for (int e = 0; e < d; ++e) oh[e] = f32_to_bf16(acc[e] / z);
            }
        }
        free(path);
        free(s);
        free(acc);
    }
}

/* SwiGLU gate: out = bf16(silu(gate) * up), silu(a) = a / (1 + exp(-a)); gate and up bf16. */
void orc_swiglu(const uint16_t *gate, const uint16_t *up, int64_t n, uint16_t *out) {
    for (int64_t i = 0; i < n; ++i) {
        float a = bf16_to_f32(gate[i]);
        float silu = a / (1.0f + expf(-a));
        out[i] = f32_to_bf16(silu * bf16_to_f32(up[i]));
    }
}

/* x = bf16(x + bf16(y)) elementwise: the residual add after a projection. */
static void residual_add(uint16_t *x, const float *y, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        x[i] = f32_to_bf16(bf16_to_f32(x[i]) + bf16_to_f32(f32_to_bf16(y[i])));
}

/* ------------------------------------------------------------------------------------------ */
/* One decoder layer over the m draft nodes of one request                                    */
/* ------------------------------------------------------------------------------------------ */

/* The MLP block: x += W_down . swiglu(gate, up), [gate | up] = RMSNorm(x) * mlp_norm . W_gate_up.
 * u [m][H], y [m][max(2F, H)], gate, up, hm [m][F]: scratch. */
static void mlp_block(const orc_cfg *c, const orc_layer_w *w, int m, uint16_t *x, uint16_t *u,
                      float *y, uint16_t *gate, uint16_t *up, uint16_t *hm) {
    int H = c->hidden, F = c->ffn;
    orc_rmsnorm(x, w->mlp_norm, m, H, c->rms_eps, u);
    orc_linear(u, m, H, w->w_gate_up, 2 * F, y);
    for (int i = 0; i < m; ++i)
        for (int j = 0; j < F; ++j) {
            gate[(int64_t)i * F + j] = f32_to_bf16(y[(int64_t)i * 2 * F + j]);
            up[(int64_t)i * F + j] = f32_to_bf16(y[(int64_t)i * 2 * F + F + j]);
        }
    orc_swiglu(gate, up, (int64_t)m * F, hm);
    orc_linear(hm, m, F, w->w_down, H, y);
    residual_add(x, y, (int64_t)m * H);
}

/* x: [m][H] residual stream in/out. k_ctx, v_ctx: this layer's committed cache [ctx][nkv][d].
 * k_new, v_new: [m][nkv][d] out, the draft nodes' rotated keys and their values, node order.
 * Node i sits at position ctx + depth(i). Returns 0, or -1 for a malformed tree. */
int orc_layer_forward(const orc_cfg *c, const orc_layer_w *w, const uint16_t *k_ctx,
                      const uint16_t *v_ctx, int ctx, const int32_t *parent, int m, uint16_t *x,
                      uint16_t *k_new, uint16_t *v_new) {
    int H = c->hidden, nq = c->n_q_heads, nkv = c->n_kv_heads, d = c->head_dim, F = c->ffn;
    int nqkv = (nq + 2 * nkv) * d;
    int32_t *depth = (int32_t *)malloc(sizeof(int32_t) * (size_t)m);
    int32_t *pos = (int32_t *)malloc(sizeof(int32_t) * (size_t)m);
    if (orc_tree_depth(parent, m, depth) != 0) {
        free(depth);
        free(pos);
        return -1;
    }
    for (int i = 0; i < m; ++i) pos[i] = ctx + depth[i];

    uint16_t *u = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)m * H);
    int ywidth = nqkv;
    if (2 * F > ywidth) ywidth = 2 * F;
    if (H > ywidth) ywidth = H;
    float *y = (float *)malloc(sizeof(float) * (size_t)m * ywidth);
    uint16_t *q = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)m * nq * d);
    uint16_t *o = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)m * nq * d);
    uint16_t *gate = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)m * F);
    uint16_t *up = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)m * F);
    uint16_t *hm = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)m * F);

    /* attention block */
    orc_rmsnorm(x, w->attn_norm, m, H, c->rms_eps, u);
    orc_linear(u, m, H, w->w_qkv, nqkv, y);
    for (int i = 0; i < m; ++i) {
        const float *yi = y + (int64_t)i * nqkv;
        for (int j = 0; j < nq * d; ++j) q[(int64_t)i * nq * d + j] = f32_to_bf16(yi[j]);
        for (int j = 0; j < nkv * d; ++j) {
            k_new[(int64_t)i * nkv * d + j] = f32_to_bf16(yi[nq * d + j]);
            v_new[(int64_t)i * nkv * d + j] = f32_to_bf16(yi[nq * d + nkv * d + j]);
        }
    }
    orc_rope(q, pos, m, nq, d, c->rope_theta);
    orc_rope(k_new, pos, m, nkv, d, c->rope_theta);
    orc_attention(q, k_ctx, v_ctx, ctx, k_new, v_new, parent, m, nq, nkv, d, o);
    orc_linear(o, m, nq * d, w->w_o, H, y);
    residual_add(x, y, (int64_t)m * H);

    mlp_block(c, w, m, x, u, y, gate, up, hm);

    free(depth); free(pos); free(u); free(y); free(q); free(o); free(gate); free(up); free(hm);
    return 0;
}

/* Token embedding: x[i] = E[tok[i]]. Returns -1 if a token is out of range. */
int orc_embed(const uint16_t *embed, int vocab, int h, const int32_t *tok, int m, uint16_t *x) {
    for (int i = 0; i < m; ++i) {
        if (tok[i] < 0 || tok[i] >= vocab) return -1;
        memcpy(x + (int64_t)i * h, embed + (int64_t)tok[i] * h, sizeof(uint16_t) * (size_t)h);
    }
    return 0;
}

/* Final RMSNorm and output head: logits[i][v] = norm(x_i) . W_lm[v], fp32, not rounded. */
void orc_logits(const orc_cfg *c, const uint16_t *final_norm, const uint16_t *lm_head,
                const uint16_t *x, int m, float *logits) {
    uint16_t *u = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)m * c->hidden);
    orc_rmsnorm(x, final_norm, m, c->hidden, c->rms_eps, u);
    orc_linear(u, m, c->hidden, lm_head, c->vocab, logits);
    free(u);
}

/* Greedy choice per row: the lowest index holding the row maximum, and the margin between the
 * largest and the second-largest value (0 when the maximum is held twice). */
void orc_argmax(const float *logits, int m, int vocab, int32_t *arg, float *margin) {
    for (int i = 0; i < m; ++i) {
        const float *r = logits + (int64_t)i * vocab;
        int best = 0;
        for (int v = 1; v < vocab; ++v) if (r[v] > r[best]) best = v;
        float second = -INFINITY;
        for (int v = 0; v < vocab; ++v) if (v != best && r[v] > second) second = r[v];
        arg[i] = best;
        if (margin) margin[i] = r[best] - second;
    }
}

/* Longest accepted root path. Node i is accepted when its parent is accepted and its token is
 * the target's greedy choice after the parent; the root is accepted by definition. The deepest
 * accepted node wins (lowest node id among equals). Outputs: the number of accepted draft
 * tokens (the root is not counted), the bonus token (the target's choice after the deepest
 * accepted node) and the node ids on the accepted path from the root, -1 after its end.
 * Returns 0, or -1 for a malformed tree (then the outputs are -1). */
int orc_accept(const int32_t *tok, const int32_t *parent, const int32_t *arg, int k,
               int32_t *accepted_len, int32_t *bonus, int32_t *path) {
    int32_t *depth = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
    char *ok = (char *)malloc((size_t)k);
    for (int i = 0; i < k; ++i) path[i] = -1;
    if (orc_tree_depth(parent, k, depth) != 0) {
        *accepted_len = -1;
        *bonus = -1;
        free(depth);
        free(ok);
        return -1;
    }
    ok[0] = 1;
    int best = 0;
    for (int i = 1; i < k; ++i) {
        ok[i] = ok[parent[i]] && tok[i] == arg[parent[i]];
        if (ok[i] && depth[i] > depth[best]) best = i;
    }
    *accepted_len = depth[best];
    *bonus = arg[best];
    for (int node = best; node >= 0; node = parent[node]) path[depth[node]] = node;
    free(depth);
    free(ok);
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* W12: lossless 12-bit storage of bf16 weights                                               */
/* ------------------------------------------------------------------------------------------ */
/*
 * The SpecPilot digest (airadar.tv — "Reasons") names a lossless 12-bit weight format, W12:
 * each bf16 weight is split into three 4-bit planes that the GEMM reassembles bit for bit in
 * registers. The pages give neither the planes' contents nor how values that do not fit are
 * kept. The reading implemented here:
 *   - a bf16 value is (sign s, exponent field e of 8 bits, mantissa m of 7 bits);
 *   - a matrix has one window of 16 consecutive exponent fields [b, b + 15], b even, b <= 240;
 *   - plane 0 holds bits 3..0 (mantissa low bits), plane 1 bits 7..4 (e's lowest bit and the
 *     mantissa's top three), plane 2 holds (s, (e - b) >> 1): since b is even, e >> 1 equals
 *     b / 2 + ((e - b) >> 1), so the upper byte of the value comes back with one add;
 *   - a value whose exponent field lies outside the window is an exception: its planes carry
 *     the low byte and a zero nibble, and its full 16 bits are kept in a separate list.
 * The window is the one that leaves the fewest exceptions (lowest b on ties).
 */

static int w12_in_window(uint16_t v, int b) {
    const int e = (v >> 7) & 0xff;
    return e >= b && e <= b + 15;
}

/* The even window base b in [0, 240] with the most values inside [b, b + 15]. */
int orc_w12_base(const uint16_t *w, int64_t n) {
    int64_t hist[256];
    memset(hist, 0, sizeof(hist));
    for (int64_t i = 0; i < n; ++i) hist[(w[i] >> 7) & 0xff] += 1;
    int best_b = 0;
    int64_t best = -1;
    for (int b = 0; b <= 240; b += 2) {
        int64_t c = 0;
        for (int e = b; e <= b + 15; ++e) c += hist[e];
        if (c > best) {
            best = c;
            best_b = b;
        }
    }
    return best_b;
}

/* Planes of n values for window base b: lo[i] = planes 1 and 0 (the low byte), nib[i] = plane
 * 2; esc[i] = 1 for an exception (then nib[i] = 0). Returns the number of exceptions. */
int64_t orc_w12_encode(const uint16_t *w, int64_t n, int b, uint8_t *lo, uint8_t *nib, uint8_t *esc) {
    int64_t ne = 0;
    for (int64_t i = 0; i < n; ++i) {
        const uint16_t v = w[i];
        lo[i] = (uint8_t)(v & 0xff);
        if (w12_in_window(v, b)) {
            const int e = (v >> 7) & 0xff;
            nib[i] = (uint8_t)(((v >> 15) << 3) | ((e - b) >> 1));
            esc[i] = 0;
        } else {
            nib[i] = 0;
            esc[i] = 1;
            ne += 1;
        }
    }
    return ne;
}

/* bf16 values back from the planes; then the exceptions (element index, 16-bit value) are put
 * in place. */
void orc_w12_decode(const uint8_t *lo, const uint8_t *nib, int64_t n, int b,
                    const int64_t *esc_idx, const uint16_t *esc_val, int64_t n_esc, uint16_t *out) {
    for (int64_t i = 0; i < n; ++i) {
        const int s = nib[i] >> 3;
        const int hi = (b >> 1) + (nib[i] & 7);     /* e >> 1 */
        out[i] = (uint16_t)((s << 15) | (hi << 8) | lo[i]);
    }
    for (int64_t j = 0; j < n_esc; ++j) out[esc_idx[j]] = esc_val[j];
}

/* ------------------------------------------------------------------------------------------ */
/* Recurrent layers of a hybrid target: tree verification by forking the state                 */
/* ------------------------------------------------------------------------------------------ */
/* The SpecPilot digest (airadar.tv — "Reasons") and news piece (wireai.ir — key innovations)
 * name tree verification for targets that mix recurrent layers in, without giving the
 * recurrence. The reading used here is a scalar-gated linear recurrence per head (the form of
 * gated linear attention and of Mamba-2's state-space layer): with a state S of dk x dv values,
 *     S <- a S + k v^T,   a = exp(g),   then   o = S^T q,
 * for each token, with q, k in R^dk, v in R^dv and the log-gate g <= 0 per (token, head).
 * In a draft tree every node continues its parent's state, and the root continues the committed
 * state S0. The oracle runs that definition as written: for each node it walks the node's root
 * path and applies the recurrence token by token from S0, in float64. Inputs q, k, v are bf16,
 * S0 and g fp32. Layouts: S0 [B][H][dk][dv], q and k [B][K][H][dk], v [B][K][H][dv],
 * g [B][K][H], out [B][K][H][dv]. */

/* Root path of node i (root first) into path[]; its length, or -1 if a parent link is
 * malformed (the root's parent must be -1, any other node's parent an earlier node). */
static int rec_path(const int32_t *parent, int k, int i, int *path) {
    int n = 0;
    for (int j = i; j != -1; j = parent[j]) {
        if (n >= k) return -1;
        if (j == 0 ? parent[0] != -1 : (parent[j] < 0 || parent[j] >= j)) return -1;
        path[n++] = j;
    }
    for (int a = 0, b = n - 1; a < b; ++a, --b) {
        const int t = path[a];
        path[a] = path[b];
        path[b] = t;
    }
    return n;
}

/* The state after the tokens path[0..n-1] of request b, head h, from S0 (float64 [dk][dv]). */
static void rec_run(const float *S0, const uint16_t *kk, const uint16_t *v, const float *g,
                    int K, int H, int dk, int dv, int b, int h, const int *path, int n, double *S) {
    const float *s0 = S0 + ((int64_t)b * H + h) * dk * dv;
    for (int64_t e = 0; e < (int64_t)dk * dv; ++e) S[e] = s0[e];
    for (int t = 0; t < n; ++t) {
        const int64_t tok = (int64_t)b * K + path[t];
        const double a = exp((double)g[tok * H + h]);
        const uint16_t *kr = kk + (tok * H + h) * dk;
        const uint16_t *vr = v + (tok * H + h) * dv;
        for (int r = 0; r < dk; ++r) {
            const double kv = bf16_to_f32(kr[r]);
            for (int c = 0; c < dv; ++c)
                S[(int64_t)r * dv + c] = a * S[(int64_t)r * dv + c] + kv * (double)bf16_to_f32(vr[c]);
        }
    }
}

/* Outputs o = S_i^T q_i of every node (float64). parent NULL = a chain. status[b] = 1 for a
 * malformed tree (its outputs zero), else 0. */
void orc_rec_tree(const float *S0, const uint16_t *q, const uint16_t *kk, const uint16_t *v,
                  const float *g, const int32_t *parent, int B, int K, int H, int dk, int dv,
                  double *out, int32_t *status) {
    for (int b = 0; b < B; ++b) {
        int32_t *par = malloc(sizeof(int32_t) * K);
        int *path = malloc(sizeof(int) * K);
        for (int i = 0; i < K; ++i) par[i] = parent ? parent[(int64_t)b * K + i] : i - 1;
        status[b] = 0;
        for (int i = 0; i < K; ++i)
            if (rec_path(par, K, i, path) < 0) status[b] = 1;
        free(path);
#pragma omp parallel for collapse(2) schedule(dynamic)
        for (int i = 0; i < K; ++i)
            for (int h = 0; h < H; ++h) {
                double *o = out + (((int64_t)b * K + i) * H + h) * dv;
                if (status[b]) {
                    for (int c = 0; c < dv; ++c) o[c] = 0.0;
                    continue;
                }
                int *pth = malloc(sizeof(int) * K);
                double *S = malloc(sizeof(double) * dk * dv);
                const int n = rec_path(par, K, i, pth);
                rec_run(S0, kk, v, g, K, H, dk, dv, b, h, pth, n, S);
                const uint16_t *qr = q + (((int64_t)b * K + i) * H + h) * dk;
                for (int c = 0; c < dv; ++c) {
                    double acc = 0.0;
                    for (int r = 0; r < dk; ++r) acc += S[(int64_t)r * dv + c] * (double)bf16_to_f32(qr[r]);
                    o[c] = acc;
                }
                free(S);
                free(pth);
            }
        free(par);
    }
}

/* The committed state after acceptance: for each request whose accepted_len a is in [0, K) and
 * whose path entries path[b][0..a] are node ids in [0, K), the state after those tokens (the
 * accepted root path, the root first), from S0, into S_out (float64, same layout as S0). Any
 * other request (a < 0, a >= K, or a node id outside [0, K)) keeps S0: there is no accepted path
 * of that request to apply. */
void orc_rec_commit(const float *S0, const uint16_t *kk, const uint16_t *v, const float *g,
                    const int32_t *accepted_len, const int32_t *accepted_path, int B, int K, int H,
                    int dk, int dv, double *S_out) {
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            const int a = accepted_len[b];
            int *pth = malloc(sizeof(int) * K);
            int n = (a < 0 || a >= K) ? 0 : a + 1;
            for (int t = 0; t < n; ++t) {
                const int id = accepted_path[(int64_t)b * K + t];
                if (id < 0 || id >= K) { n = 0; break; }
                pth[t] = id;
            }
            rec_run(S0, kk, v, g, K, H, dk, dv, b, h, pth, n, S_out + ((int64_t)b * H + h) * dk * dv);
            free(pth);
        }
}

/* ------------------------------------------------------------------------------------------ */
/* A recurrent layer of a hybrid target                                                       */
/* ------------------------------------------------------------------------------------------ */
/* The pages name targets that mix recurrent layers in (SpecPilot digest, airadar.tv —
 * "Reasons") but give neither the recurrence nor the layer around it. The reading used here: the
 * attention mixer of a decoder layer is replaced by the scalar-gated recurrence above, with
 * nh = n_q_heads heads of d = head_dim:
 *   u = RMSNorm(x) * attn_norm;
 *   [q | k | v | a] = u . W^T, W = w_qkv with 3 nh d + nh rows (q heads, k heads, v heads, then
 *   one gate row per head), each rounded to bf16 like every projection output;
 *   g = -softplus(a) = -log(1 + e^a) per (node, head), in fp32 (a > 20: -a);
 *   o = S_i^T q for each node i, S_i the state after the root path of node i applied to the
 *   committed state S0 (see orc_rec_tree), rounded to fp32, then to bf16;
 *   x += o . W_o^T (w_o [H][nh d]), then the MLP block.
 * No position enters the recurrent layer (no RoPE). */
static float neg_softplus(float a) { return a > 20.0f ? -a : -log1pf(expf(a)); }

/* x [m][H] in/out; S0 [nh][d][d] fp32 (S[r][c]: key index r, value index c), read only;
 * k_out, v_out [m][nh][d] bf16 and g_out [m][nh] fp32: the nodes' keys, values and log-gates
 * (what a commit applies to the state). Returns 0, or -1 for a malformed tree. */
int orc_rec_layer_forward(const orc_cfg *c, const orc_layer_w *w, const float *S0,
                          const int32_t *parent, int m, uint16_t *x, uint16_t *k_out,
                          uint16_t *v_out, float *g_out) {
    int H = c->hidden, nh = c->n_q_heads, d = c->head_dim, F = c->ffn;
    int nrow = 3 * nh * d + nh;
    int32_t *depth = (int32_t *)malloc(sizeof(int32_t) * (size_t)m);
    if (orc_tree_depth(parent, m, depth) != 0) {
        free(depth);
        return -1;
    }
    int ywidth = nrow;
    if (2 * F > ywidth) ywidth = 2 * F;
    if (H > ywidth) ywidth = H;
    uint16_t *u = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)m * H);
    float *y = (float *)malloc(sizeof(float) * (size_t)m * ywidth);
    uint16_t *q = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)m * nh * d);
    uint16_t *o = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)m * nh * d);
    double *o64 = (double *)malloc(sizeof(double) * (size_t)m * nh * d);
    int32_t st = 0;
    uint16_t *gate = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)m * F);
    uint16_t *up = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)m * F);
    uint16_t *hm = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)m * F);

    /* recurrent mixer */
    orc_rmsnorm(x, w->attn_norm, m, H, c->rms_eps, u);
    orc_linear(u, m, H, w->w_qkv, nrow, y);
    for (int i = 0; i < m; ++i) {
        const float *yi = y + (int64_t)i * nrow;
        for (int j = 0; j < nh * d; ++j) {
            q[(int64_t)i * nh * d + j] = f32_to_bf16(yi[j]);
            k_out[(int64_t)i * nh * d + j] = f32_to_bf16(yi[nh * d + j]);
            v_out[(int64_t)i * nh * d + j] = f32_to_bf16(yi[2 * nh * d + j]);
        }
        for (int h = 0; h < nh; ++h)
            g_out[(int64_t)i * nh + h] = neg_softplus(bf16_to_f32(f32_to_bf16(yi[3 * nh * d + h])));
    }
    orc_rec_tree(S0, q, k_out, v_out, g_out, parent, 1, m, nh, d, d, o64, &st);
    for (int64_t e = 0; e < (int64_t)m * nh * d; ++e) o[e] = f32_to_bf16((float)o64[e]);
    orc_linear(o, m, nh * d, w->w_o, H, y);
    residual_add(x, y, (int64_t)m * H);

    mlp_block(c, w, m, x, u, y, gate, up, hm);

    free(depth); free(u); free(y); free(q); free(o); free(o64); free(gate); free(up); free(hm);
    return 0;
}
