/*
 * sanitize_driver.c — runs every entry point of the CPU oracle on small seeded inputs, the
 * degenerate and malformed cases included, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitizers.py compiles it with the oracle in one unit:
 *   gcc -O1 -g -fsanitize=address,undefined -fno-sanitize-recover=all -fopenmp sanitize_driver.c -lm).
 * A sanitizer report aborts the run; a wrong result of a case whose answer is fixed here returns
 * a nonzero status. TEST INFRASTRUCTURE, like the oracle itself.
 */
#include "specverify_oracle.c"

#include <stdio.h>

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static double urand(void) {   /* splitmix64 -> [0, 1) */
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
    return (double)(z >> 11) / 9007199254740992.0;
}
static uint16_t rbf(double scale) { return f32_to_bf16((float)((urand() * 2.0 - 1.0) * scale)); }
static uint16_t *rbf_array(int64_t n, double scale) {
    uint16_t *a = malloc(sizeof(uint16_t) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) a[i] = rbf(scale);
    return a;
}

static int failures = 0;
#define EXPECT(c)                                                                    \
    do {                                                                             \
        if (!(c)) {                                                                  \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #c); \
            ++failures;                                                              \
        }                                                                            \
    } while (0)

int main(void) {
    orc_set_threads(2);
    /* a small model: 2 layers, hidden 64, 4 q / 2 kv heads of 16, MLP 96, vocab 48 */
    orc_cfg c = {2, 64, 4, 2, 16, 96, 48, 1e-6f, 10000.0};
    const int H = c.hidden, nq = c.n_q_heads, nkv = c.n_kv_heads, d = c.head_dim, F = c.ffn, V = c.vocab;
    const int nqkv = (nq + 2 * nkv) * d, nrec = 3 * nq * d + nq;
    uint16_t *ones = malloc(sizeof(uint16_t) * H);
    for (int i = 0; i < H; ++i) ones[i] = f32_to_bf16(1.0f);
    uint16_t *w_qkv = rbf_array((int64_t)nqkv * H, 0.1), *w_rec = rbf_array((int64_t)nrec * H, 0.1);
    uint16_t *w_o = rbf_array((int64_t)H * nq * d, 0.1), *w_gu = rbf_array((int64_t)2 * F * H, 0.1);
    uint16_t *w_down = rbf_array((int64_t)H * F, 0.1);
    orc_layer_w la = {ones, w_qkv, w_o, ones, w_gu, w_down};
    orc_layer_w lr = {ones, w_rec, w_o, ones, w_gu, w_down};
    uint16_t *embed = rbf_array((int64_t)V * H, 0.5), *lm = rbf_array((int64_t)V * H, 0.2);

    /* trees: a valid 7-node tree, a chain, and malformed ones */
    const int K = 7;
    int32_t tree[7] = {-1, 0, 0, 1, 1, 2, 5}, chain[7], bad_root[7], bad_order[7], depth[7];
    for (int i = 0; i < K; ++i) chain[i] = i - 1;
    memcpy(bad_root, tree, sizeof tree);
    bad_root[0] = 0;
    memcpy(bad_order, tree, sizeof tree);
    bad_order[3] = 5;
    EXPECT(orc_tree_depth(tree, K, depth) == 0 && depth[6] == 3);
    EXPECT(orc_tree_depth(bad_root, K, depth) == -1);
    EXPECT(orc_tree_depth(bad_order, K, depth) == -1);
    EXPECT(orc_tree_depth(tree, 0, depth) == -1);

    /* attention layer over contexts 0 and 5, both trees; malformed tree refused */
    for (int ctx = 0; ctx <= 5; ctx += 5) {
        uint16_t *kc = rbf_array((int64_t)ctx * nkv * d, 1.0), *vc = rbf_array((int64_t)ctx * nkv * d, 1.0);
        uint16_t *x = rbf_array((int64_t)K * H, 0.5), *kn = malloc(2 * (size_t)K * nkv * d), *vn = malloc(2 * (size_t)K * nkv * d);
        EXPECT(orc_layer_forward(&c, &la, kc, vc, ctx, tree, K, x, kn, vn) == 0);
        EXPECT(orc_layer_forward(&c, &la, kc, vc, ctx, chain, K, x, kn, vn) == 0);
        EXPECT(orc_layer_forward(&c, &la, kc, vc, ctx, bad_order, K, x, kn, vn) == -1);
        EXPECT(orc_layer_forward(&c, &la, kc, vc, ctx, tree, 1, x, kn, vn) == 0);
        free(kc); free(vc); free(x); free(kn); free(vn);
    }

    /* recurrent layer (hybrid target), its tree pass and commit */
    {
        float *S0 = malloc(sizeof(float) * (size_t)2 * nq * d * d);
        for (int64_t i = 0; i < (int64_t)2 * nq * d * d; ++i) S0[i] = (float)(urand() - 0.5);
        uint16_t *x = rbf_array((int64_t)K * H, 0.5), *kk = malloc(2 * (size_t)2 * K * nq * d), *vv = malloc(2 * (size_t)2 * K * nq * d);
        float *g = malloc(sizeof(float) * (size_t)2 * K * nq);
        EXPECT(orc_rec_layer_forward(&c, &lr, S0, tree, K, x, kk, vv, g) == 0);
        EXPECT(orc_rec_layer_forward(&c, &lr, S0, bad_root, K, x, kk, vv, g) == -1);
        for (int i = 0; i < K * nq; ++i) EXPECT(g[i] <= 0.0f);
        /* two requests: q, k, v, g drawn; the second request's tree malformed */
        uint16_t *q = rbf_array((int64_t)2 * K * nq * d, 0.3);
        uint16_t *k2 = rbf_array((int64_t)2 * K * nq * d, 0.3), *v2 = rbf_array((int64_t)2 * K * nq * d, 1.0);
        for (int i = 0; i < 2 * K * nq; ++i) g[i] = (float)(-urand());
        int32_t par[14], st[2];
        memcpy(par, tree, sizeof tree);
        memcpy(par + 7, bad_order, sizeof tree);
        double *out = malloc(sizeof(double) * (size_t)2 * K * nq * d), *Sout = malloc(sizeof(double) * (size_t)2 * nq * d * d);
        orc_rec_tree(S0, q, k2, v2, g, par, 2, K, nq, d, d, out, st);
        EXPECT(st[0] == 0 && st[1] == 1);
        for (int64_t i = (int64_t)K * nq * d; i < (int64_t)2 * K * nq * d; ++i) EXPECT(out[i] == 0.0);
        orc_rec_tree(S0, q, k2, v2, g, NULL, 2, K, nq, d, d, out, st);
        EXPECT(st[0] == 0 && st[1] == 0);
        /* commit: accepted_len -1, 0, K - 1, K (out of range), and an out-of-range node id */
        const int32_t cases[5][2] = {{-1, 0}, {0, 0}, {K - 1, 0}, {K, 0}, {2, 1}};
        for (int ci = 0; ci < 5; ++ci) {
            int32_t al[2] = {cases[ci][0], 0}, ap[14];
            for (int t = 0; t < 14; ++t) ap[t] = t % 7;
            if (cases[ci][1]) ap[1] = K + 3;
            orc_rec_commit(S0, k2, v2, g, al, ap, 2, K, nq, d, d, Sout);
            const int keeps = al[0] < 0 || al[0] >= K || cases[ci][1];
            if (keeps)
                for (int64_t e = 0; e < (int64_t)nq * d * d; ++e) EXPECT(Sout[e] == (double)S0[e]);
        }
        free(S0); free(x); free(kk); free(vv); free(g); free(q); free(k2); free(v2); free(out); free(Sout);
    }

    /* building blocks directly */
    {
        uint16_t *x = rbf_array((int64_t)3 * H, 2.0), *u = malloc(2 * (size_t)3 * H);
        float *y = malloc(sizeof(float) * (size_t)3 * nqkv);
        orc_rmsnorm(x, ones, 3, H, c.rms_eps, u);
        orc_linear(u, 3, H, w_qkv, nqkv, y);
        int32_t pos[3] = {0, 1, 1000000};
        orc_rope(u, pos, 3, H / d, d, c.rope_theta);
        uint16_t *hm = malloc(2 * (size_t)3 * H);
        orc_swiglu(x, u, (int64_t)3 * H, hm);
        free(x); free(u); free(y); free(hm);
    }

    /* embedding (an out-of-range token refused), logits, argmax with exact ties, acceptance */
    {
        int32_t tok[7] = {1, 2, 3, 4, 5, 6, 47}, bad[2] = {3, 48}, neg[2] = {-1, 0};
        uint16_t *x = malloc(2 * (size_t)K * H);
        EXPECT(orc_embed(embed, V, H, tok, K, x) == 0);
        EXPECT(orc_embed(embed, V, H, bad, 2, x) == -1);
        EXPECT(orc_embed(embed, V, H, neg, 2, x) == -1);
        float *lg = malloc(sizeof(float) * (size_t)K * V);
        orc_logits(&c, ones, lm, x, K, lg);
        for (int j = 0; j < V; ++j) lg[j] = 1.0f;          /* row 0: all tied */
        int32_t arg[7], al, bonus, path[7];
        float margin[7];
        orc_argmax(lg, K, V, arg, margin);
        EXPECT(arg[0] == 0 && margin[0] == 0.0f);
        EXPECT(orc_accept(tok, tree, arg, K, &al, &bonus, path) == 0 && al >= 0 && al < K);
        EXPECT(orc_accept(tok, bad_root, arg, K, &al, &bonus, path) == -1 && al == -1 && bonus == -1);
        /* a chain whose tokens are all greedy is accepted whole */
        int32_t ctok[7], carg[7];
        for (int i = 0; i < K; ++i) { ctok[i] = i + 1; carg[i] = i + 2; }
        orc_accept(ctok, chain, carg, K, &al, &bonus, path);
        EXPECT(al == K - 1 && bonus == K + 1 && path[K - 1] == K - 1);
        free(x); free(lg);
    }

    /* W12: every bf16 pattern round-trips */
    {
        const int64_t n = 65536;
        uint16_t *w = malloc(sizeof(uint16_t) * n), *back = malloc(sizeof(uint16_t) * n);
        for (int64_t i = 0; i < n; ++i) w[i] = (uint16_t)i;
        uint8_t *lo = malloc(n), *nib = malloc(n), *esc = malloc(n);
        const int b = orc_w12_base(w, n);
        const int64_t ne = orc_w12_encode(w, n, b, lo, nib, esc);
        int64_t *ei = malloc(sizeof(int64_t) * (size_t)(ne > 0 ? ne : 1));
        uint16_t *ev = malloc(sizeof(uint16_t) * (size_t)(ne > 0 ? ne : 1));
        int64_t j = 0;
        for (int64_t i = 0; i < n; ++i)
            if (esc[i]) { ei[j] = i; ev[j] = w[i]; ++j; }
        orc_w12_decode(lo, nib, n, b, ei, ev, ne, back);
        EXPECT(j == ne && memcmp(w, back, sizeof(uint16_t) * n) == 0);
        free(w); free(back); free(lo); free(nib); free(esc); free(ei); free(ev);
    }

    free(ones); free(w_qkv); free(w_rec); free(w_o); free(w_gu); free(w_down); free(embed); free(lm);
    if (failures) fprintf(stderr, "%d expectation(s) failed\n", failures);
    else printf("oracle sanitizer run: all cases clean\n");
    return failures ? 1 : 0;
}
