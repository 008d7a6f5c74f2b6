/*
 * host_sanitize_driver.c — exercises the host side of libspecverify (argument checks, shape
 * planning, workspace layout) through the C ABI, for a build whose host code carries
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers.py builds both). Only
 * calls that return before anything is enqueued are made, so no GPU is needed: workspace sizes
 * over many shapes, and every refusal path of the entry points (NULL pointers, bad shapes, bad
 * trees of layer kinds, a workspace one byte short). Returns nonzero when an expected return code
 * is not met; a sanitizer report aborts.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "specverify.h"

static int failures = 0;
#define EXPECT(c)                                                                        \
    do {                                                                                 \
        if (!(c)) {                                                                      \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #c);  \
            ++failures;                                                                  \
        }                                                                                \
    } while (0)

int main(void) {
    const spec_model_cfg dense27 = {64, 5120, 40, 8, 128, 17408, 151936, 1e-6f, 10000.0};
    const spec_model_cfg tiny = {2, 256, 4, 2, 64, 704, 1024, 1e-6f, 10000.0};
    size_t bytes = 0;

    /* workspace sizes: batches, draft sizes and page budgets across the planning branches */
    const int batches[] = {1, 2, 3, 8, 32, 64};
    const int ks[] = {1, 2, 5, 13, 16, 17, 31, 64};
    const int pages[] = {1, 9, 257, 513, 4096};
    for (int ib = 0; ib < 6; ++ib)
        for (int ik = 0; ik < 8; ++ik)
            for (int ip = 0; ip < 5; ++ip) {
                EXPECT(spec_workspace_bytes(&dense27, batches[ib], ks[ik], pages[ip], &bytes) == SPEC_OK);
                EXPECT(bytes > 0);
                EXPECT(spec_workspace_bytes(&tiny, batches[ib], ks[ik], pages[ip], &bytes) == SPEC_OK);
            }
    EXPECT(spec_workspace_bytes(&tiny, 1, 65, 9, &bytes) == SPEC_EUNSUPPORTED);
    EXPECT(spec_workspace_bytes(&tiny, 0, 4, 9, &bytes) == SPEC_EINVAL);
    EXPECT(spec_workspace_bytes(&tiny, 1, 4, 0, &bytes) == SPEC_EINVAL);
    EXPECT(spec_workspace_bytes(NULL, 1, 4, 9, &bytes) == SPEC_EINVAL);
    EXPECT(spec_workspace_bytes(&tiny, 1, 4, 9, NULL) == SPEC_EINVAL);
    spec_model_cfg bad = tiny;
    bad.head_dim = 96;
    EXPECT(spec_workspace_bytes(&bad, 1, 4, 9, &bytes) == SPEC_EUNSUPPORTED);
    bad = tiny;
    bad.n_q_heads = 3;
    EXPECT(spec_workspace_bytes(&bad, 1, 4, 9, &bytes) == SPEC_EUNSUPPORTED);
    bad = tiny;
    bad.rms_eps = -1.0f;
    EXPECT(spec_workspace_bytes(&bad, 1, 4, 9, &bytes) == SPEC_EINVAL);
    EXPECT(spec_accept_workspace_bytes(4, 16, 151936, &bytes) == SPEC_OK);
    EXPECT(spec_accept_workspace_bytes(4, 65, 151936, &bytes) == SPEC_EUNSUPPORTED);

    /* spec_verify refusals: fake (never dereferenced) device pointers, host arrays real */
    static char dev[1 << 12] __attribute__((aligned(256)));
    void *D = dev;
    spec_layer_weights lw[2];
    for (int l = 0; l < 2; ++l) {
        lw[l].attn_norm = D; lw[l].w_qkv = D; lw[l].w_o = D;
        lw[l].mlp_norm = D; lw[l].w_gate_up = D; lw[l].w_down = D;
    }
    spec_weights w;
    memset(&w, 0, sizeof w);
    w.cfg = tiny;
    w.layers = lw;
    w.embed = D;
    w.final_norm = D;
    w.lm_head = D;
    const int32_t table[2] = {0, 1};
    spec_kv_cache kv;
    memset(&kv, 0, sizeof kv);
    kv.k_pool = D;
    kv.v_pool = D;
    kv.block_table = table;
    kv.n_pages = 2;
    kv.max_pages_per_req = 2;
    int32_t *I = (int32_t *)dev;
    size_t need = 0;
    EXPECT(spec_workspace_bytes(&tiny, 1, 4, 2, &need) == SPEC_OK);
    /* a workspace one byte short is refused after every other check has passed */
    EXPECT(spec_verify(&w, &kv, I, NULL, I, 1, 4, I, I, I, NULL, D, need - 1, 0) == SPEC_EWORKSPACE);
    EXPECT(spec_verify(NULL, &kv, I, NULL, I, 1, 4, I, I, I, NULL, D, need, 0) == SPEC_EINVAL);
    EXPECT(spec_verify(&w, &kv, NULL, NULL, I, 1, 4, I, I, I, NULL, D, need, 0) == SPEC_EINVAL);
    EXPECT(spec_verify(&w, &kv, I, NULL, I, 1, 65, I, I, I, NULL, D, need, 0) == SPEC_EUNSUPPORTED);
    EXPECT(spec_verify(&w, &kv, I, NULL, I, 1, 4, I, I, I, NULL, (char *)D + 8, need, 0) == SPEC_EINVAL);
    spec_verify_extras ex;
    memset(&ex, 0, sizeof ex);
    ex.path = 7;
    EXPECT(spec_verify(&w, &kv, I, NULL, I, 1, 4, I, I, I, &ex, D, need, 0) == SPEC_EINVAL);
    /* hybrid: an unknown layer kind; a recurrent layer without states or without the pass's
     * buffers; W12 with a recurrent layer */
    int32_t kinds[2] = {0, 5};
    w.layer_kind = kinds;
    EXPECT(spec_verify(&w, &kv, I, NULL, I, 1, 4, I, I, I, NULL, D, need, 0) == SPEC_EINVAL);
    kinds[1] = SPEC_LAYER_RECURRENT;
    EXPECT(spec_verify(&w, &kv, I, NULL, I, 1, 4, I, I, I, NULL, D, need, 0) == SPEC_EINVAL);
    float *states[2] = {NULL, (float *)D};
    kv.rec_state = states;
    EXPECT(spec_verify(&w, &kv, I, NULL, I, 1, 4, I, I, I, NULL, D, need, 0) == SPEC_EINVAL);
    kv.rec_k = D;
    kv.rec_v = D;
    kv.rec_g = (float *)D;
    EXPECT(spec_verify(&w, &kv, I, NULL, I, 1, 4, I, I, I, NULL, D, need - 1, 0) == SPEC_EWORKSPACE);
    ex.path = SPEC_PATH_PERSISTENT;
    EXPECT(spec_verify(&w, &kv, I, NULL, I, 1, 4, I, I, I, &ex, D, need, 0) == SPEC_EUNSUPPORTED);
    EXPECT(spec_prefill(&w, &kv, I, I, 1, 4, I, NULL, D, 1 << 30, 0) == SPEC_EUNSUPPORTED);
    w.layer_kind = NULL;
    kv.rec_state = NULL;

    /* spec_commit_kv, spec_accept and the recurrent primitives: refusals */
    EXPECT(spec_commit_kv(&tiny, &kv, NULL, I, I, 1, 4, 0) == SPEC_EINVAL);
    EXPECT(spec_commit_kv(&tiny, &kv, I, I, I, 0, 4, 0) == SPEC_EINVAL);
    EXPECT(spec_commit_kv(&tiny, &kv, I, I, I, 1, 65, 0) == SPEC_EUNSUPPORTED);
    kv.rec_state = states;
    kv.rec_k = NULL;
    EXPECT(spec_commit_kv(&tiny, &kv, I, I, I, 1, 4, 0) == SPEC_EINVAL);
    kv.rec_state = NULL;
    EXPECT(spec_rec_tree_verify(NULL, D, D, D, (float *)D, NULL, 1, 4, 2, 64, (float *)D, I, 0) == SPEC_EINVAL);
    EXPECT(spec_rec_tree_verify((float *)D, D, D, D, (float *)D, NULL, 1, 4, 2, 96, (float *)D, I, 0) == SPEC_EUNSUPPORTED);
    EXPECT(spec_rec_commit((float *)D, D, D, (float *)D, I, I, 1, 65, 2, 64, 0) == SPEC_EUNSUPPORTED);

    /* every return code has its text */
    const int codes[] = {SPEC_OK, SPEC_EINVAL, SPEC_EUNSUPPORTED, SPEC_EWORKSPACE, SPEC_EHIP, SPEC_ESCRATCH, 12345};
    for (int i = 0; i < 7; ++i) EXPECT(spec_strerror(codes[i]) != NULL && spec_strerror(codes[i])[0] != 0);

    if (failures) fprintf(stderr, "%d expectation(s) failed\n", failures);
    else printf("host sanitizer run: all cases clean\n");
    return failures ? 1 : 0;
}
