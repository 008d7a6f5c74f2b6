// specverify.hip — host side of libspecverify: argument checks, the per-call plan (GEMM tiles
// and waves, attention chunks, workspace layout) and the launch sequence of one
// verification pass. Everything is enqueued on the caller's stream; nothing here waits for
// the device, allocates, or keeps global state.
#include <string.h>

#include <mutex>

#include "specverify.h"
#include "kernels.hpp"

namespace {

using namespace sv;

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

struct Carver {
    size_t off = 0;
    size_t take(size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes);
        return o;
    }
};

struct Plan {
    int B, K, M;
    int L, H, nq, nkv, D, F, V;
    int qd, nqkv;
    GemmShape g_qkv, g_o, g_gu, g_down, g_lm;
    bool qkv_fused;         // QKV with its RoPE epilogue (no split-K pass): passes of <= 16 rows
    GemmShape g_qkvf;       // its plan (bf16 and W12 alike)
    int nrec;               // rows of a recurrent layer's projection (q, k, v, gates, padding)
    GemmShape g_rqkv;
    GemmShape w_qkv, w_o, w_gu, w_down, w_lm;   // the same projections over W12 weights (M <= 64)
    int lm_groups, lm_groups_w12;
    int attn_chunks;
    int n_ctr;              // arrival counters of a balanced gate/up launch (0: none)
    size_t o_depth, o_pos, o_status, o_anc, o_rope, o_x, o_u, o_q, o_attn, o_h, o_part, o_po,
        o_pml, o_amv, o_ami, o_rq, o_ro, o_rs, o_ctr, total;
    // the persistent path (rows <= 16): its own buffers, sized for up to kFusedSizeG workgroups
    bool fused_shape;
    size_t total_steps;     // the per-step plan's part of the workspace (the persistent one follows)
    size_t f_x, f_ssq_o, f_ssq_d, f_q, f_ao, f_h, f_u, f_part[4], f_att_o, f_att_ml, f_sync;
};

// Workgroups the persistent path is sized for (one per compute unit; more units are left idle).
constexpr int kFusedSizeG = 512;

// Counts of the persistent path for G workgroups (see FusedPhase): per projection the split,
// the largest group share and the most groups one workgroup touches; the attention items.
struct FusedCounts {
    int G;
    int S[4], groups[4], units[4], g_eff[4], max_parts[4], max_seg[4];
    int CH, n_chunks, n_items, tiles, n_tasks, n_sync;
};

int fused_wg_of(int64_t u, int g_eff, int units) { return (int)(((u + 1) * g_eff - 1) / units); }

void fused_counts(const Plan &p, int G, int max_pages, FusedCounts &f) {
    f.G = G;
    const int N[4] = {p.nqkv, p.H, 2 * p.F, p.H};
    const int Kd[4] = {p.H, p.qd, p.H, p.F};
    for (int ph = 0; ph < 4; ++ph) {
        f.S[ph] = Kd[ph] / 32;
        f.groups[ph] = N[ph] / 64;
        f.units[ph] = f.S[ph] * f.groups[ph];
        f.g_eff[ph] = G < f.units[ph] ? G : f.units[ph];
        int mp = 1, ms = 1;
        for (int g = 0; g < f.groups[ph]; ++g) {
            const int a = fused_wg_of((int64_t)g * f.S[ph], f.g_eff[ph], f.units[ph]);
            const int b = fused_wg_of((int64_t)(g + 1) * f.S[ph] - 1, f.g_eff[ph], f.units[ph]);
            if (b - a + 1 > mp) mp = b - a + 1;
        }
        for (int w = 0; w < f.g_eff[ph]; ++w) {
            const int u0 = (int)((int64_t)f.units[ph] * w / f.g_eff[ph]);
            const int u1 = (int)((int64_t)f.units[ph] * (w + 1) / f.g_eff[ph]);
            const int seg = (u1 - 1) / f.S[ph] - u0 / f.S[ph] + 1;
            if (seg > ms) ms = seg;
        }
        f.max_parts[ph] = mp;
        f.max_seg[ph] = ms;
    }
    // attention: about G / (B * n_kv) chunks per (request, kv head), whole 32-key steps, at most
    // 160 keys (the registers of one item); more items than workgroups run in turns
    const int64_t max_keys = (int64_t)max_pages * SPEC_PAGE_SIZE;
    int per = G / (p.B * p.nkv);
    if (per < 1) per = 1;
    int64_t ch = (max_keys + 32LL * per - 1) / (32LL * per) * 32;
    if (ch > 160) ch = 160;
    if (ch < 32) ch = 32;
    f.CH = (int)ch;
    f.n_chunks = (int)((max_keys + ch - 1) / ch);
    f.n_items = p.B * p.nkv * f.n_chunks;
    f.tiles = (p.nq / p.nkv * p.K + 15) / 16;
    f.n_tasks = p.B * p.nkv * f.tiles * 4;
    int nflag = f.n_items + f.n_tasks + 1;
    for (int ph = 0; ph < 4; ++ph) nflag += 2 * f.groups[ph];
    f.n_sync = nflag;
}

// The persistent path takes the shape (its device check comes at the call).
bool fused_shape_ok(const Plan &p) {
    return p.M <= 16 && (p.D == 64 || p.D == 128) && p.nq / p.nkv <= 8;
}

int check_cfg(const spec_model_cfg *c) {
    if (c == nullptr) return SPEC_EINVAL;
    if (c->n_layers < 1 || c->hidden < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 ||
        c->head_dim < 1 || c->ffn < 1 || c->vocab < 1)
        return SPEC_EINVAL;
    if (!(c->rms_eps >= 0.0f) || !(c->rope_theta > 0.0)) return SPEC_EINVAL;
    if (c->head_dim != 64 && c->head_dim != 128) return SPEC_EUNSUPPORTED;
    if (c->n_q_heads % c->n_kv_heads != 0) return SPEC_EUNSUPPORTED;
    if (c->hidden % 64 != 0 || (c->n_q_heads * c->head_dim) % 32 != 0 || c->ffn % 32 != 0)
        return SPEC_EUNSUPPORTED;
    if (c->hidden > 16384) return SPEC_EUNSUPPORTED;
    if (c->vocab % 64 != 0) return SPEC_EUNSUPPORTED;
    return SPEC_OK;
}

int make_plan(const spec_model_cfg *c, int B, int K, int max_pages, Plan &p) {
    int rc = check_cfg(c);
    if (rc != SPEC_OK) return rc;
    if (B < 1 || K < 1 || max_pages < 1) return SPEC_EINVAL;
    if (K > SPEC_MAX_K) return SPEC_EUNSUPPORTED;
    if ((int64_t)B * K > (1 << 20)) return SPEC_EUNSUPPORTED;
    p.B = B;
    p.K = K;
    p.M = B * K;
    p.L = c->n_layers;
    p.H = c->hidden;
    p.nq = c->n_q_heads;
    p.nkv = c->n_kv_heads;
    p.D = c->head_dim;
    p.F = c->ffn;
    p.V = c->vocab;
    p.qd = p.nq * p.D;
    p.nqkv = (p.nq + 2 * p.nkv) * p.D;
    const int M = p.M;
    p.g_qkv = plan_gemm(M, p.nqkv, p.H, true);
    // at most one block of 16 rows: the QKV projection runs whole-K with the RoPE and cache-write
    // epilogue, so no split-K pass sits between it and attention
    p.qkv_fused = M <= 16;
    p.g_qkvf = plan_gemm_qkv(M, p.nqkv, p.H);
    p.g_o = plan_gemm(M, p.H, p.qd, true);
    p.g_gu = plan_gemm_swiglu(M, 2 * p.F, p.H, false);
    p.g_down = plan_gemm(M, p.H, p.F, true);
    p.g_lm = plan_gemm(M, p.V, p.H, false);
    if (p.g_gu.nt < 2) return SPEC_EUNSUPPORTED;
    p.lm_groups = gemm_groups(p.g_lm);
    p.w_qkv = plan_gemm_w12(M, p.nqkv, p.H, true);
    p.w_o = plan_gemm_w12(M, p.H, p.qd, true);
    p.w_gu = plan_gemm_swiglu(M, 2 * p.F, p.H, true);
    p.w_down = plan_gemm_w12(M, p.H, p.F, true);
    p.w_lm = plan_gemm_w12(M, p.V, p.H, false);
    p.lm_groups_w12 = gemm_groups(p.w_lm);
    p.nrec = (3 * p.qd + p.nq + 15) / 16 * 16;
    p.g_rqkv = plan_gemm(M, p.nrec, p.H, true);
    const int64_t max_keys = (int64_t)max_pages * SPEC_PAGE_SIZE;
    p.attn_chunks = (int)((max_keys + kAttnChunk - 1) / kAttnChunk);
    const int group = p.nq / p.nkv;
    size_t part = 16;
    for (const GemmShape *g : {&p.g_qkv, &p.g_o, &p.g_down, &p.w_qkv, &p.w_o, &p.w_down, &p.g_rqkv}) {
        const size_t b = (size_t)g->splits * M * g->N * sizeof(float);
        if (b > part) part = b;
    }
    // a balanced gate/up launch keeps its K-part sums in the partials buffer (free between the O
    // pass's reduction and the down projection)
    for (const GemmShape *g : {&p.g_gu, &p.w_gu})
        if (gemm_bal_scratch_bytes(*g) > part) part = gemm_bal_scratch_bytes(*g);
    p.n_ctr = gemm_bal_counters(p.g_gu) > gemm_bal_counters(p.w_gu) ? gemm_bal_counters(p.g_gu)
                                                                     : gemm_bal_counters(p.w_gu);

    int amax_groups = p.lm_groups > argmax_chunks(p.V) ? p.lm_groups : argmax_chunks(p.V);
    if (p.lm_groups_w12 > amax_groups) amax_groups = p.lm_groups_w12;
    Carver cv;
    p.o_depth = cv.take(sizeof(int32_t) * M);
    p.o_pos = cv.take(sizeof(int32_t) * M);
    p.o_status = cv.take(sizeof(int32_t) * B);
    p.o_anc = cv.take(sizeof(uint64_t) * M);
    p.o_rope = cv.take(sizeof(float2) * M * (p.D / 2));
    const size_t Mp = (size_t)(M + 15) / 16 * 16;   // projection operands: whole 16-row blocks
    p.o_x = cv.take(sizeof(uint16_t) * M * p.H);
    p.o_u = cv.take(sizeof(uint16_t) * Mp * p.H);
    p.o_q = cv.take(sizeof(uint16_t) * M * p.qd);
    p.o_attn = cv.take(sizeof(uint16_t) * Mp * p.qd);
    p.o_h = cv.take(sizeof(uint16_t) * Mp * p.F);
    p.o_part = cv.take(part);
    p.o_po = cv.take(sizeof(float) * (size_t)B * p.nkv * p.attn_chunks * group * K * p.D);
    p.o_pml = cv.take(sizeof(float2) * (size_t)B * p.nkv * p.attn_chunks * group * K);
    p.o_amv = cv.take(sizeof(float) * (size_t)amax_groups * M);
    p.o_ami = cv.take(sizeof(int32_t) * (size_t)amax_groups * M);
    // recurrent layers of a hybrid target: q, the tree pass's output, its status
    p.o_rq = cv.take(sizeof(uint16_t) * M * p.qd);
    p.o_ro = cv.take(sizeof(float) * M * p.qd);
    p.o_rs = cv.take(sizeof(int32_t) * B);
    p.o_ctr = cv.take(sizeof(int32_t) * (p.n_ctr > 0 ? p.n_ctr : 1));
    p.fused_shape = fused_shape_ok(p);
    p.total_steps = cv.off;
    if (p.fused_shape) {
        FusedCounts f;
        fused_counts(p, kFusedSizeG, max_pages, f);
        const size_t nl = kFusedMaxLayers;
        p.f_x = cv.take(sizeof(uint16_t) * 2 * nl * 16 * p.H);      // x_o slots, then x_d slots
        p.f_ssq_o = cv.take(sizeof(float) * (p.H / 64) * 16);
        p.f_ssq_d = cv.take(sizeof(float) * (p.H / 64) * 16);
        p.f_q = cv.take(sizeof(uint16_t) * nl * M * p.qd);
        p.f_ao = cv.take(sizeof(uint16_t) * nl * 16 * p.qd);
        p.f_h = cv.take(sizeof(uint16_t) * nl * 16 * p.F);
        p.f_u = cv.take(sizeof(uint16_t) * 16 * p.H);
        for (int ph = 0; ph < 4; ++ph)
            p.f_part[ph] = cv.take(sizeof(float) * 1024 * (size_t)f.groups[ph] * f.max_parts[ph]);
        p.f_att_o = cv.take(sizeof(float) * (size_t)f.n_items * f.tiles * 16 * p.D);
        p.f_att_ml = cv.take(sizeof(uint64_t) * (size_t)f.n_items * f.tiles * 16);
        p.f_sync = cv.take(sizeof(uint32_t) * (size_t)f.n_sync);
    }
    p.total = cv.off;
    return SPEC_OK;
}

template <typename T>
T *at(void *ws, size_t off) {
    return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

bool w12_ok(const spec_w12_matrix &m) { return m.planes && m.plan && m.exc; }

W12Ref w12_ref(const spec_w12_matrix &m) {
    W12Ref r;
    r.planes = static_cast<const uint32_t *>(m.planes);
    r.plan = m.plan;
    r.exc = reinterpret_cast<const int2 *>(m.exc);
    return r;
}

#define SV_TRY(x)                                  \
    do {                                           \
        if ((x) != hipSuccess) return SPEC_EHIP;   \
    } while (0)

}  // namespace

extern "C" {

const char *spec_strerror(int code) {
    switch (code) {
        case SPEC_OK: return "ok";
        case SPEC_EINVAL: return "invalid argument";
        case SPEC_EUNSUPPORTED: return "unsupported shape";
        case SPEC_EWORKSPACE: return "workspace too small";
        case SPEC_EHIP: return "HIP runtime error";
        case SPEC_ESCRATCH: return "larger than the fixed scratch of the no-allocation entry point";
        default: return "unknown error";
    }
}

int spec_workspace_bytes(const spec_model_cfg *cfg, int batch, int k, int max_pages_per_req,
                         size_t *bytes) {
    if (bytes == nullptr) return SPEC_EINVAL;
    Plan p;
    const int rc = make_plan(cfg, batch, k, max_pages_per_req, p);
    if (rc != SPEC_OK) return rc;
    *bytes = p.total;
    return SPEC_OK;
}

int spec_verify(const spec_weights *w, const spec_kv_cache *kv, const int32_t *draft_tokens,
                const int32_t *tree_parent, const int32_t *ctx_len, int batch, int k,
                int32_t *accepted_len, int32_t *bonus_token, int32_t *accepted_path,
                const spec_verify_extras *extras, void *workspace, size_t workspace_bytes,
                hipStream_t stream) {
    if (w == nullptr || kv == nullptr || draft_tokens == nullptr || ctx_len == nullptr ||
        accepted_len == nullptr || bonus_token == nullptr || accepted_path == nullptr ||
        workspace == nullptr)
        return SPEC_EINVAL;
    if (w->layers == nullptr || w->embed == nullptr || w->final_norm == nullptr) return SPEC_EINVAL;
    if (kv->k_pool == nullptr || kv->v_pool == nullptr || kv->block_table == nullptr ||
        kv->n_pages < 1 || kv->max_pages_per_req < 1)
        return SPEC_EINVAL;
    Plan p;
    int rc = make_plan(&w->cfg, batch, k, kv->max_pages_per_req, p);
    if (rc != SPEC_OK) return rc;
    const bool w12 = w->w12_layers != nullptr;
    const bool w12_lm = w->w12_lm_head.planes != nullptr;
    if ((w12 || w12_lm) && p.M > 64) return SPEC_EUNSUPPORTED;
    if (!w12_lm && w->lm_head == nullptr) return SPEC_EINVAL;
    if (w12_lm && !w12_ok(w->w12_lm_head)) return SPEC_EINVAL;
    for (int l = 0; l < p.L; ++l) {
        const spec_layer_weights &lw = w->layers[l];
        if (!lw.attn_norm || !lw.mlp_norm) return SPEC_EINVAL;
        if (w12) {
            const spec_w12_layer &q = w->w12_layers[l];
            if (!w12_ok(q.w_qkv) || !w12_ok(q.w_o) || !w12_ok(q.w_gate_up) || !w12_ok(q.w_down))
                return SPEC_EINVAL;
        } else if (!lw.w_qkv || !lw.w_o || !lw.w_gate_up || !lw.w_down) {
            return SPEC_EINVAL;
        }
    }
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return SPEC_EINVAL;
    // recurrent layers (hybrid targets): their states and the pass's buffers, bf16 weights, the
    // per-step plan
    bool any_rec = false;
    if (w->layer_kind != nullptr) {
        for (int l = 0; l < p.L; ++l) {
            const int kd = w->layer_kind[l];
            if (kd != SPEC_LAYER_ATTENTION && kd != SPEC_LAYER_RECURRENT) return SPEC_EINVAL;
            if (kd == SPEC_LAYER_RECURRENT) {
                any_rec = true;
                if (kv->rec_state == nullptr || kv->rec_state[l] == nullptr) return SPEC_EINVAL;
            }
        }
    }
    if (any_rec) {
        if (kv->rec_k == nullptr || kv->rec_v == nullptr || kv->rec_g == nullptr) return SPEC_EINVAL;
        if (w12 || w12_lm) return SPEC_EUNSUPPORTED;
        if (p.K > kRecMaxK) return SPEC_EUNSUPPORTED;
    }

    const int want = extras ? extras->path : SPEC_PATH_AUTO;
    if (want != SPEC_PATH_AUTO && want != SPEC_PATH_STEPS && want != SPEC_PATH_PERSISTENT) return SPEC_EINVAL;
    // the persistent path: the shape, bf16 weights, and a device whose compute units each hold one
    // of its workgroups
    FusedCounts fc;
    bool fused = false;
    if (want == SPEC_PATH_PERSISTENT && p.fused_shape && !w12 && !w12_lm && !any_rec) {
        int dev = 0, ncu = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            ncu >= 1 && fused_occupancy(p.D) >= 1) {
            fused_counts(p, ncu < kFusedSizeG ? ncu : kFusedSizeG, kv->max_pages_per_req, fc);
            fused = fc.max_seg[FUSED_QKV] <= 2 && fc.max_seg[FUSED_O] <= 2 && fc.max_seg[FUSED_GU] <= 4 &&
                    fc.max_seg[FUSED_DOWN] <= 2;
        }
    }
    if (want == SPEC_PATH_PERSISTENT && !fused) return SPEC_EUNSUPPORTED;
    // spec_workspace_bytes covers both plans; a caller that forces the per-step plan may pass
    // that plan's part alone
    if (workspace_bytes < (want == SPEC_PATH_STEPS ? p.total_steps : p.total)) return SPEC_EWORKSPACE;

    float *logits = extras ? extras->logits : nullptr;
    int32_t *greedy = extras ? extras->greedy : nullptr;
    bf16 *trace = extras ? static_cast<bf16 *>(extras->hidden) : nullptr;
    hipEvent_t *gu_events = extras ? extras->gate_up_events : nullptr;
    const float eps = w->cfg.rms_eps;
    const int M = p.M;

    NodeInfo ni;
    ni.depth = at<int32_t>(workspace, p.o_depth);
    ni.pos = at<int32_t>(workspace, p.o_pos);
    ni.status = at<int32_t>(workspace, p.o_status);
    ni.anc = at<uint64_t>(workspace, p.o_anc);
    ni.rope = at<float2>(workspace, p.o_rope);
    bf16 *x = at<bf16>(workspace, p.o_x);
    bf16 *u = at<bf16>(workspace, p.o_u);
    bf16 *q = at<bf16>(workspace, p.o_q);
    bf16 *attn = at<bf16>(workspace, p.o_attn);
    bf16 *h = at<bf16>(workspace, p.o_h);
    float *part = at<float>(workspace, p.o_part);
    float *amv = at<float>(workspace, p.o_amv);
    int *ami = at<int>(workspace, p.o_ami);
    bf16 *k_pool = static_cast<bf16 *>(kv->k_pool);
    bf16 *v_pool = static_cast<bf16 *>(kv->v_pool);
    const int64_t layer_stride = (int64_t)kv->n_pages * p.nkv * SPEC_PAGE_SIZE * p.D;

    SV_TRY(tree_prep(draft_tokens, tree_parent, ctx_len, kv->block_table, kv->max_pages_per_req,
                     kv->n_pages, p.B, p.K, p.V, ni, stream));
    int *ctr = p.n_ctr > 0 ? at<int>(workspace, p.o_ctr) : nullptr;
    if (ctr) SV_TRY(zero_ints(ctr, p.n_ctr, stream));
    SV_TRY(rope_table(ni, M, p.D, w->cfg.rope_theta, stream));
    if (fused) {
        FusedArgs fa = {};
        fa.Lt = p.L;
        fa.H = p.H;
        fa.nq = p.nq;
        fa.nkv = p.nkv;
        fa.D = p.D;
        fa.F = p.F;
        fa.B = p.B;
        fa.K = p.K;
        fa.M = M;
        fa.G = fc.G;
        fa.eps = eps;
        fa.scale_log2 = kLog2e / sqrtf((float)p.D);
        fa.g_final = static_cast<const bf16 *>(w->final_norm);
        fa.k_pool = static_cast<bf16 *>(kv->k_pool);
        fa.v_pool = static_cast<bf16 *>(kv->v_pool);
        fa.layer_stride = layer_stride;
        fa.block_table = kv->block_table;
        fa.max_pages = kv->max_pages_per_req;
        fa.ctx_len = ctx_len;
        fa.status = ni.status;
        fa.anc = ni.anc;
        fa.rope = ni.rope;
        fa.x_o = at<bf16>(workspace, p.f_x);
        fa.x_d = fa.x_o + (size_t)kFusedMaxLayers * 16 * p.H;
        fa.ssq_o = at<float>(workspace, p.f_ssq_o);
        fa.ssq_d = at<float>(workspace, p.f_ssq_d);
        fa.q = at<bf16>(workspace, p.f_q);
        fa.ao = at<bf16>(workspace, p.f_ao);
        fa.h = at<bf16>(workspace, p.f_h);
        fa.u_head = at<bf16>(workspace, p.f_u);
        fa.trace = trace;
        uint32_t *sync = at<uint32_t>(workspace, p.f_sync);
        uint32_t *sw = sync;
        for (int ph = 0; ph < 4; ++ph) {
            FusedPhase &q = fa.ph[ph];
            q.S = fc.S[ph];
            q.groups = fc.groups[ph];
            q.units = fc.units[ph];
            q.g_eff = fc.g_eff[ph];
            q.max_parts = fc.max_parts[ph];
            q.part = at<float>(workspace, p.f_part[ph]);
            q.cnt = sw;
            sw += q.groups;
            q.flag = sw;
            sw += q.groups;
        }
        fa.CH = fc.CH;
        fa.n_chunks = fc.n_chunks;
        fa.n_items = fc.n_items;
        fa.n_tasks = fc.n_tasks;
        fa.att_o = at<float>(workspace, p.f_att_o);
        fa.att_ml = at<uint64_t>(workspace, p.f_att_ml);
        fa.f_att = sw;
        sw += fc.n_items;
        fa.f_comb = sw;
        sw += fc.n_tasks;
        fa.err = sw;
        fa.trace_t = extras ? extras->phase_trace : nullptr;
        SV_TRY(fused_prep(fa, draft_tokens, static_cast<const bf16 *>(w->embed), p.V, sync, fc.n_sync, stream));
        hipEvent_t *lev = extras ? extras->layer_events : nullptr;
        for (int l0 = 0, launch = 0; l0 < p.L; l0 += kFusedMaxLayers, ++launch) {
            fa.L0 = l0;
            fa.nl = p.L - l0 < kFusedMaxLayers ? p.L - l0 : kFusedMaxLayers;
            for (int li = 0; li < fa.nl; ++li) {
                const spec_layer_weights &lw = w->layers[l0 + li];
                fa.w[li][FUSED_QKV] = static_cast<const bf16 *>(lw.w_qkv);
                fa.w[li][FUSED_O] = static_cast<const bf16 *>(lw.w_o);
                fa.w[li][FUSED_GU] = static_cast<const bf16 *>(lw.w_gate_up);
                fa.w[li][FUSED_DOWN] = static_cast<const bf16 *>(lw.w_down);
                fa.g_attn[li] = static_cast<const bf16 *>(lw.attn_norm);
                fa.g_mlp[li] = static_cast<const bf16 *>(lw.mlp_norm);
            }
            if (lev) SV_TRY(hipEventRecord(lev[2 * launch], stream));
            SV_TRY(fused_layers(fa, stream));
            if (lev) SV_TRY(hipEventRecord(lev[2 * launch + 1], stream));
        }
        GemmEpi ep = {};
        ep.logits = logits;
        ep.amax_val = amv;
        ep.amax_idx = ami;
        GemmIn in = {};
        in.Xp = fa.u_head;
        SV_TRY(gemm(p.g_lm, EPI_ARGMAX, in, static_cast<const bf16 *>(w->lm_head), ep, stream));
        SV_TRY(argmax_accept(amv, ami, p.lm_groups, draft_tokens, tree_parent, ni, p.B, p.K, greedy,
                             accepted_len, bonus_token, accepted_path, stream, fa.err));
        return SPEC_OK;
    }

    SV_TRY(embed_norm(draft_tokens, static_cast<const bf16 *>(w->embed),
                      static_cast<const bf16 *>(w->layers[0].attn_norm), M, p.H, p.V, eps, x, u, trace,
                      stream));

    GemmEpi ep = {};
    ep.F = p.F;
    ep.rope = ni.rope;
    ep.status = ni.status;
    ep.ctx_len = ctx_len;
    ep.block_table = kv->block_table;
    ep.max_pages = kv->max_pages_per_req;
    ep.K = p.K;
    ep.nq = p.nq;
    ep.nkv = p.nkv;
    ep.D = p.D;
    ep.q = q;
    ep.y = part;
    ep.ctr = ctr;
    ep.h = h;
    ep.logits = logits;
    ep.amax_val = amv;
    ep.amax_idx = ami;
    auto operand = [](const bf16 *Xp) {
        GemmIn in = {};
        in.Xp = Xp;
        return in;
    };

    AttnArgs aa;
    aa.q = q;
    aa.block_table = kv->block_table;
    aa.max_pages = kv->max_pages_per_req;
    aa.n_pages = kv->n_pages;
    aa.ctx_len = ctx_len;
    aa.anc = ni.anc;
    aa.status = ni.status;
    aa.B = p.B;
    aa.K = p.K;
    aa.nq = p.nq;
    aa.nkv = p.nkv;
    aa.D = p.D;
    aa.n_chunks = p.attn_chunks;
    aa.part_o = at<float>(workspace, p.o_po);
    aa.part_ml = at<float2>(workspace, p.o_pml);
    aa.out = attn;

    // one projection: bf16 fragments, or the same matrix in W12
    auto proj = [&](const GemmShape &gb, const GemmShape &gw, int epi, const GemmIn &in, const void *wb,
                    const spec_w12_matrix *wq) -> hipError_t {
        if (wq != nullptr) return gemm_w12(gw, epi, in, w12_ref(*wq), ep, stream);
        return gemm(gb, epi, in, static_cast<const bf16 *>(wb), ep, stream);
    };

    for (int l = 0; l < p.L; ++l) {
        const spec_layer_weights &lw = w->layers[l];
        const spec_w12_layer *lq = w12 ? &w->w12_layers[l] : nullptr;
        bf16 *kl = k_pool + l * layer_stride;
        bf16 *vl = v_pool + l * layer_stride;
        if (any_rec && w->layer_kind[l] == SPEC_LAYER_RECURRENT) {
            // recurrent mixer: [q | k | v | a] = u . W^T; g = -softplus(a); the tree pass over the
            // committed state; its output, rounded to bf16, is the O projection's operand. The
            // pass's keys, values and gates stay in the cache struct's buffers for the commit.
            const int64_t rl = (int64_t)l * M * p.qd;
            bf16 *rk = static_cast<bf16 *>(kv->rec_k) + rl;
            bf16 *rv = static_cast<bf16 *>(kv->rec_v) + rl;
            float *rg = kv->rec_g + (int64_t)l * M * p.nq;
            bf16 *rq = at<bf16>(workspace, p.o_rq);
            float *ro = at<float>(workspace, p.o_ro);
            SV_TRY(gemm(p.g_rqkv, EPI_PARTIAL, operand(u), static_cast<const bf16 *>(lw.w_qkv), ep, stream));
            SV_TRY(reduce_rec(part, p.g_rqkv.splits, M, p.nrec, p.nq, p.D, rq, rk, rv, rg, stream));
            SV_TRY(rec_tree(kv->rec_state[l], rq, rk, rv, rg, tree_parent, p.B, p.K, p.nq, p.D, ro,
                            at<int32_t>(workspace, p.o_rs), stream));
            SV_TRY(rec_operand(ro, M, p.qd, attn, stream));
        } else {
        // q, k, v = u . Wqkv^T (u = RMSNorm(x) * attn_norm); RoPE; K/V into the cache
        if (p.qkv_fused) {
            ep.k_pool = kl;
            ep.v_pool = vl;
            SV_TRY(proj(p.g_qkvf, p.g_qkvf, EPI_QKV, operand(u), lw.w_qkv, lq ? &lq->w_qkv : nullptr));
        } else {
            SV_TRY(proj(p.g_qkv, p.w_qkv, EPI_PARTIAL, operand(u), lw.w_qkv, lq ? &lq->w_qkv : nullptr));
            SV_TRY(reduce_qkv(part, lq ? p.w_qkv.splits : p.g_qkv.splits, ni, ctx_len, kv->block_table,
                              kv->max_pages_per_req, p.B, p.K, p.nq, p.nkv, p.D, q, kl, vl, stream));
        }
        aa.k_pool = kl;
        aa.v_pool = vl;
        SV_TRY(attention(aa, stream));
        }
        // x += o . Wo^T; u = RMSNorm(x) * mlp_norm
        SV_TRY(proj(p.g_o, p.w_o, EPI_PARTIAL, operand(attn), lw.w_o, lq ? &lq->w_o : nullptr));
        SV_TRY(reduce_resid_norm(part, lq ? p.w_o.splits : p.g_o.splits, M, p.H, static_cast<const bf16 *>(lw.mlp_norm),
                                 eps, x, u, nullptr, stream));
        // h = silu(u . Wgate^T) * (u . Wup^T)
        if (gu_events) SV_TRY(hipEventRecord(gu_events[2 * l], stream));
        SV_TRY(proj(p.g_gu, p.w_gu, EPI_SWIGLU, operand(u), lw.w_gate_up, lq ? &lq->w_gate_up : nullptr));
        if (gu_events) SV_TRY(hipEventRecord(gu_events[2 * l + 1], stream));
        // x += h . Wdown^T; u = RMSNorm(x) * (next layer's attn_norm, or the final norm)
        const bf16 *next_gain = l + 1 < p.L ? static_cast<const bf16 *>(w->layers[l + 1].attn_norm)
                                            : static_cast<const bf16 *>(w->final_norm);
        SV_TRY(proj(p.g_down, p.w_down, EPI_PARTIAL, operand(h), lw.w_down, lq ? &lq->w_down : nullptr));
        SV_TRY(reduce_resid_norm(part, lq ? p.w_down.splits : p.g_down.splits, M, p.H, next_gain, eps, x, u,
                                 trace ? trace + (int64_t)(l + 1) * M * p.H : nullptr, stream));
    }
    SV_TRY(proj(p.g_lm, p.w_lm, EPI_ARGMAX, operand(u), w->lm_head, w12_lm ? &w->w12_lm_head : nullptr));
    SV_TRY(argmax_accept(amv, ami, w12_lm ? p.lm_groups_w12 : p.lm_groups, draft_tokens, tree_parent, ni, p.B, p.K, greedy,
                         accepted_len, bonus_token, accepted_path, stream));
    return SPEC_OK;
}

int spec_commit_kv(const spec_model_cfg *cfg, const spec_kv_cache *kv, const int32_t *accepted_len,
                   const int32_t *accepted_path, int32_t *ctx_len, int batch, int k,
                   hipStream_t stream) {
    int rc = check_cfg(cfg);
    if (rc != SPEC_OK) return rc;
    if (kv == nullptr || accepted_len == nullptr || accepted_path == nullptr || ctx_len == nullptr)
        return SPEC_EINVAL;
    if (kv->k_pool == nullptr || kv->v_pool == nullptr || kv->block_table == nullptr ||
        kv->n_pages < 1 || kv->max_pages_per_req < 1)
        return SPEC_EINVAL;
    if (batch < 1 || k < 1) return SPEC_EINVAL;
    if (k > SPEC_MAX_K) return SPEC_EUNSUPPORTED;
    if (kv->rec_state != nullptr && (kv->rec_k == nullptr || kv->rec_v == nullptr || kv->rec_g == nullptr))
        return SPEC_EINVAL;
    SV_TRY(commit_kv(accepted_len, accepted_path, ctx_len, kv->block_table, kv->max_pages_per_req,
                     kv->n_pages, cfg->n_layers, batch, k, cfg->n_kv_heads, cfg->head_dim,
                     static_cast<bf16 *>(kv->k_pool), static_cast<bf16 *>(kv->v_pool), stream));
    SV_TRY(commit_ctx(accepted_len, accepted_path, kv->block_table, kv->max_pages_per_req,
                      kv->n_pages, k, ctx_len, batch, stream));
    if (kv->rec_state != nullptr) {
        // recurrent layers of a hybrid target: each state after the accepted path, from the
        // pass's keys, values and gates
        const int64_t M = (int64_t)batch * k;
        const int qd = cfg->n_q_heads * cfg->head_dim;
        for (int l = 0; l < cfg->n_layers; ++l) {
            if (kv->rec_state[l] == nullptr) continue;
            SV_TRY(rec_commit(kv->rec_state[l], static_cast<const bf16 *>(kv->rec_k) + l * M * qd,
                              static_cast<const bf16 *>(kv->rec_v) + l * M * qd,
                              kv->rec_g + l * M * cfg->n_q_heads, accepted_len, accepted_path, batch, k,
                              cfg->n_q_heads, cfg->head_dim, stream));
        }
    }
    return SPEC_OK;
}

static int skinny_shape(int m, int n, int kd, GemmShape &g, bool w12 = false) {
    if (m < 1 || n < 1 || kd < 1) return SPEC_EINVAL;
    if (kd % 32 != 0 || n % 16 != 0) return SPEC_EUNSUPPORTED;
    g = w12 ? plan_gemm_w12(m, n, kd, true) : plan_gemm(m, n, kd, true);
    return SPEC_OK;
}

int spec_pack_weight(const void *w, int n, int kd, void *packed, hipStream_t stream) {
    if (w == nullptr || packed == nullptr) return SPEC_EINVAL;
    if (n < 1 || kd < 1) return SPEC_EINVAL;
    if (n % 16 != 0 || kd % 32 != 0) return SPEC_EUNSUPPORTED;
    if (w == packed) return SPEC_EINVAL;
    // rows are read and written 16 bytes at a time
    if (reinterpret_cast<uintptr_t>(w) % 16 != 0 || reinterpret_cast<uintptr_t>(packed) % 16 != 0)
        return SPEC_EINVAL;
    SV_TRY(pack_weight(static_cast<const bf16 *>(w), n, kd, static_cast<bf16 *>(packed), stream));
    return SPEC_OK;
}

// The partials, then (256-byte aligned) x in fragment order.
static size_t skinny_partial_bytes(const GemmShape &g, int m, int n) {
    return ((size_t)g.splits * m * n * sizeof(float) + 255) / 256 * 256;
}
static size_t skinny_total_bytes(const GemmShape &g, int m, int n, int kd) {
    return skinny_partial_bytes(g, m, n) + (size_t)(m + 15) / 16 * 16 * kd * sizeof(uint16_t);
}

int spec_skinny_gemm_bytes(int m, int n, int kd, size_t *bytes) {
    if (bytes == nullptr) return SPEC_EINVAL;
    GemmShape g, gq;
    int rc = skinny_shape(m, n, kd, g);
    if (rc != SPEC_OK) return rc;
    rc = skinny_shape(m, n, kd, gq, true);
    if (rc != SPEC_OK) return rc;
    const size_t a = skinny_total_bytes(g, m, n, kd), b = skinny_total_bytes(gq, m, n, kd);
    *bytes = a > b ? a : b;
    return SPEC_OK;
}

int spec_skinny_gemm(const void *x, int m, int kd, const void *w, int n, float *partials,
                     size_t partial_bytes, int *splits, hipStream_t stream) {
    if (x == nullptr || w == nullptr || partials == nullptr || splits == nullptr) return SPEC_EINVAL;
    GemmShape g;
    const int rc = skinny_shape(m, n, kd, g);
    if (rc != SPEC_OK) return rc;
    if (partial_bytes < skinny_total_bytes(g, m, n, kd)) return SPEC_EWORKSPACE;
    if (reinterpret_cast<uintptr_t>(partials) % 256 != 0) return SPEC_EINVAL;
    if (reinterpret_cast<uintptr_t>(x) % 16 != 0) return SPEC_EINVAL;   // rows read 16 bytes at a time
    *splits = g.splits;
    bf16 *xp = reinterpret_cast<bf16 *>(reinterpret_cast<char *>(partials) +
                                        skinny_partial_bytes(g, m, n));
    SV_TRY(pack_weight(static_cast<const bf16 *>(x), m, kd, xp, stream));
    GemmIn in = {};
    in.Xp = xp;
    GemmEpi ep = {};
    ep.y = partials;
    SV_TRY(gemm(g, EPI_PARTIAL, in, static_cast<const bf16 *>(w), ep, stream));
    return SPEC_OK;
}

int spec_skinny_gemm_w12(const void *x, int m, int kd, const spec_w12_matrix *w, int n,
                         float *partials, size_t partial_bytes, int *splits, hipStream_t stream) {
    if (x == nullptr || w == nullptr || partials == nullptr || splits == nullptr) return SPEC_EINVAL;
    if (!w12_ok(*w)) return SPEC_EINVAL;
    GemmShape g;
    const int rc = skinny_shape(m, n, kd, g, true);
    if (rc != SPEC_OK) return rc;
    if (partial_bytes < skinny_total_bytes(g, m, n, kd)) return SPEC_EWORKSPACE;
    if (reinterpret_cast<uintptr_t>(partials) % 256 != 0) return SPEC_EINVAL;
    if (reinterpret_cast<uintptr_t>(x) % 16 != 0) return SPEC_EINVAL;   // rows read 16 bytes at a time
    *splits = g.splits;
    bf16 *xp = reinterpret_cast<bf16 *>(reinterpret_cast<char *>(partials) +
                                        skinny_partial_bytes(g, m, n));
    SV_TRY(pack_weight(static_cast<const bf16 *>(x), m, kd, xp, stream));
    GemmIn in = {};
    in.Xp = xp;
    GemmEpi ep = {};
    ep.y = partials;
    SV_TRY(gemm_w12(g, EPI_PARTIAL, in, w12_ref(*w), ep, stream));
    return SPEC_OK;
}

static int w12_dims(int n, int kd) {
    if (n < 1 || kd < 1) return SPEC_EINVAL;
    if (n % 16 != 0 || kd % 32 != 0) return SPEC_EUNSUPPORTED;
    if ((int64_t)kd * 16 > (1 << 30)) return SPEC_EUNSUPPORTED;   // positions fit an int32
    return SPEC_OK;
}

// a row-major source matrix: read 16 bytes at a time
static int w12_shape(const void *w, int n, int kd) {
    if (w == nullptr || reinterpret_cast<uintptr_t>(w) % 16 != 0) return SPEC_EINVAL;
    return w12_dims(n, kd);
}

int spec_w12_plan_ints(int n, int kd, size_t *ints) {
    if (ints == nullptr) return SPEC_EINVAL;
    int rc = w12_dims(n, kd);
    if (rc != SPEC_OK) return rc;
    *ints = (size_t)w12_plan_ints(n);
    return SPEC_OK;
}

int spec_w12_plan(const void *w, int n, int kd, int32_t *plan, hipStream_t stream) {
    int rc = w12_shape(w, n, kd);
    if (rc != SPEC_OK) return rc;
    if (plan == nullptr) return SPEC_EINVAL;
    SV_TRY(w12_plan(static_cast<const bf16 *>(w), n, kd, plan, stream));
    return SPEC_OK;
}

int spec_w12_pack(const void *w, int n, int kd, const int32_t *plan, void *planes, int32_t *exc,
                  hipStream_t stream) {
    int rc = w12_shape(w, n, kd);
    if (rc != SPEC_OK) return rc;
    if (plan == nullptr || planes == nullptr || exc == nullptr) return SPEC_EINVAL;
    if (reinterpret_cast<uintptr_t>(planes) % 16 != 0 || reinterpret_cast<uintptr_t>(exc) % 8 != 0)
        return SPEC_EINVAL;
    SV_TRY(w12_pack(static_cast<const bf16 *>(w), n, kd, plan, static_cast<uint32_t *>(planes),
                    reinterpret_cast<int2 *>(exc), stream));
    return SPEC_OK;
}

// The chunked prefill: up to kPrefillRows prompt positions per pass (over all requests), each
// pass a full target pass over those rows: the tile projections (matrix-core bound at hundreds of
// rows), RoPE and the cache writes, causal attention over the cache, the output head only for the
// last position of each request.
constexpr int kPrefillRows = 4096;

struct PrefillLayout {
    int C;                           // prompt positions per request per pass
    GemmShape g_lm, w_lm;
    int n_ctr;                       // arrival counters of a balanced gate/up launch (0: none)
    size_t x, u, q, attn, h, part, pos, rope, status, failed, tokens, head_u, amv, ami, ctr, total;
};

static void prefill_shapes(const spec_model_cfg *cfg, int M, GemmShape (&g)[4], GemmShape (&w)[4]) {
    const int qd = cfg->n_q_heads * cfg->head_dim, nqkv = (cfg->n_q_heads + 2 * cfg->n_kv_heads) * cfg->head_dim;
    const int N[4] = {nqkv, cfg->hidden, 2 * cfg->ffn, cfg->hidden};
    const int Kd[4] = {cfg->hidden, qd, cfg->hidden, cfg->ffn};
    for (int i = 0; i < 4; ++i) {
        g[i] = plan_gemm(M, N[i], Kd[i], i != 2);
        w[i] = plan_gemm_w12(M, N[i], Kd[i], i != 2);
    }
}

// Sized for the longest prompt the page budget allows (max_pages * 16 positions per request).
static int prefill_layout(const spec_model_cfg *cfg, int batch, int max_pages, PrefillLayout &o) {
    int rc = check_cfg(cfg);
    if (rc != SPEC_OK) return rc;
    if (batch < 1 || max_pages < 1) return SPEC_EINVAL;
    if ((int64_t)batch > kPrefillRows * 16) return SPEC_EUNSUPPORTED;
    o.C = kPrefillRows / batch;
    if (o.C < 1) o.C = 1;
    if ((int64_t)o.C > (int64_t)max_pages * SPEC_PAGE_SIZE) o.C = max_pages * SPEC_PAGE_SIZE;
    const int M = batch * o.C, Mp = (M + 15) / 16 * 16, Bp = (batch + 15) / 16 * 16;
    const int H = cfg->hidden, qd = cfg->n_q_heads * cfg->head_dim, F = cfg->ffn, D = cfg->head_dim;
    GemmShape g[4], w[4];
    prefill_shapes(cfg, M, g, w);
    size_t part = 16;
    for (int i = 0; i < 4; ++i)
        for (const GemmShape *s : {&g[i], &w[i]}) {
            const size_t b = (size_t)s->splits * M * s->N * sizeof(float);
            if (i != 2 && b > part) part = b;
        }
    // a pass of 17..127 rows (a short last pass) runs gate/up on the wide kernel, balanced over the
    // compute units where the shape allows: its scratch and counters
    const GemmShape gb = plan_gemm(64, 2 * F, H, false);
    if (gemm_bal_scratch_bytes(gb) > part) part = gemm_bal_scratch_bytes(gb);
    o.n_ctr = gemm_bal_counters(gb);
    o.g_lm = plan_gemm(batch, cfg->vocab, H, false);
    o.w_lm = plan_gemm_w12(batch, cfg->vocab, H, false);
    const int groups = gemm_groups(o.g_lm) > gemm_groups(o.w_lm) ? gemm_groups(o.g_lm) : gemm_groups(o.w_lm);
    Carver cv;
    o.x = cv.take(sizeof(uint16_t) * M * H);
    o.u = cv.take(sizeof(uint16_t) * Mp * H);
    o.q = cv.take(sizeof(uint16_t) * M * qd);
    o.attn = cv.take(sizeof(uint16_t) * Mp * qd);
    o.h = cv.take(sizeof(uint16_t) * Mp * F);
    o.part = cv.take(part);
    o.pos = cv.take(sizeof(int32_t) * M);
    o.rope = cv.take(sizeof(float) * 2 * M * (D / 2));
    o.status = cv.take(sizeof(int32_t) * batch);
    o.failed = cv.take(sizeof(int32_t) * batch);
    o.tokens = cv.take(sizeof(int32_t) * M);
    o.head_u = cv.take(sizeof(uint16_t) * Bp * H);
    o.amv = cv.take(sizeof(float) * groups * batch);
    o.ami = cv.take(sizeof(int32_t) * groups * batch);
    o.ctr = cv.take(sizeof(int32_t) * (o.n_ctr > 0 ? o.n_ctr : 1));
    o.total = cv.off;
    return SPEC_OK;
}

int spec_prefill_workspace_bytes(const spec_model_cfg *cfg, int batch, int max_pages_per_req, int want_logits,
                                 size_t *bytes) {
    (void)want_logits;   // the last positions' logits go straight to the caller's buffer
    if (bytes == nullptr) return SPEC_EINVAL;
    PrefillLayout o;
    const int rc = prefill_layout(cfg, batch, max_pages_per_req, o);
    if (rc != SPEC_OK) return rc;
    *bytes = o.total;
    return SPEC_OK;
}

int spec_prefill(const spec_weights *weights, const spec_kv_cache *kv, const int32_t *prompt,
                 int32_t *ctx_len, int batch, int p, int32_t *next_token, float *last_logits,
                 void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (weights == nullptr || kv == nullptr || prompt == nullptr || ctx_len == nullptr ||
        next_token == nullptr || workspace == nullptr)
        return SPEC_EINVAL;
    if (batch < 1 || p < 1) return SPEC_EINVAL;
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return SPEC_EINVAL;
    if (kv->k_pool == nullptr || kv->v_pool == nullptr || kv->block_table == nullptr || kv->n_pages < 1 ||
        kv->max_pages_per_req < 1)
        return SPEC_EINVAL;
    const spec_weights *w = weights;
    if (w->layers == nullptr || w->embed == nullptr || w->final_norm == nullptr) return SPEC_EINVAL;
    if (w->layer_kind != nullptr)
        for (int l = 0; l < w->cfg.n_layers; ++l)
            if (w->layer_kind[l] != SPEC_LAYER_ATTENTION) return SPEC_EUNSUPPORTED;
    const bool w12 = w->w12_layers != nullptr;
    const bool w12_lm = w->w12_lm_head.planes != nullptr;
    if (!w12_lm && w->lm_head == nullptr) return SPEC_EINVAL;
    if (w12_lm && !w12_ok(w->w12_lm_head)) return SPEC_EINVAL;
    for (int l = 0; l < w->cfg.n_layers; ++l) {
        const spec_layer_weights &lw = w->layers[l];
        if (!lw.attn_norm || !lw.mlp_norm) return SPEC_EINVAL;
        if (w12) {
            const spec_w12_layer &q = w->w12_layers[l];
            if (!w12_ok(q.w_qkv) || !w12_ok(q.w_o) || !w12_ok(q.w_gate_up) || !w12_ok(q.w_down)) return SPEC_EINVAL;
        } else if (!lw.w_qkv || !lw.w_o || !lw.w_gate_up || !lw.w_down) {
            return SPEC_EINVAL;
        }
    }
    const spec_model_cfg *cfg = &w->cfg;
    if (cfg->n_q_heads / cfg->n_kv_heads > 8) return SPEC_EUNSUPPORTED;   // query tiles per workgroup
    PrefillLayout o;
    int rc = prefill_layout(cfg, batch, kv->max_pages_per_req, o);
    if (rc != SPEC_OK) return rc;
    if (workspace_bytes < o.total) return SPEC_EWORKSPACE;

    const int H = cfg->hidden, nq = cfg->n_q_heads, nkv = cfg->n_kv_heads, D = cfg->head_dim, V = cfg->vocab;
    const float eps = cfg->rms_eps;
    bf16 *x = at<bf16>(workspace, o.x), *u = at<bf16>(workspace, o.u), *q = at<bf16>(workspace, o.q);
    bf16 *attn = at<bf16>(workspace, o.attn), *h = at<bf16>(workspace, o.h);
    float *part = at<float>(workspace, o.part);
    int32_t *status = at<int32_t>(workspace, o.status), *failed = at<int32_t>(workspace, o.failed);
    int32_t *tokens = at<int32_t>(workspace, o.tokens);
    float *amv = at<float>(workspace, o.amv);
    int *ami = at<int>(workspace, o.ami);
    NodeInfo ni = {};
    ni.pos = at<int32_t>(workspace, o.pos);
    ni.status = status;
    ni.rope = at<float2>(workspace, o.rope);
    bf16 *k_pool = static_cast<bf16 *>(kv->k_pool), *v_pool = static_cast<bf16 *>(kv->v_pool);
    const int64_t layer_stride = (int64_t)kv->n_pages * nkv * SPEC_PAGE_SIZE * D;

    GemmEpi ep = {};
    ep.F = cfg->ffn;
    ep.y = part;
    ep.h = h;
    ep.ctr = o.n_ctr > 0 ? at<int>(workspace, o.ctr) : nullptr;
    auto operand = [](const bf16 *Xp) {
        GemmIn in = {};
        in.Xp = Xp;
        return in;
    };
    SV_TRY(prefill_init(failed, batch, stream));
    if (ep.ctr) SV_TRY(zero_ints(ep.ctr, o.n_ctr, stream));
    for (int c0 = 0; c0 < p; c0 += o.C) {
        const int n = p - c0 < o.C ? p - c0 : o.C;
        const int M = batch * n;
        const bool last = c0 + n == p;
        GemmShape g[4], gw[4];
        prefill_shapes(cfg, M, g, gw);
        auto proj = [&](int i, int epi, const GemmIn &in, const void *wb, const spec_w12_matrix *wq) -> hipError_t {
            if (wq != nullptr) return gemm_w12(gw[i], epi, in, w12_ref(*wq), ep, stream);
            return gemm(g[i], epi, in, static_cast<const bf16 *>(wb), ep, stream);
        };
        SV_TRY(prefill_gather(prompt, p, c0, n, batch, tokens, stream));
        SV_TRY(prefill_prep(tokens, n, batch, V, ctx_len, kv->block_table, kv->max_pages_per_req, kv->n_pages,
                            failed, ni.pos, status, stream));
        SV_TRY(rope_table(ni, M, D, cfg->rope_theta, stream));
        SV_TRY(embed_norm(tokens, static_cast<const bf16 *>(w->embed),
                          static_cast<const bf16 *>(w->layers[0].attn_norm), M, H, V, eps, x, u, nullptr, stream));
        for (int l = 0; l < cfg->n_layers; ++l) {
            const spec_layer_weights &lw = w->layers[l];
            const spec_w12_layer *lq = w12 ? &w->w12_layers[l] : nullptr;
            bf16 *kl = k_pool + l * layer_stride, *vl = v_pool + l * layer_stride;
            SV_TRY(proj(0, EPI_PARTIAL, operand(u), lw.w_qkv, lq ? &lq->w_qkv : nullptr));
            SV_TRY(reduce_qkv(part, (lq ? gw[0] : g[0]).splits, ni, ctx_len, kv->block_table, kv->max_pages_per_req,
                              batch, n, nq, nkv, D, q, kl, vl, stream));
            SV_TRY(prefill_attention(q, kl, vl, kv->block_table, kv->max_pages_per_req, ctx_len, status, batch, n, nq,
                                     nkv, D, attn, stream));
            SV_TRY(proj(1, EPI_PARTIAL, operand(attn), lw.w_o, lq ? &lq->w_o : nullptr));
            SV_TRY(reduce_resid_norm(part, (lq ? gw[1] : g[1]).splits, M, H, static_cast<const bf16 *>(lw.mlp_norm),
                                     eps, x, u, nullptr, stream));
            SV_TRY(proj(2, EPI_SWIGLU, operand(u), lw.w_gate_up, lq ? &lq->w_gate_up : nullptr));
            const bf16 *next_gain = l + 1 < cfg->n_layers ? static_cast<const bf16 *>(w->layers[l + 1].attn_norm)
                                                          : static_cast<const bf16 *>(w->final_norm);
            SV_TRY(proj(3, EPI_PARTIAL, operand(h), lw.w_down, lq ? &lq->w_down : nullptr));
            SV_TRY(reduce_resid_norm(part, (lq ? gw[3] : g[3]).splits, M, H, next_gain, eps, x, u, nullptr, stream));
        }
        int groups = 0;
        if (last) {
            // the output head for each request's last position only
            bf16 *hu = at<bf16>(workspace, o.head_u);
            SV_TRY(prefill_last_rows(u, n, batch, H, hu, stream));
            GemmEpi eh = {};
            eh.logits = last_logits;
            eh.amax_val = amv;
            eh.amax_idx = ami;
            if (w12_lm) {
                SV_TRY(gemm_w12(o.w_lm, EPI_ARGMAX, operand(hu), w12_ref(w->w12_lm_head), eh, stream));
                groups = gemm_groups(o.w_lm);
            } else {
                SV_TRY(gemm(o.g_lm, EPI_ARGMAX, operand(hu), static_cast<const bf16 *>(w->lm_head), eh, stream));
                groups = gemm_groups(o.g_lm);
            }
        }
        SV_TRY(prefill_finish(amv, ami, groups, batch, n, last, status, failed, ctx_len, next_token, stream));
    }
    return SPEC_OK;
}

static int rec_args(const void *a, const void *b, const void *c, const void *d, int batch, int k,
                    int n_heads, int head_dim) {
    for (const void *p : {a, b, c, d})
        if (p == nullptr || reinterpret_cast<uintptr_t>(p) % 16 != 0) return SPEC_EINVAL;
    if (batch < 1 || k < 1 || n_heads < 1) return SPEC_EINVAL;
    if (k > SPEC_MAX_K || (head_dim != 64 && head_dim != 128)) return SPEC_EUNSUPPORTED;
    if ((int64_t)batch * n_heads > (1 << 24)) return SPEC_EUNSUPPORTED;
    return SPEC_OK;
}

int spec_rec_tree_verify(const float *state, const void *q, const void *k, const void *v,
                         const float *log_gate, const int32_t *tree_parent, int batch, int k_nodes,
                         int n_heads, int head_dim, float *out, int32_t *status, hipStream_t stream) {
    int rc = rec_args(state, q, k, v, batch, k_nodes, n_heads, head_dim);
    if (rc != SPEC_OK) return rc;
    if (log_gate == nullptr || out == nullptr || status == nullptr) return SPEC_EINVAL;
    if (reinterpret_cast<uintptr_t>(out) % 16 != 0) return SPEC_EINVAL;
    SV_TRY(rec_tree(state, static_cast<const bf16 *>(q), static_cast<const bf16 *>(k),
                    static_cast<const bf16 *>(v), log_gate, tree_parent, batch, k_nodes, n_heads,
                    head_dim, out, status, stream));
    return SPEC_OK;
}

int spec_rec_commit(float *state, const void *k, const void *v, const float *log_gate,
                    const int32_t *accepted_len, const int32_t *accepted_path, int batch,
                    int k_nodes, int n_heads, int head_dim, hipStream_t stream) {
    int rc = rec_args(state, k, v, state, batch, k_nodes, n_heads, head_dim);
    if (rc != SPEC_OK) return rc;
    if (log_gate == nullptr || accepted_len == nullptr || accepted_path == nullptr) return SPEC_EINVAL;
    SV_TRY(rec_commit(state, static_cast<const bf16 *>(k), static_cast<const bf16 *>(v), log_gate,
                      accepted_len, accepted_path, batch, k_nodes, n_heads, head_dim, stream));
    return SPEC_OK;
}

int spec_read_probe(const void *buf, size_t bytes, uint32_t *out, hipStream_t stream) {
    if (buf == nullptr || out == nullptr || bytes == 0 || bytes % 16 != 0) return SPEC_EINVAL;
    if (reinterpret_cast<uintptr_t>(buf) % 16 != 0) return SPEC_EINVAL;
    SV_TRY(read_probe(buf, (int64_t)bytes, out, stream));
    return SPEC_OK;
}

int spec_accept_workspace_bytes(int batch, int k, int vocab, size_t *bytes) {
    if (bytes == nullptr || batch < 1 || k < 1 || vocab < 1) return SPEC_EINVAL;
    if (k > SPEC_MAX_K) return SPEC_EUNSUPPORTED;
    const int M = batch * k;
    const int nc = argmax_chunks(vocab);
    Carver cv;
    cv.take(sizeof(int32_t) * M);        // depth
    cv.take(sizeof(int32_t) * M);        // pos
    cv.take(sizeof(int32_t) * batch);    // status
    cv.take(sizeof(uint64_t) * M);       // anc
    cv.take(sizeof(float) * (size_t)nc * M);
    cv.take(sizeof(int32_t) * (size_t)nc * M);
    *bytes = cv.off;
    return SPEC_OK;
}

int spec_accept(const float *logits, const int32_t *draft_tokens, const int32_t *tree_parent,
                int batch, int k, int vocab, int32_t *accepted_len, int32_t *bonus_token,
                int32_t *accepted_path, int32_t *greedy, void *workspace, size_t workspace_bytes,
                hipStream_t stream) {
    if (logits == nullptr || draft_tokens == nullptr || accepted_len == nullptr ||
        bonus_token == nullptr || accepted_path == nullptr || workspace == nullptr)
        return SPEC_EINVAL;
    size_t need = 0;
    int rc = spec_accept_workspace_bytes(batch, k, vocab, &need);
    if (rc != SPEC_OK) return rc;
    if (workspace_bytes < need) return SPEC_EWORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return SPEC_EINVAL;
    const int M = batch * k;
    const int nc = argmax_chunks(vocab);
    Carver cv;
    NodeInfo ni;
    ni.depth = at<int32_t>(workspace, cv.take(sizeof(int32_t) * M));
    ni.pos = at<int32_t>(workspace, cv.take(sizeof(int32_t) * M));
    ni.status = at<int32_t>(workspace, cv.take(sizeof(int32_t) * batch));
    ni.anc = at<uint64_t>(workspace, cv.take(sizeof(uint64_t) * M));
    ni.rope = nullptr;
    float *amv = at<float>(workspace, cv.take(sizeof(float) * (size_t)nc * M));
    int *ami = at<int>(workspace, cv.take(sizeof(int32_t) * (size_t)nc * M));
    SV_TRY(tree_prep(draft_tokens, tree_parent, nullptr, nullptr, 0, 0, batch, k, vocab, ni, stream));
    SV_TRY(argmax_partials(logits, M, vocab, amv, ami, nc, stream));
    SV_TRY(argmax_accept(amv, ami, nc, draft_tokens, tree_parent, ni, batch, k, greedy, accepted_len,
                         bonus_token, accepted_path, stream));
    return SPEC_OK;
}

// ---- spec_accept without allocation: a static device scratch per GPU -----------------------------
// Largest spec_accept workspace within the limits: depth, pos, status, anc for 4096 rows and the
// greedy partials of 128 vocab chunks of 2048 (262144 / 2048) per row, each 256-byte aligned.
static_assert(SPEC_NOALLOC_SCRATCH_BYTES ==
                  4096 * 4 + 4096 * 4 + 4096 * 4 + 4096 * 8 + 128 * 4096 * 4 + 128 * 4096 * 4,
              "scratch size = the spec_accept layout at the limits");

}  // extern "C"

namespace {
// In host code this name is only a stand-in for the per-device copies; kernels get the address
// hipGetSymbolAddress returns on each device.
static __device__ __align__(256) unsigned char scratch[SPEC_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address, looked up once per device with that device current.
int scratch_ptr(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return SPEC_EHIP;
    if (dev < 0 || dev >= kMaxDevices) return SPEC_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SPEC_EHIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SPEC_OK;
}
}  // namespace

extern "C" {

int spec_accept_noalloc(const float *logits, const int32_t *draft_tokens, const int32_t *tree_parent,
                        int batch, int k, int vocab, int32_t *accepted_len, int32_t *bonus_token,
                        int32_t *accepted_path, int32_t *greedy, hipStream_t stream) {
    if (batch < 1 || k < 1 || vocab < 1) return SPEC_EINVAL;
    if ((int64_t)batch * k > SPEC_NOALLOC_MAX_ROWS || vocab > SPEC_NOALLOC_MAX_VOCAB) return SPEC_ESCRATCH;
    size_t need = 0;
    int rc = spec_accept_workspace_bytes(batch, k, vocab, &need);
    if (rc != SPEC_OK) return rc;
    if (need > SPEC_NOALLOC_SCRATCH_BYTES) return SPEC_ESCRATCH;
    void *ws = nullptr;
    rc = scratch_ptr(&ws);
    if (rc != SPEC_OK) return rc;
    return spec_accept(logits, draft_tokens, tree_parent, batch, k, vocab, accepted_len, bonus_token,
                       accepted_path, greedy, ws, SPEC_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
