"""The full 27B-class stack (64 layers + output head over 151936 tokens, ~45 GB of bf16
weights drawn on the GPU) at the launch configuration bench.py times, checked layer by layer
with teacher forcing: the oracle (and an exact float64 evaluation) take the GPU's own residual
stream entering a sampled layer, and their outputs are compared with the GPU's output of that
layer; the output head and the greedy walk are checked from the GPU's final residual stream.
Teacher forcing separates kernel errors from the growth of legitimate rounding differences over
64 layers of a random-weight model."""
import numpy as np
import pytest
import torch

import oracle
import ref64
import synth
import tree_verification_skinny_amd as tv
from tree_verification_skinny_amd import kvlayout

from helpers import bits, check_accept, check_as_exact, check_logits, oracle_cfg, run_verify

pytestmark = pytest.mark.gpu
DEV = "cuda"
SEED = 27


@pytest.fixture(scope="module")
def stack():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    shape = synth.DENSE_27B
    layers = [synth.layer_weights(shape, SEED, l, DEV) for l in range(shape.n_layers)]
    embed = synth.randn_bf16((shape.vocab, shape.hidden), 0.02, DEV, SEED, "embed")
    lm = synth.randn_bf16((shape.vocab, shape.hidden), 0.02, DEV, SEED, "lm_head")
    fn = torch.ones(shape.hidden, dtype=torch.bfloat16, device=DEV)
    w = tv.Weights(tv.ModelCfg.of(shape), embed, fn, lm, layers)
    yield shape, w
    del w, layers, embed, lm
    torch.cuda.empty_cache()


def _case(shape, w, kind, path="auto"):
    if kind == "block":
        k, ctx = 16, 4096
        parent = oracle.chain(k)
        tokens = synth.uniform_tokens(k, shape.vocab, SEED, "blk")
    else:
        k, ctx = 64, 8192
        parent = synth.random_tree(k, 10, SEED, "tree")
        tokens = synth.tree_tokens(parent, shape.vocab, SEED, "tree")
    pages = (ctx + k + 15) // 16
    table = torch.arange(pages, dtype=torch.int32).view(1, pages)
    kv = tv.PagedKV.empty(w.cfg, pages, table, DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(SEED)
    kv.k_pool.normal_(generator=g)
    kv.v_pool.normal_(generator=g)
    ctx_rows = [kvlayout.read_rows(kv, l, 0, torch.arange(ctx)) for l in range(shape.n_layers)]
    out = run_verify(w, kv, tokens[None], None if kind == "block" else parent[None], [ctx],
                     want_hidden=True, path=path)
    return k, ctx, parent, tokens, kv, ctx_rows, out


@pytest.mark.parametrize("kind,path", [("block", "persistent"), ("block", "steps"), ("tree", "auto")])
def test_27b_stack_teacher_forced(stack, kind, path):
    """The block runs both launch plans: the persistent kernel (the default at 16 rows) and one
    kernel per step; the 64-node tree runs the per-step plan."""
    shape, w = stack
    print(f"27B stack {kind} path={path}", flush=True)
    k, ctx, parent, tokens, kv, ctx_rows, out = _case(shape, w, kind, path)
    cfg = oracle_cfg(shape)
    for l in (0, 1, 31, 62, 63):
        lw = {nm: bits(t) for nm, t in w.rowmajor["layers"][l].items()}
        kc, vc = bits(ctx_rows[l][0]), bits(ctx_rows[l][1])
        x_in = bits(out.hidden[l])
        x_o, k_o, v_o = oracle.layer_forward(cfg, lw, kc, vc, parent, x_in)
        x_r, _, _ = ref64.layer(shape, lw, kc, vc, parent, x_in)
        kg, vg = kvlayout.read_rows(kv, l, 0, torch.arange(ctx, ctx + k))
        check_logits(kg.float().cpu().numpy(), oracle.from_bf16(k_o), f"layer {l} k_new")
        check_logits(vg.float().cpu().numpy(), oracle.from_bf16(v_o), f"layer {l} v_new")
        print(check_as_exact(out.hidden[l + 1].float().cpu().numpy(), oracle.from_bf16(x_o),
                             x_r.numpy(), f"layer {l} output"))
    # output head and greedy walk from the GPU's final residual stream: fixed tolerance
    model = oracle.Model(cfg, bits(w.tensors["embed"][:1]), bits(w.tensors["final_norm"]),
                         bits(w.rowmajor["lm_head"]), layers=[])
    lg = oracle.logits(model, bits(out.hidden[shape.n_layers]))
    err = check_logits(out.logits[0], lg, "output head")
    arg, margin = oracle.argmax(lg)
    a, b, p = oracle.accept(tokens, parent, arg)
    r = oracle.VerifyResult(lg, arg, margin, a, b, p, [], [], [])
    near = check_accept(r, tokens, parent, out.greedy[0], int(out.accepted_len[0]),
                        int(out.bonus[0]), out.path[0])
    print(f"{kind}: head max err {err:.2e}, accepted {out.accepted_len[0]}, near-tie {near}")


def test_27b_batched_teacher_forced(stack):
    """The batched launch configuration: 32 requests x block of 16 (512 rows, the matrix-core
    tile projections and the range attention), contexts uniform in [512, 8192], shuffled pages.
    Sampled requests are checked layer by layer with teacher forcing, then through the output
    head and the greedy walk from the GPU's final residual stream."""
    shape, w = stack
    B, k = 32, 16
    rng = np.random.default_rng(synth.seed_of(SEED, "batched ctx"))
    ctxs = [int(c) for c in rng.integers(512, 8193, B)]
    table, n_pages = synth.page_table(B, [(c + k + 15) // 16 for c in ctxs], SEED, shuffle=True)
    kv = tv.PagedKV.empty(w.cfg, n_pages, torch.from_numpy(table), DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(SEED + 1)
    kv.k_pool.normal_(generator=g)
    kv.v_pool.normal_(generator=g)
    tokens = np.stack([synth.uniform_tokens(k, shape.vocab, SEED, "batched", b) for b in range(B)])
    tokens = tokens.astype(np.int32)
    out = run_verify(w, kv, tokens, None, ctxs, want_hidden=True)
    cfg = oracle_cfg(shape)
    parent = oracle.chain(k)
    for b in (0, 13, 31):
        rows = slice(b * k, (b + 1) * k)
        for l in (0, 37, 63):
            lw = {nm: bits(t) for nm, t in w.rowmajor["layers"][l].items()}
            kc, vc = kvlayout.read_rows(kv, l, b, torch.arange(ctxs[b]))
            kc, vc = bits(kc), bits(vc)
            x_in = bits(out.hidden[l][rows])
            x_o, k_o, v_o = oracle.layer_forward(cfg, lw, kc, vc, parent, x_in)
            x_r, _, _ = ref64.layer(shape, lw, kc, vc, parent, x_in)
            kg, vg = kvlayout.read_rows(kv, l, b, torch.arange(ctxs[b], ctxs[b] + k))
            check_logits(kg.float().cpu().numpy(), oracle.from_bf16(k_o), f"request {b} layer {l} k_new")
            check_logits(vg.float().cpu().numpy(), oracle.from_bf16(v_o), f"request {b} layer {l} v_new")
            print(check_as_exact(out.hidden[l + 1][rows].float().cpu().numpy(), oracle.from_bf16(x_o),
                                 x_r.numpy(), f"request {b} layer {l} output"))
        model = oracle.Model(cfg, bits(w.tensors["embed"][:1]), bits(w.tensors["final_norm"]),
                             bits(w.rowmajor["lm_head"]), layers=[])
        lg = oracle.logits(model, bits(out.hidden[shape.n_layers][rows]))
        err = check_logits(out.logits[b], lg, f"request {b} output head")
        arg, margin = oracle.argmax(lg)
        a, bo, p = oracle.accept(tokens[b], parent, arg)
        r = oracle.VerifyResult(lg, arg, margin, a, bo, p, [], [], [])
        near = check_accept(r, tokens[b], parent, out.greedy[b], int(out.accepted_len[b]),
                            int(out.bonus[b]), out.path[b])
        print(f"batched request {b} (ctx {ctxs[b]}): head max err {err:.2e}, near-tie {near}")


def test_27b_stack_w12_bit_identical(stack):
    """The same stack with its projections and output head in the lossless 12-bit layout: the
    block and the tree pass give bit-identical logits, residual streams, cache rows and accepted
    paths to the bf16 passes, so the teacher-forced oracle checks above carry over unchanged."""
    shape, w = stack
    w12 = tv.Weights(w.cfg, w.tensors["embed"], w.tensors["final_norm"], w.rowmajor["lm_head"],
                     w.rowmajor["layers"], w12=True)
    n_exc = sum(m.n_exc for lw in w12.w12["layers"] for m in lw.values()) + w12.w12["lm_head"].n_exc
    for kind in ("block", "tree"):
        # W12 runs the per-step kernels with the bf16 plans: compare with the bf16 per-step pass
        k, ctx, parent, tokens, kv, _, out = _case(shape, w, kind, "steps")
        k2, _, _, _, kv2, _, out2 = _case(shape, w12, kind)
        assert np.array_equal(out.logits.view(np.int32), out2.logits.view(np.int32)), kind
        assert torch.equal(out.hidden.view(torch.int16), out2.hidden.view(torch.int16)), kind
        assert np.array_equal(out.greedy, out2.greedy) and np.array_equal(out.path, out2.path)
        assert (out.accepted_len[0], out.bonus[0]) == (out2.accepted_len[0], out2.bonus[0])
        for l in (0, 63):
            a = kvlayout.read_rows(kv, l, 0, torch.arange(ctx, ctx + k))
            b = kvlayout.read_rows(kv2, l, 0, torch.arange(ctx, ctx + k))
            assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
            assert torch.equal(a[1].view(torch.int16), b[1].view(torch.int16))
        del kv, kv2, out, out2
    print(f"W12 stack: {n_exc} exceptions over {len(w12.w12['layers']) * 4 + 1} matrices")
    del w12
    torch.cuda.empty_cache()
