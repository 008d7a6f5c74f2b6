"""Verify passes replayed from a captured HIP graph, the way bench.py times them, equal the eager
pass bit for bit on every replay. Between replays the program does eager work of its own: an eager
pass with other draft tokens over the same cache, workspace and output buffers, then the outputs
overwritten with garbage. Cases: the tiny decoder's block of 16 (the automatic and the per-step
plans) and a batch of two 64-node trees, and a 64-row tree pass and a block of 16 whose gate/up
runs balanced over the compute units (the wide and the skinny kernel; the arrival counters are
cleared inside the pass by a fill kernel, never by a memset, and left zero by the last arriver);
and prompt prefills from an empty context."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tree_verification_skinny_amd as tv
from tree_verification_skinny_amd import kvlayout

from helpers import bits, device_weights, make_kv, upload_context

pytestmark = pytest.mark.gpu
DEV = "cuda"

BALANCED = synth.Shape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=17408, vocab=1024)


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tv.lib()


@pytest.mark.parametrize("shape_name,B,K,tree,path", [("tiny", 1, 16, False, "auto"), ("tiny", 1, 16, False, "steps"),
                                                      ("tiny", 2, 64, True, "auto"), ("balanced", 1, 64, True, "auto"),
                                                      ("balanced", 1, 16, False, "auto")])
def test_graph_replays_equal_eager(shape_name, B, K, tree, path):
    shape = synth.TINY if shape_name == "tiny" else BALANCED
    seed = 2100 + 10 * B + K + (1 if path == "steps" else 0)
    ctxs = [300, 900][:B]
    w = synth.model_weights(shape, seed)
    weights = device_weights(shape, w, DEV)
    kv = make_kv(shape, ctxs, K, seed, DEV)
    for b, ctx in enumerate(ctxs):
        kvs = [synth.kv_context(shape, ctx, seed, l, request=b) for l in range(shape.n_layers)]
        upload_context(kv, b, [np.ascontiguousarray(bits(x)) for x, _ in kvs],
                       [np.ascontiguousarray(bits(y)) for _, y in kvs])
    if tree:
        parents = np.stack([synth.random_tree(K, 10, seed, "graph", b) for b in range(B)]).astype(np.int32)
    else:
        parents = np.stack([oracle.chain(K)] * B).astype(np.int32)
    tokens = np.stack([synth.uniform_tokens(K, shape.vocab, seed, "graph", b) for b in range(B)]).astype(np.int32)
    other = np.stack([synth.uniform_tokens(K, shape.vocab, seed, "graph other", b) for b in range(B)]).astype(np.int32)

    M = B * K
    t_tok = torch.from_numpy(tokens).to(DEV)
    t_other = torch.from_numpy(other).to(DEV)
    t_par = torch.from_numpy(parents).to(DEV) if tree else None
    t_ctx = torch.tensor(ctxs, dtype=torch.int32, device=DEV)
    acc = torch.empty(B, dtype=torch.int32, device=DEV)
    bonus = torch.empty(B, dtype=torch.int32, device=DEV)
    path_t = torch.empty((B, K), dtype=torch.int32, device=DEV)
    greedy = torch.empty(M, dtype=torch.int32, device=DEV)
    logits = torch.empty((M, shape.vocab), dtype=torch.float32, device=DEV)
    ws = tv.workspace(tv.spec_workspace_bytes(weights.cfg, B, K, kv.max_pages), DEV)
    ws.fill_(0xFF)

    def run(toks):
        tv.spec_verify(weights, kv, toks, t_par, t_ctx, B, K, acc, bonus, path_t, ws, logits=logits,
                       greedy=greedy, path=path)

    def outputs():
        return [logits.view(torch.int32).clone(), greedy.clone(), acc.clone(), bonus.clone(), path_t.clone()]

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        run(t_tok)
    stream.synchronize()
    ref = outputs()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        run(t_tok)
    torch.cuda.synchronize()

    for i in range(3):
        with torch.cuda.stream(stream):
            run(t_other)                        # the program's own eager pass, other draft tokens
            logits.fill_(float("nan"))
            for t in (greedy, acc, bonus, path_t):
                t.fill_(-7)
            graph.replay()
        stream.synchronize()
        got = outputs()
        for name, a, b in zip(("logits", "greedy", "accepted_len", "bonus", "path"), ref, got):
            assert torch.equal(a, b), f"replay {i}: {name} differs from the eager pass"
    del graph


@pytest.mark.parametrize("B,p", [(2, 40), (1, 300)])
def test_graph_prefill_replays_equal_eager(B, p):
    """spec_prefill from an empty context replayed from a graph (as bench.py times a prefill): each
    replay, after the contexts are reset eagerly and an eager prefill of another prompt has run,
    gives the eager pass's next tokens, last-position logits and cache rows bit for bit."""
    shape = synth.TINY
    seed = 2300 + B + p
    w = synth.model_weights(shape, seed)
    weights = device_weights(shape, w, DEV)
    kv = make_kv(shape, [p] * B, 1, seed, DEV)
    rng = np.random.default_rng(synth.seed_of(seed, "graph prefill"))
    prompts = torch.from_numpy(rng.integers(0, shape.vocab, (B, p)).astype(np.int32)).to(DEV)
    other = torch.from_numpy(rng.integers(0, shape.vocab, (B, p)).astype(np.int32)).to(DEV)
    ws = tv.workspace(tv.spec_prefill_workspace_bytes(weights.cfg, B, kv.max_pages, True), DEV)
    ctx = torch.zeros(B, dtype=torch.int32, device=DEV)
    nt = torch.empty(B, dtype=torch.int32, device=DEV)
    lg = torch.empty((B, shape.vocab), dtype=torch.float32, device=DEV)

    def run(pr):
        tv.spec_prefill(weights, kv, pr, ctx, nt, ws, last_logits=lg)

    def rows():
        return [torch.cat([t.view(torch.int16).reshape(-1) for t in kvlayout.read_rows(kv, l, b, torch.arange(p))])
                for l in range(shape.n_layers) for b in range(B)]

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        run(prompts)
    stream.synchronize()
    ref = [nt.clone(), lg.view(torch.int32).clone(), ctx.clone()] + rows()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        ctx.zero_()
    stream.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        run(prompts)
    torch.cuda.synchronize()

    for i in range(3):
        with torch.cuda.stream(stream):
            ctx.zero_()
            run(other)                          # the program's own eager prefill, another prompt
            ctx.zero_()
            nt.fill_(-7)
            lg.fill_(float("nan"))
            graph.replay()
        stream.synchronize()
        got = [nt.clone(), lg.view(torch.int32).clone(), ctx.clone()] + rows()
        for j, (a, b) in enumerate(zip(ref, got)):
            assert torch.equal(a, b), f"replay {i}: output {j} differs from the eager prefill"
    del graph
