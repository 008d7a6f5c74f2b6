"""Verify passes replayed from a captured HIP graph, the way bench.py times them, equal the eager
pass bit for bit on every replay. Between replays the program does eager work of its own: an eager
pass with other draft tokens over the same cache, workspace and output buffers, then the outputs
overwritten with garbage. Cases: the tiny decoder's block of 16 (the automatic and the per-step
plans) and a batch of two 64-node trees, and a 64-row tree pass whose gate/up runs balanced over
the compute units (its arrival counters are cleared inside the pass by a fill kernel, never by a
memset, and left zero by the last arriver)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tree_verification_skinny_amd as tv

from helpers import bits, device_weights, make_kv, upload_context

pytestmark = pytest.mark.gpu
DEV = "cuda"

BALANCED = synth.Shape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=17408, vocab=1024)


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tv.lib()


@pytest.mark.parametrize("shape_name,B,K,tree,path", [("tiny", 1, 16, False, "auto"), ("tiny", 1, 16, False, "steps"),
                                                      ("tiny", 2, 64, True, "auto"), ("balanced", 1, 64, True, "auto")])
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
