"""Pins of the oracle's hybrid target: attention and recurrent layers in one decoder.

The pages name tree verification for targets that mix recurrent layers in (SpecPilot digest,
airadar.tv — "Reasons") and condition every draft token on its own root path (JetSpec article,
seventnews.com — "Technical architecture"). The oracle's reading of the recurrent layer is written
out in specverify_oracle.c (a gated linear recurrence per head in place of the attention mixer).
What must hold whatever the layer's internals:
  * every tree node's logits equal those of its root path run as a chain, bit for bit (attention
    over the ancestors only, the recurrent state continued along the path only);
  * the recurrence itself: from a zero state, o = v0 (k0 . q0) for the root and
    o = e^g1 v0 (k0 . q1) + v1 (k1 . q1) for its child (S <- e^g S + k v^T, o = S^T q), and
    g = -log(1 + e^a) for the bf16 gate input a;
  * a commit followed by the next pass agrees with one pass over the longer chain (up to the fp32
    storage of the committed state).
"""
import numpy as np
import torch

import oracle
import synth

from helpers import bits, oracle_cfg

SHAPE = synth.HYBRID_TINY
KINDS = synth.HYBRID_KINDS


def hybrid_model(seed: int, shape=SHAPE, kinds=KINDS):
    w = synth.model_weights(shape, seed)
    layers = []
    for l, kind in enumerate(kinds):
        lw = synth.rec_layer_weights(shape, seed, l) if kind == oracle.RECURRENT else w["layers"][l]
        layers.append({k: bits(v) for k, v in lw.items()})
    return oracle.Model(oracle_cfg(shape), bits(w["embed"]), bits(w["final_norm"]), bits(w["lm_head"]),
                        layers, kinds=kinds)


def caches(shape, kinds, ctx: int, seed: int):
    kc, vc, st = [], [], []
    for l, kind in enumerate(kinds):
        if kind == oracle.RECURRENT:
            kc.append(np.zeros((0, shape.n_kv_heads, shape.head_dim), np.uint16))
            vc.append(np.zeros((0, shape.n_kv_heads, shape.head_dim), np.uint16))
            st.append(synth.rec_state(shape, seed, l)[0].numpy())
        else:
            k, v = synth.kv_context(shape, ctx, seed, l)
            kc.append(bits(k))
            vc.append(bits(v))
            st.append(None)
    return kc, vc, st


def root_path(parent, i):
    p = []
    while i != -1:
        p.append(i)
        i = int(parent[i])
    return p[::-1]


def test_tree_nodes_equal_their_root_path_chains():
    m = hybrid_model(61)
    kc, vc, st = caches(SHAPE, KINDS, 37, 61)
    k = 11
    parent = synth.random_tree(k, 5, 61, "hybrid tree")
    tokens = synth.tree_tokens(parent, SHAPE.vocab, 61, "hybrid tree")
    r = oracle.verify(m, kc, vc, tokens, parent, state=st)
    assert np.isfinite(r.logits).all()
    for i in range(k):
        path = root_path(parent, i)
        rc = oracle.verify(m, kc, vc, tokens[path], oracle.chain(len(path)), state=st)
        assert np.array_equal(rc.logits[-1].view(np.uint32), r.logits[i].view(np.uint32)), f"node {i}"
        for l, kind in enumerate(KINDS):
            assert np.array_equal(rc.k_new[l][-1], r.k_new[l][i]) and np.array_equal(rc.v_new[l][-1], r.v_new[l][i])
            if kind == oracle.RECURRENT:
                assert np.array_equal(rc.g_new[l][-1].view(np.uint32), r.g_new[l][i].view(np.uint32))
    # the acceptance walk over the tree: the deepest root path whose tokens are all greedy
    best = 0
    for i in range(k):
        path = root_path(parent, i)
        if all(tokens[path[t + 1]] == r.arg[path[t]] for t in range(len(path) - 1)):
            best = max(best, len(path) - 1)
    assert r.accepted_len == best


def test_recurrent_layer_closed_form_from_zero_state():
    # hidden = nh * d, W_o = identity and W_down = 0, so the layer adds exactly bf16(o) to x
    nh, d = 2, 64
    shape = synth.Shape(n_layers=1, hidden=nh * d, n_q_heads=nh, n_kv_heads=1, head_dim=d, ffn=64,
                        vocab=64)
    cfg = oracle_cfg(shape)
    lw = synth.rec_layer_weights(shape, 5, 0)
    lw["w_o"] = torch.eye(nh * d, dtype=torch.bfloat16)
    lw["w_down"] = torch.zeros_like(lw["w_down"])
    lw = {k: bits(v) for k, v in lw.items()}
    x = bits(synth.randn_bf16((2, shape.hidden), 1.0, "cpu", 5, "x"))
    S0 = np.zeros((nh, d, d), np.float32)
    x_out, kk, vv, g = oracle.rec_layer_forward(cfg, lw, S0, oracle.chain(2), x)

    u = oracle.rmsnorm(x, lw["attn_norm"], shape.rms_eps)
    y = oracle.linear(u, lw["w_qkv"])
    q = oracle.from_bf16(oracle.to_bf16(y[:, :nh * d])).astype(np.float64).reshape(2, nh, d)
    k = oracle.from_bf16(oracle.to_bf16(y[:, nh * d:2 * nh * d])).astype(np.float64).reshape(2, nh, d)
    v = oracle.from_bf16(oracle.to_bf16(y[:, 2 * nh * d:3 * nh * d])).astype(np.float64).reshape(2, nh, d)
    a = oracle.from_bf16(oracle.to_bf16(y[:, 3 * nh * d:])).astype(np.float64)
    assert np.array_equal(oracle.from_bf16(kk).astype(np.float64), k)
    assert np.array_equal(oracle.from_bf16(vv).astype(np.float64), v)
    np.testing.assert_allclose(g, -np.logaddexp(0.0, a), rtol=2e-7, atol=1e-30)
    o = np.empty((2, nh, d))
    for h in range(nh):
        o[0, h] = v[0, h] * (k[0, h] @ q[0, h])
        o[1, h] = np.exp(float(g[1, h])) * v[0, h] * (k[0, h] @ q[1, h]) + v[1, h] * (k[1, h] @ q[1, h])
    o16 = oracle.to_bf16(o.reshape(2, -1).astype(np.float32))
    want = oracle.to_bf16(oracle.from_bf16(x) + oracle.from_bf16(o16))
    assert np.array_equal(x_out, want)
    # the same with S0 = the transposed state would give k (v . q): different outputs
    assert not np.allclose(oracle.from_bf16(o16).reshape(2, nh, d)[0], (k[0] * (v[0] * q[0]).sum(-1, keepdims=True)), atol=1e-3)


def test_commit_then_next_pass_matches_the_longer_chain():
    m = hybrid_model(62)
    kc, vc, st = caches(SHAPE, KINDS, 21, 62)
    toks = synth.uniform_tokens(12, SHAPE.vocab, 62, "chain")
    first, second = toks[:7], toks[6:]          # the second pass starts at the first's last token
    r1 = oracle.verify(m, kc, vc, first, state=st)
    # commit all of the first block but its last token (a = 5: nodes 0..5)
    r1.accepted_len = 5
    r1.path = np.array([0, 1, 2, 3, 4, 5, -1], np.int32)
    kc2, vc2 = oracle.commit(kc, vc, r1)
    st2 = oracle.commit_rec(m, st, r1)
    r2 = oracle.verify(m, kc2, vc2, second, state=st2)
    whole = oracle.verify(m, kc, vc, toks, state=st)
    np.testing.assert_allclose(r2.logits, whole.logits[6:], rtol=0, atol=2e-4)
    for l, kind in enumerate(KINDS):
        if kind == oracle.ATTENTION:
            assert np.array_equal(kc2[l][21:], whole.k_new[l][:6])
    # a failed request (accepted_len -1) keeps its state
    r1.accepted_len = -1
    st3 = oracle.commit_rec(m, st, r1)
    for l, kind in enumerate(KINDS):
        if kind == oracle.RECURRENT:
            assert np.array_equal(st3[l], st[l])
