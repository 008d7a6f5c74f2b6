"""Whole-model pins of the CPU oracle on the tiny decoder.

* An independent float64 PyTorch decoder (same bf16 storage points, torch's own SDPA, SiLU and
  complex-free rotate-half) agrees with the oracle's logits within an accumulation bound.
* Lossless greedy verification must emit exactly what one-token-at-a-time greedy decoding emits
  [SpecPilot digest, airadar.tv — "Risks"]; in the oracle, whose rows never depend on the batch,
  a block pass, a chain-tree pass and AR decoding are bit-identical.
* Tree tokens are conditioned on their own path [JetSpec article, seventnews.com — "Technical
  architecture"]: brute force over every root path of small trees reproduces the tree pass.
* Committing the accepted path leaves the same cache as decoding those tokens one at a time.
"""
import numpy as np
import pytest
import torch

import oracle
import ref64
import synth


def bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def oracle_model(shape, seed):
    w = synth.model_weights(shape, seed)
    cfg = oracle.Cfg(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads,
                     shape.head_dim, shape.ffn, shape.vocab, shape.rms_eps, shape.rope_theta)
    layers = [{k: bits(v) for k, v in lw.items()} for lw in w["layers"]]
    return oracle.Model(cfg, bits(w["embed"]), bits(w["final_norm"]), bits(w["lm_head"]), layers), w


@pytest.fixture(scope="module")
def tiny():
    m, w = oracle_model(synth.TINY, 11)
    prompt = synth.uniform_tokens(128, synth.TINY.vocab, 11, "prompt")
    kc, vc, last = oracle.prefill(m, prompt)
    g1 = int(np.argmax(last))
    return m, w, prompt, kc, vc, g1


# ------------------------------------------------------------------------------------------
# independent float64 decoder (tests/ref64.py)
# ------------------------------------------------------------------------------------------

def ref_decoder(w, shape, tokens, parent, k_ctx, v_ctx):
    return ref64.decoder(w, shape, tokens, parent, k_ctx, v_ctx)[0]


@pytest.mark.parametrize("kind", ["chain", "tree"])
def test_oracle_matches_independent_float64_decoder(tiny, kind):
    m, w, prompt, kc, vc, g1 = tiny
    if kind == "chain":
        parent = oracle.chain(8)
        tokens = np.concatenate([[g1], synth.uniform_tokens(7, 1024, 5, "d")]).astype(np.int32)
    else:
        parent = synth.random_tree(16, 5, 5, "t")
        tokens = synth.tree_tokens(parent, 1024, 5, "t")
    r = oracle.verify(m, kc, vc, tokens, parent)
    ref = ref_decoder(w, synth.TINY, tokens, parent, kc, vc)
    err = np.abs(r.logits - ref)
    # logits here have magnitude ~0.3-1.5; independent rounding of the two float paths moves
    # bf16 intermediates by an ulp now and then, which shifts logits by ~1e-3 at most
    assert err.max() < 1e-2, err.max()
    assert np.mean(err) < 1e-3
    assert np.abs(ref).max() > 0.5


def test_float64_decoder_distinguishes_a_wrong_model(tiny):
    """The comparison above has teeth: a slightly different model is far outside its bound."""
    m, w, prompt, kc, vc, g1 = tiny
    tokens = np.array([g1, 1, 2, 3], np.int32)
    r = oracle.verify(m, kc, vc, tokens)
    w2 = {**w, "layers": [dict(lw) for lw in w["layers"]]}
    w2["layers"][1]["w_o"] = w["layers"][1]["w_o"].flip(0)
    ref = ref_decoder(w2, synth.TINY, tokens, oracle.chain(4), kc, vc)
    assert np.abs(r.logits - ref).max() > 5e-2


# ------------------------------------------------------------------------------------------
# AR == block == chain tree, bit-exact
# ------------------------------------------------------------------------------------------

def test_block_equals_ar_greedy_bit_exact(tiny):
    m, w, prompt, kc, vc, g1 = tiny
    toks, lgs, kc_ar, vc_ar = oracle.ar_greedy(m, kc, vc, g1, 8)
    block = np.concatenate([[g1], toks[:7]]).astype(np.int32)
    r = oracle.verify(m, kc, vc, block)
    assert np.array_equal(r.logits, lgs)
    assert np.array_equal(r.arg, toks)
    assert r.accepted_len == 7 and r.bonus == toks[7]
    assert list(r.path) == list(range(8))
    # committing the accepted path gives the cache AR decoding built, bit for bit
    kc2, vc2 = oracle.commit(kc, vc, r)
    for l in range(m.cfg.n_layers):
        assert np.array_equal(kc2[l], kc_ar[l]) and np.array_equal(vc2[l], vc_ar[l])


def test_chain_given_as_tree_with_extra_branches_bit_exact(tiny):
    m, w, prompt, kc, vc, g1 = tiny
    toks, lgs, _, _ = oracle.ar_greedy(m, kc, vc, g1, 7)
    rng = np.random.default_rng(0)
    parent, tokens, chain_ids = [-1], [g1], [0]
    for depth in range(1, 7):
        level = [len(parent) + j for j in range(3)]
        where = int(rng.integers(0, 3))
        for j, node in enumerate(level):
            if j == where:
                parent.append(chain_ids[-1])
                tokens.append(int(toks[depth - 1]))
                chain_ids.append(node)
            else:
                parent.append(chain_ids[-1] if rng.random() < 0.5 else level[0] - 1)
                t = int(rng.integers(0, 1024))
                tokens.append(t if t != toks[depth - 1] else (t + 1) % 1024)
    parent = np.array(parent, np.int32)
    r = oracle.verify(m, kc, vc, np.array(tokens, np.int32), parent)
    assert np.array_equal(r.logits[chain_ids], lgs)
    assert r.accepted_len == 6
    assert list(r.path[:7]) == chain_ids and r.bonus == int(toks[6])


def test_prefill_in_two_pieces_bit_exact(tiny):
    m, w, prompt, kc, vc, g1 = tiny
    ka, va, _ = oracle.prefill(m, prompt[:50])
    kb, vb, last = oracle.prefill(m, prompt[50:], ka, va)
    assert int(np.argmax(last)) == g1
    for l in range(m.cfg.n_layers):
        assert np.array_equal(kb[l], kc[l]) and np.array_equal(vb[l], vc[l])


# ------------------------------------------------------------------------------------------
# brute force over every root path of small trees
# ------------------------------------------------------------------------------------------

def forced_passes(m, kc, vc, seq):
    """Feed ``seq`` one token per pass; return each pass's logits."""
    out = []
    kc, vc = list(kc), list(vc)
    for t in seq:
        r = oracle.verify(m, kc, vc, np.array([t], np.int32), np.array([-1], np.int32))
        kc = [np.concatenate([kc[l], r.k_new[l]]) for l in range(len(kc))]
        vc = [np.concatenate([vc[l], r.v_new[l]]) for l in range(len(vc))]
        out.append(r.logits[0])
    return np.stack(out), kc, vc


@pytest.mark.parametrize("seed", range(6))
def test_tree_verify_equals_brute_force_over_paths(tiny, seed):
    m, w, prompt, kc, vc, g1 = tiny
    rng = np.random.default_rng(100 + seed)
    k = int(rng.integers(2, 13))
    parent = synth.random_tree(k, int(rng.integers(1, k)) if k > 1 else 1, seed, "bf")
    tokens = np.zeros(k, np.int32)
    tokens[0] = g1
    paths = {}
    for i in range(k):
        p = [] if i == 0 else paths[int(parent[i])]
        paths[i] = p + [i]
    greedy_after = {}
    for i in range(k):                      # BFS ids: a parent is settled before its children
        if i > 0:
            par = int(parent[i])
            sib = {int(tokens[j]) for j in range(1, i) if parent[j] == par}
            want = greedy_after[par]
            if rng.random() < 0.65 and want not in sib:
                tokens[i] = want
            else:
                t = int(rng.integers(0, 1024))
                while t in sib or t == want:
                    t = (t + 1) % 1024
                tokens[i] = t
        lg, _, _ = forced_passes(m, kc, vc, tokens[paths[i]])
        greedy_after[i] = int(np.argmax(lg[-1]))
    r = oracle.verify(m, kc, vc, tokens, parent)
    for i in range(k):                      # every node's logits == its own path's AR pass
        lg, _, _ = forced_passes(m, kc, vc, tokens[paths[i]])
        assert np.array_equal(r.logits[i], lg[-1])
    best = max(range(k), key=lambda i: (all(tokens[paths[i][t + 1]] == greedy_after[paths[i][t]]
                                            for t in range(len(paths[i]) - 1)) * (len(paths[i]) * 1000) - i))
    assert r.accepted_len == len(paths[best]) - 1
    assert list(r.path[: r.accepted_len + 1]) == paths[best]
    assert r.bonus == greedy_after[best]
    kc2, vc2 = oracle.commit(kc, vc, r)
    _, kc_ar, vc_ar = forced_passes(m, kc, vc, tokens[paths[best]])
    for l in range(m.cfg.n_layers):
        assert np.array_equal(kc2[l], kc_ar[l]) and np.array_equal(vc2[l], vc_ar[l])
