"""A hybrid target (attention and recurrent layers alternating, the tiny shape with 4 layers)
verified end to end through spec_verify and committed through spec_commit_kv, against the
oracle's hybrid model (tests/test_oracle_hybrid.py pins it).

Tree verification for targets that mix recurrent layers in is named by the SpecPilot digest
(airadar.tv — "Reasons"); every draft token is conditioned on its own root path (JetSpec
article, seventnews.com — "Technical architecture"), for the recurrent state as for attention.
Same parity rules as the dense tiny model: logits within 2e-2 + 1e-2|x|, acceptance exact up
to logged near-ties. After the commit: attention layers' rows are the pass's own rows moved
bit for bit; each recurrent state equals the oracle's commit of the pass's own keys, values and
gates along the accepted path (fp32 arithmetic against float64: within 1e-5 relative to the
state's scale); a second pass over the committed cache and states meets the oracle's second
pass over its own committed ones."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tree_verification_skinny_amd as tv
from tree_verification_skinny_amd import kvlayout

from helpers import bits, check_accept, check_logits, make_kv, oracle_cfg, run_verify, upload_context

pytestmark = pytest.mark.gpu
DEV = "cuda"
SHAPE = synth.HYBRID_TINY
KINDS = synth.HYBRID_KINDS


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tv.lib()


class Case:
    pass


def build(seed: int, ctxs, k: int):
    """Weights (oracle and device), per-request oracle caches and states, the device cache."""
    c = Case()
    w = synth.model_weights(SHAPE, seed)
    layers = [synth.rec_layer_weights(SHAPE, seed, l, pad16=True) if kd == oracle.RECURRENT else w["layers"][l]
              for l, kd in enumerate(KINDS)]
    c.m = oracle.Model(oracle_cfg(SHAPE), bits(w["embed"]), bits(w["final_norm"]), bits(w["lm_head"]),
                       [{n: bits(t) for n, t in lw.items()} for lw in layers], kinds=KINDS)
    c.weights = tv.Weights(tv.ModelCfg.of(SHAPE), w["embed"].to(DEV), w["final_norm"].to(DEV),
                           w["lm_head"].to(DEV), [{n: t.to(DEV) for n, t in lw.items()} for lw in layers],
                           kinds=KINDS)
    B = len(ctxs)
    c.kv = make_kv(SHAPE, ctxs, k, seed, DEV, extra_pages=1)
    c.kc, c.vc, c.st = [], [], []
    for b, ctx in enumerate(ctxs):
        kc, vc = [], []
        for l, kd in enumerate(KINDS):
            if kd == oracle.RECURRENT:
                kc.append(np.zeros((0, SHAPE.n_kv_heads, SHAPE.head_dim), np.uint16))
                vc.append(np.zeros((0, SHAPE.n_kv_heads, SHAPE.head_dim), np.uint16))
            else:
                x, y = synth.kv_context(SHAPE, ctx, seed, l, request=b)
                kc.append(bits(x))
                vc.append(bits(y))
        upload_context(c.kv, b, kc, vc)
        c.kc.append(kc)
        c.vc.append(vc)
    states = []
    for l, kd in enumerate(KINDS):
        if kd == oracle.RECURRENT:
            S = synth.rec_state(SHAPE, seed, l, requests=B)             # [B][nh][d][d], S[r][c]
            states.append(S)
        else:
            states.append(None)
    c.st = [[None if S is None else S[b].numpy() for S in states] for b in range(B)]
    # the device keeps each head's S transposed
    dev_states = [None if S is None else S.transpose(-1, -2).contiguous().to(DEV) for S in states]
    c.kv.attach_rec(tv.ModelCfg.of(SHAPE), dev_states, B, k)
    c.ctxs = list(ctxs)
    return c


def greedy_block(c, b, k, seed, replace_at=None):
    """A block for request b whose tokens follow the oracle's own greedy decoding, with one token
    replaced at replace_at (so acceptance stops there)."""
    first = int(synth.uniform_tokens(1, SHAPE.vocab, seed, "first", b)[0])
    cont, _, _, _, _ = oracle.ar_greedy_hybrid(c.m, c.kc[b], c.vc[b], c.st[b], first, k - 1)
    tok = np.concatenate([[first], cont]).astype(np.int32)
    if replace_at is not None:
        tok[replace_at] = synth.other_token(int(tok[replace_at]), SHAPE.vocab, seed, "rep", b)
    return tok


def test_hybrid_block_batch_matches_oracle():
    k = 8
    c = build(71, [37, 90], k)
    tokens = np.stack([greedy_block(c, 0, k, 71), greedy_block(c, 1, k, 71, replace_at=4)])
    out = run_verify(c.weights, c.kv, tokens, None, c.ctxs)
    for b in range(2):
        r = oracle.verify(c.m, c.kc[b], c.vc[b], tokens[b], state=c.st[b])
        check_logits(out.logits[b], r.logits, f"request {b} logits")
        check_accept(r, tokens[b], None, out.greedy[b], int(out.accepted_len[b]), int(out.bonus[b]), out.path[b])
    assert int(out.accepted_len[1]) <= 3


def test_hybrid_tree_matches_oracle():
    k = 13
    c = build(72, [55], k)
    parent = synth.random_tree(k, 6, 72, "hybrid gpu tree")
    tokens = synth.tree_tokens(parent, SHAPE.vocab, 72, "hybrid gpu tree")
    # make the first two levels follow the target's greedy choice where the tree allows
    r0 = oracle.verify(c.m, c.kc[0], c.vc[0], tokens[:1], oracle.chain(1), state=c.st[0])
    kids = [i for i in range(1, k) if parent[i] == 0]
    if kids:
        tokens[kids[0]] = int(r0.arg[0])
    out = run_verify(c.weights, c.kv, tokens[None], parent[None], c.ctxs)
    r = oracle.verify(c.m, c.kc[0], c.vc[0], tokens, parent, state=c.st[0])
    check_logits(out.logits[0], r.logits, "tree logits")
    check_accept(r, tokens, parent, out.greedy[0], int(out.accepted_len[0]), int(out.bonus[0]), out.path[0])


def test_hybrid_commit_then_second_pass():
    """Commit of KV rows and recurrent states together, then the next block over them."""
    k = 8
    c = build(73, [29, 64], k)
    tokens = np.stack([greedy_block(c, 0, k, 73), greedy_block(c, 1, k, 73, replace_at=3)])
    out = run_verify(c.weights, c.kv, tokens, None, c.ctxs)
    rows_before = [[kvlayout.read_rows(c.kv, l, b, torch.arange(c.ctxs[b], c.ctxs[b] + k))
                    for l in range(SHAPE.n_layers)] for b in range(2)]
    tv.spec_commit_kv(c.weights.cfg, c.kv, out.acc_t, out.path_t, out.ctx, 2, k)
    torch.cuda.synchronize()
    ctx_after = out.ctx.cpu().numpy()
    kc2, vc2, st2, nxt = [], [], [], []
    for b in range(2):
        r = oracle.verify(c.m, c.kc[b], c.vc[b], tokens[b], state=c.st[b])
        near = check_accept(r, tokens[b], None, out.greedy[b], int(out.accepted_len[b]), int(out.bonus[b]),
                            out.path[b])
        print(f"request {b}: accepted {int(out.accepted_len[b])} (oracle {r.accepted_len}), near-tie {near}")
        # the oracle commits along the GPU's accepted path (equal unless a logged near-tie flipped)
        a = int(out.accepted_len[b])
        r.accepted_len, r.path, r.bonus = a, np.asarray(out.path[b], np.int32), int(out.bonus[b])
        assert ctx_after[b] == c.ctxs[b] + a + 1
        path = out.path[b][:a + 1]
        for l, kd in enumerate(KINDS):
            if kd != oracle.ATTENTION:
                continue
            kg, vg = kvlayout.read_rows(c.kv, l, b, torch.arange(c.ctxs[b], c.ctxs[b] + a + 1))
            assert torch.equal(kg, rows_before[b][l][0][path]) and torch.equal(vg, rows_before[b][l][1][path])
        st_o = oracle.commit_rec(c.m, c.st[b], r)
        for l, kd in enumerate(KINDS):
            if kd != oracle.RECURRENT:
                continue
            # the commit applies the pass's own keys, values and gates (as the KV rows above are
            # the pass's own rows): the oracle's commit of those, float64 against fp32
            kk = bits(c.kv.rec_k[l].view(2, k, SHAPE.n_q_heads, SHAPE.head_dim)[b])
            vv = bits(c.kv.rec_v[l].view(2, k, SHAPE.n_q_heads, SHAPE.head_dim)[b])
            gg = c.kv.rec_g[l].view(2, k, SHAPE.n_q_heads)[b].cpu().numpy()
            want = oracle.rec_commit(c.st[b][l][None], kk[None], vv[None], gg[None],
                                     np.array([a], np.int32), np.asarray(out.path[b], np.int32)[None])[0]
            S_gpu = c.kv.rec_states[l][b].transpose(-1, -2).cpu().numpy()
            scale = float(np.abs(want).max())
            err = float(np.abs(S_gpu - want).max())
            assert err <= 1e-5 * scale, f"request {b} layer {l} state: max err {err:.3e} (scale {scale:.3e})"
        k2, v2 = oracle.commit(c.kc[b], c.vc[b], r)
        kc2.append(k2)
        vc2.append(v2)
        st2.append(st_o)
        nxt.append(int(r.bonus))
    # the next block over the committed cache and states (oracle: its own committed ones)
    tokens2 = np.stack([np.concatenate([[nxt[b]], synth.uniform_tokens(k - 1, SHAPE.vocab, 73, "second", b)])
                        for b in range(2)]).astype(np.int32)
    out2 = run_verify(c.weights, c.kv, tokens2, None, list(ctx_after))
    for b in range(2):
        r2 = oracle.verify(c.m, kc2[b], vc2[b], tokens2[b], state=st2[b])
        check_logits(out2.logits[b], r2.logits, f"second pass request {b}")
        check_accept(r2, tokens2[b], None, out2.greedy[b], int(out2.accepted_len[b]), int(out2.bonus[b]),
                     out2.path[b])


def test_hybrid_refusals():
    """Recurrent layers without states, or forced onto the persistent plan, are refused."""
    k = 4
    c = build(74, [10], k)
    tokens = synth.uniform_tokens(k, SHAPE.vocab, 74, "ref")[None].astype(np.int32)
    with pytest.raises(tv.SpecError) as e:
        run_verify(c.weights, c.kv, tokens, None, c.ctxs, path="persistent")
    assert e.value.code == tv.SPEC_EUNSUPPORTED
    bare = make_kv(SHAPE, [10], k, 74, DEV)
    with pytest.raises(tv.SpecError) as e:
        run_verify(c.weights, bare, tokens, None, [10])
    assert e.value.code == tv.SPEC_EINVAL
