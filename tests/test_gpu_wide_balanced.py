"""The gate/up projection balanced over the compute units: passes of 17..64 rows whose gate/up has
a few more 128-column groups than there are compute units (the wide kernel, one workgroup per
unit), and passes of 1..16 rows with a few more 32-column groups than twice the units (the skinny
kernel, two workgroups per unit). Each workgroup takes one group over all of K and a K part of one
leftover gate/up pair; the last of a pair's parts to arrive adds them in index order and applies
SwiGLU. Whole verify passes at two such shapes against the CPU oracle
(logits at the fixed tolerance, acceptance exact up to logged near-ties) on a workspace poisoned
with 0xFF bytes (the pass clears the arrival counters itself), a second pass bit for bit equal to
the first (the counters are left zero), and the W12 pass bit for bit equal to the bf16 one (the
same partition and order of sums)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tree_verification_skinny_amd as tv

from helpers import (bits, check_accept, check_logits, device_weights, make_kv, oracle_model_from, run_verify,
                     upload_context)
from test_gpu_parity import planted_tree

pytestmark = pytest.mark.gpu
DEV = "cuda"


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tv.lib()


# Wide kernel: ffn 16896, 264 groups of four pairs, the 32 leftover pairs in 8 parts of one K step
# each (three of a workgroup's four waves have no step of its part); ffn 17408: 272 groups, 64
# leftover pairs in 4 parts of two steps. 64, 48 and 32 rows: four, four (the last row block partly
# empty) and two row blocks per launch.
# Skinny kernel (16 rows or fewer): ffn 17408 at hidden 512, 544 groups of two pairs on 512
# workgroups, the 64 leftover pairs in 8 parts of two K steps; ffn 16896 at hidden 1024: 528
# groups, the 32 leftover pairs in 16 parts of two steps; ffn 18432 at hidden 256: 576 groups, 128
# leftover pairs in 4 parts of two steps; ffn 24576: 768 groups, 512 leftover pairs each in one
# part (each pair finished by the one workgroup that computes it).
@pytest.mark.parametrize("ffn,hidden,B,k,kind", [(16896, 256, 1, 64, "tree"), (17408, 256, 2, 24, "chain"),
                                                 (17408, 256, 2, 16, "tree"), (17408, 512, 1, 16, "tree"),
                                                 (17408, 512, 1, 5, "chain"), (16896, 1024, 1, 16, "chain"),
                                                 (18432, 256, 1, 16, "tree"), (24576, 256, 1, 7, "chain")])
def test_balanced_gate_up_pass(ffn, hidden, B, k, kind):
    shape = synth.Shape(n_layers=2, hidden=hidden, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=ffn, vocab=1024)
    seed = 1300 + ffn % 97 + 7 * B + k + hidden // 256 - 1
    ctxs = [300, 900][:B]
    w = synth.model_weights(shape, seed)
    m = oracle_model_from(shape, w)
    weights = device_weights(shape, w, DEV)
    kv = make_kv(shape, ctxs, k, seed, DEV)
    toks, pars, cases = [], [], []
    for b, ctx in enumerate(ctxs):
        kvs = [synth.kv_context(shape, ctx, seed, l, request=b) for l in range(2)]
        kc = [np.ascontiguousarray(bits(x)) for x, _ in kvs]
        vc = [np.ascontiguousarray(bits(y)) for _, y in kvs]
        upload_context(kv, b, kc, vc)
        if kind == "tree":
            tokens, parent = planted_tree(m, kc, vc, k, seed + b)
        else:
            parent = oracle.chain(k)
            tokens = synth.uniform_tokens(k, shape.vocab, seed, "bal", b)
        toks.append(tokens)
        pars.append(parent)
        cases.append((kc, vc))
    tokens = np.stack(toks).astype(np.int32)
    parents = np.stack(pars).astype(np.int32)
    out = run_verify(weights, kv, tokens, parents, ctxs, ws_fill=0xFF)
    near = 0
    for b in range(B):
        kc, vc = cases[b]
        r = oracle.verify(m, kc, vc, tokens[b], parents[b])
        assert np.isfinite(out.logits[b]).all(), f"request {b}"
        check_logits(out.logits[b], r.logits, f"ffn {ffn} request {b}")
        near += check_accept(r, tokens[b], parents[b], out.greedy[b], int(out.accepted_len[b]),
                             int(out.bonus[b]), out.path[b])
    assert near <= 1

    again = run_verify(weights, kv, tokens, parents, ctxs)
    assert np.array_equal(out.logits.view(np.int32), again.logits.view(np.int32))

    dev = {nm: w[nm].to(DEV) for nm in ("embed", "final_norm", "lm_head")}
    layers = [{nm: v.to(DEV) for nm, v in lw.items()} for lw in w["layers"]]
    w12 = tv.Weights(tv.ModelCfg.of(shape), dev["embed"], dev["final_norm"], dev["lm_head"], layers, w12=True)
    o12 = run_verify(w12, kv, tokens, parents, ctxs, ws_fill=0xFF)
    assert np.array_equal(out.logits.view(np.int32), o12.logits.view(np.int32))
    assert np.array_equal(out.path, o12.path) and np.array_equal(out.accepted_len, o12.accepted_len)
