"""The persistent path of spec_verify (one kernel per group of up to 16 layers for batch * k <= 16
rows) against the CPU oracle, and against the per-step path, on the tiny decoder: blocks, a tree,
a batch of two requests with different contexts and shuffled pages, a failed request, and a
model deeper than one launch (more than 16 layers, so the layers span launches).

Same parity rules as the per-step path (logits within 2e-2 + 1e-2|x|; acceptance exact up to
logged near-ties [SpecPilot digest, airadar.tv — "Risks"]). Only the order of the split-K sums
and of the norm's sum of squares differs between the two paths, so their logits also agree
within that tolerance."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tree_verification_skinny_amd as tv
from tree_verification_skinny_amd import kvlayout

from helpers import (bits, check_accept, check_logits, device_weights, make_kv, oracle_model_from,
                     run_verify, tiny_case, upload_context)
from test_gpu_parity import planted_tree

pytestmark = pytest.mark.gpu
DEV = "cuda"


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tv.lib()


def _both(weights, kv_fn, tokens, parent, ctxs, want_hidden=False):
    outs = {}
    for path in ("persistent", "steps"):
        print(f"  path {path}", flush=True)
        outs[path] = run_verify(weights, kv_fn(), tokens, parent, ctxs, want_hidden=want_hidden, path=path)
    return outs


def test_tiny_block_persistent_matches_oracle_and_steps():
    near = 0
    for seed in range(24):
        print(f"tiny block seed {seed}", flush=True)
        w, m, kc, vc, tokens, G = tiny_case(seed)
        k = tokens.size
        r = oracle.verify(m, kc, vc, tokens)
        weights = device_weights(synth.TINY, w, DEV)

        def kv_fn():
            kv = make_kv(synth.TINY, [128], k, seed, DEV)
            upload_context(kv, 0, kc, vc)
            return kv
        kv = kv_fn()
        out = run_verify(weights, kv, tokens[None], None, [128], path="persistent")
        check_logits(out.logits[0], r.logits, f"seed {seed} logits")
        near += check_accept(r, tokens, None, out.greedy[0], int(out.accepted_len[0]),
                             int(out.bonus[0]), out.path[0])
        for l in range(2):
            kg, vg = kvlayout.read_rows(kv, l, 0, torch.arange(128, 128 + k))
            check_logits(kg.float().cpu().numpy(), oracle.from_bf16(r.k_new[l]), f"k_new l{l}")
            check_logits(vg.float().cpu().numpy(), oracle.from_bf16(r.v_new[l]), f"v_new l{l}")
        o2 = run_verify(weights, kv_fn(), tokens[None], None, [128], path="steps")
        check_logits(out.logits[0], o2.logits[0], f"seed {seed} persistent vs steps")
    assert near <= 6


@pytest.mark.parametrize("k", [13, 16])
def test_tiny_tree_persistent(k):
    for seed in range(3):
        print(f"tiny tree k={k} seed {seed}", flush=True)
        w = synth.model_weights(synth.TINY, 900 + seed)
        m = oracle_model_from(synth.TINY, w)
        ctx = 40 + 53 * seed
        kvs = [synth.kv_context(synth.TINY, ctx, seed, l) for l in range(2)]
        kc = [np.ascontiguousarray(bits(x)) for x, _ in kvs]
        vc = [np.ascontiguousarray(bits(y)) for _, y in kvs]
        tokens, parent = planted_tree(m, kc, vc, k, seed)
        r = oracle.verify(m, kc, vc, tokens, parent)
        weights = device_weights(synth.TINY, w, DEV)
        kv = make_kv(synth.TINY, [ctx], k, seed, DEV)
        upload_context(kv, 0, kc, vc)
        out = run_verify(weights, kv, tokens[None], parent[None], [ctx], path="persistent")
        check_logits(out.logits[0], r.logits)
        check_accept(r, tokens, parent, out.greedy[0], int(out.accepted_len[0]), int(out.bonus[0]),
                     out.path[0])


def test_tiny_batch_of_two_and_a_failed_request():
    """B = 2 x K = 8 (16 rows) with different contexts over shuffled pages, then B = 4 x 4 with a
    request whose token is out of range: it alone fails, the others meet the oracle."""
    w = synth.model_weights(synth.TINY, 77)
    m = oracle_model_from(synth.TINY, w)
    weights = device_weights(synth.TINY, w, DEV)
    for ctxs, k, bad in (([37, 301], 8, None), ([0, 15, 130, 64], 4, 2)):
        print(f"batch ctxs={ctxs} k={k}", flush=True)
        kv = make_kv(synth.TINY, ctxs, k, 77, DEV, extra_pages=1)
        cases, toks = [], []
        for b, ctx in enumerate(ctxs):
            kvs = [synth.kv_context(synth.TINY, ctx, 77, l, request=b) for l in range(2)]
            kc = [bits(x) for x, _ in kvs]
            vc = [bits(y) for _, y in kvs]
            upload_context(kv, b, kc, vc)
            tok = synth.uniform_tokens(k, 1024, 77, b, k)
            if ctx > 0:
                cont, _, _, _ = oracle.ar_greedy(m, kc, vc, int(tok[0]), k - 1)
                tok[1:] = cont
            cases.append((kc, vc))
            toks.append(tok)
        tokens = np.stack(toks).astype(np.int32)
        if bad is not None:
            tokens[bad, 1] = 5000
        out = run_verify(weights, kv, tokens, None, ctxs, path="persistent")
        for b in range(len(ctxs)):
            if b == bad:
                assert out.accepted_len[b] == -1 and out.bonus[b] == -1
                continue
            r = oracle.verify(m, cases[b][0], cases[b][1], tokens[b])
            check_logits(out.logits[b], r.logits, f"request {b}")
            check_accept(r, tokens[b], None, out.greedy[b], int(out.accepted_len[b]),
                         int(out.bonus[b]), out.path[b])


def test_deep_tiny_model_spans_launches():
    """20 layers of the tiny shape: the persistent kernel runs layers 0-15 and 16-19 as two
    launches; residual stream per layer and logits against the oracle."""
    shape = synth.TINY.with_layers(20)
    w = synth.model_weights(shape, 5)
    m = oracle_model_from(shape, w)
    ctx, k = 50, 8
    kvs = [synth.kv_context(shape, ctx, 5, l) for l in range(20)]
    kc = [np.ascontiguousarray(bits(x)) for x, _ in kvs]
    vc = [np.ascontiguousarray(bits(y)) for _, y in kvs]
    tokens = synth.uniform_tokens(k, 1024, 5, "deep")
    r = oracle.verify(m, kc, vc, tokens, keep_hidden=True)
    weights = device_weights(shape, w, DEV)
    kv = make_kv(shape, [ctx], k, 5, DEV)
    upload_context(kv, 0, kc, vc)
    out = run_verify(weights, kv, tokens[None], None, [ctx], want_hidden=True, path="persistent")
    for l in (1, 15, 16, 17, 20):
        check_logits(out.hidden[l].float().cpu().numpy(), oracle.from_bf16(r.hidden[l]), f"hidden {l}")
    check_logits(out.logits[0], r.logits)
    check_accept(r, tokens, None, out.greedy[0], int(out.accepted_len[0]), int(out.bonus[0]), out.path[0])


def test_persistent_path_refuses_what_it_cannot_take():
    """More than 16 rows: SPEC_EUNSUPPORTED when the persistent path is forced; auto runs the
    per-step path."""
    w = synth.model_weights(synth.TINY, 3)
    weights = device_weights(synth.TINY, w, DEV)
    kv = make_kv(synth.TINY, [10, 10, 10], 8, 3, DEV)
    tokens = np.stack([synth.uniform_tokens(8, 1024, 3, b) for b in range(3)]).astype(np.int32)
    with pytest.raises(tv.SpecError) as e:
        run_verify(weights, kv, tokens, None, [10, 10, 10], path="persistent")
    assert e.value.code == tv.SPEC_EUNSUPPORTED
    out = run_verify(weights, kv, tokens, None, [10, 10, 10])
    assert (out.accepted_len >= 0).all()
