"""Prompt prefill on the GPU (spec_prefill, through the C ABI) against the CPU oracle's prefill:
the prompt's K/V rows, the last position's logits and greedy token, the advanced context, and a
verify step over the GPU-prefilled cache, i.e. the tiny workload end to end on the GPU."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tree_verification_skinny_amd as tv
from tree_verification_skinny_amd import kvlayout

from helpers import (bits, check_accept, check_logits, device_weights, make_kv, oracle_model_from,
                     run_verify, upload_context)

pytestmark = pytest.mark.gpu
DEV = "cuda"
NEAR_TIE = 1e-2


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tv.lib()


def gpu_prefill(weights, kv, prompts, ctx0, want_logits=True):
    B, p = prompts.shape
    ws = tv.workspace(tv.spec_prefill_workspace_bytes(weights.cfg, B, kv.max_pages, want_logits), DEV)
    ctx = torch.tensor(ctx0, dtype=torch.int32, device=DEV)
    nt = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    lg = torch.full((B, weights.cfg.vocab), float("nan"), device=DEV) if want_logits else None
    tv.spec_prefill(weights, kv, torch.from_numpy(np.ascontiguousarray(prompts, np.int32)).to(DEV),
                    ctx, nt, ws, last_logits=lg)
    torch.cuda.synchronize()
    return ctx.cpu().numpy(), nt.cpu().numpy(), None if lg is None else lg.cpu().numpy()


def check_rows(kv, b, kc, vc, lo, hi, what):
    for l in range(len(kc)):
        kg, vg = kvlayout.read_rows(kv, l, b, torch.arange(lo, hi))
        check_logits(kg.float().cpu().numpy(), oracle.from_bf16(kc[l][lo:hi]), f"{what} k l{l}")
        check_logits(vg.float().cpu().numpy(), oracle.from_bf16(vc[l][lo:hi]), f"{what} v l{l}")


def greedy_ok(gpu_tok, last):
    arg, margin = oracle.argmax(last[None])
    return int(gpu_tok) == int(arg[0]) or float(margin[0]) < NEAR_TIE


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_prefill_then_verify_tiny_end_to_end(seed):
    """The tiny workload with the prompt prefilled on the GPU instead of uploaded: a 128-token
    prompt (two chunks), then a block of 8 drafted from the oracle's greedy continuation."""
    shape = synth.TINY
    w = synth.model_weights(shape, seed)
    m = oracle_model_from(shape, w)
    prompt = synth.uniform_tokens(128, shape.vocab, seed, "prompt")
    kc, vc, last = oracle.prefill(m, prompt)
    weights = device_weights(shape, w, DEV)
    kv = make_kv(shape, [128], 8, seed, DEV)
    ctx, nt, lg = gpu_prefill(weights, kv, prompt[None], [0])
    assert ctx[0] == 128
    check_logits(lg[0], last, "last logits")
    assert greedy_ok(nt[0], last)
    check_rows(kv, 0, kc, vc, 0, 128, "prompt")
    # a verify step over the GPU's own cache
    g1 = int(np.argmax(last))
    cont, _, _, _ = oracle.ar_greedy(m, kc, vc, g1, 7)
    tokens = np.concatenate([[g1], cont]).astype(np.int32)
    G = synth.geometric(0.3, seed, "replace")
    if 1 + G < 8:
        tokens[1 + G] = synth.other_token(int(tokens[1 + G]), shape.vocab, seed, "replace")
    r = oracle.verify(m, kc, vc, tokens)
    out = run_verify(weights, kv, tokens[None], None, [128])
    check_logits(out.logits[0], r.logits, "verify logits")
    check_accept(r, tokens, None, out.greedy[0], int(out.accepted_len[0]), int(out.bonus[0]), out.path[0])


def test_prefill_batch_ragged_contexts_and_lengths():
    """Three requests with committed contexts of 0, 37 and 150 positions and a 100-token prompt
    (chunks of 64 and 36), shuffled pages, one request with spare pages."""
    shape = synth.TINY
    seed = 11
    w = synth.model_weights(shape, seed)
    m = oracle_model_from(shape, w)
    weights = device_weights(shape, w, DEV)
    ctx0 = [0, 37, 150]
    p = 100
    kv = make_kv(shape, [c + p for c in ctx0], 0, seed, DEV, extra_pages=1)
    prompts = np.stack([synth.uniform_tokens(p, shape.vocab, seed, "pp", b) for b in range(3)])
    refs = []
    for b, c in enumerate(ctx0):
        ctxs = [synth.kv_context(shape, c, seed, l, request=b) for l in range(shape.n_layers)]
        kc0 = [np.ascontiguousarray(bits(x)) for x, _ in ctxs]
        vc0 = [np.ascontiguousarray(bits(y)) for _, y in ctxs]
        upload_context(kv, b, kc0, vc0)
        refs.append(oracle.prefill(m, prompts[b], kc0, vc0))
    ctx, nt, lg = gpu_prefill(weights, kv, prompts, ctx0)
    for b, c in enumerate(ctx0):
        kc, vc, last = refs[b]
        assert ctx[b] == c + p
        check_logits(lg[b], last, f"request {b} last logits")
        assert greedy_ok(nt[b], last)
        check_rows(kv, b, kc, vc, 0, c + p, f"request {b}")


def test_prefill_marks_bad_requests_only():
    shape = synth.TINY
    seed = 5
    w = synth.model_weights(shape, seed)
    weights = device_weights(shape, w, DEV)
    p = 70
    # request 1's pages (3, 48 positions) do not cover the first chunk; request 2 holds a token
    # outside the vocabulary in its second chunk
    table, n_pages = synth.page_table(3, [(p + 15) // 16, 3, (p + 15) // 16], seed)
    kv = tv.PagedKV.empty(tv.ModelCfg.of(shape), n_pages, torch.from_numpy(table), DEV)
    prompts = np.stack([synth.uniform_tokens(p, shape.vocab, seed, "bad", b) for b in range(3)])
    prompts[2, 66] = shape.vocab
    ctx, nt, _ = gpu_prefill(weights, kv, prompts, [0, 0, 0], want_logits=False)
    m = oracle_model_from(shape, w)
    kc, vc, last = oracle.prefill(m, prompts[0])
    assert ctx[0] == p and greedy_ok(nt[0], last)
    check_rows(kv, 0, kc, vc, 0, p, "good request")
    assert nt[1] == -1 and ctx[1] == 0            # fails in the first chunk
    assert nt[2] == -1 and ctx[2] == 64           # fails in the second chunk, after the first


def test_prefill_over_w12_weights_equals_bf16():
    shape = synth.TINY
    seed = 3
    w = synth.model_weights(shape, seed)
    outs = []
    for fmt in (False, True):
        dev = {k: w[k].to(DEV) for k in ("embed", "final_norm", "lm_head")}
        layers = [{k: v.to(DEV) for k, v in lw.items()} for lw in w["layers"]]
        weights = tv.Weights(tv.ModelCfg.of(shape), dev["embed"], dev["final_norm"], dev["lm_head"],
                             layers, w12=fmt)
        kv = make_kv(shape, [90], 0, seed, DEV)
        prompt = synth.uniform_tokens(90, shape.vocab, seed, "w12p")
        ctx, nt, lg = gpu_prefill(weights, kv, prompt[None], [0])
        outs.append((ctx, nt, lg, kv.k_pool.clone(), kv.v_pool.clone()))
    (c1, n1, l1, k1, v1), (c2, n2, l2, k2, v2) = outs
    # W12 is lossless and runs the same plans as bf16 below 128 rows: bit-identical results
    assert np.array_equal(c1, c2) and c1[0] == 90 and np.array_equal(n1, n2)
    assert np.array_equal(l1.view(np.int32), l2.view(np.int32))
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16))
    assert torch.equal(v1.view(torch.int16), v2.view(torch.int16))


@pytest.mark.parametrize("p,ctx0", [(1, 0), (1, 20), (64, 0), (65, 3), (129, 0)])
def test_prefill_chunk_boundaries(p, ctx0):
    """Prompt lengths at and around the 64-position chunk: a single token (also with an empty
    context), exactly one chunk, one chunk plus one token, two chunks plus one."""
    shape = synth.TINY
    seed = 40 + p
    w = synth.model_weights(shape, seed)
    m = oracle_model_from(shape, w)
    weights = device_weights(shape, w, DEV)
    kv = make_kv(shape, [ctx0 + p], 0, seed, DEV)
    ctxs = [synth.kv_context(shape, ctx0, seed, l) for l in range(shape.n_layers)]
    kc0 = [np.ascontiguousarray(bits(x)) for x, _ in ctxs]
    vc0 = [np.ascontiguousarray(bits(y)) for _, y in ctxs]
    upload_context(kv, 0, kc0, vc0)
    prompt = synth.uniform_tokens(p, shape.vocab, seed, "edge")
    kc, vc, last = oracle.prefill(m, prompt, kc0, vc0)
    ctx, nt, lg = gpu_prefill(weights, kv, prompt[None], [ctx0])
    assert ctx[0] == ctx0 + p
    check_logits(lg[0], last, "last logits")
    assert greedy_ok(nt[0], last)
    check_rows(kv, 0, kc, vc, 0, ctx0 + p, "rows")
