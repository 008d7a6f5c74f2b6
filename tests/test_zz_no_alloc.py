"""spec_accept_noalloc (the library's static per-GPU scratch instead of a workspace) against
spec_accept on the same inputs, bit for bit: two calls in a row, the second smaller, so the
second runs over the scratch the first left behind."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tree_verification_skinny_amd as tv

pytestmark = pytest.mark.gpu
DEV = "cuda"


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tv.lib()


def _case(batch, k, vocab, tree, seed):
    toks, pars, lgs = [], [], []
    for b in range(batch):
        s = (seed, b)
        if tree:
            par = synth.random_tree(k, 10, s)
            tok = synth.tree_tokens(par, vocab, s)
        else:
            par = oracle.chain(k)
            tok = synth.uniform_tokens(k, vocab, s, "na")
        lg, _ = synth.planted_logits(tok, par, vocab, synth.geometric(0.25, s), s)
        toks.append(tok)
        pars.append(par)
        lgs.append(lg)
    tokens = torch.from_numpy(np.stack(toks).astype(np.int32)).to(DEV)
    parent = torch.from_numpy(np.stack(pars).astype(np.int32)).to(DEV) if tree else None
    logits = torch.from_numpy(np.stack(lgs).reshape(batch * k, vocab)).to(DEV)
    tokens[batch - 1, k - 1] = vocab          # the last request fails alone
    return tokens, parent, logits


def _outs(batch, k):
    return (torch.full((batch,), -9, dtype=torch.int32, device=DEV),
            torch.full((batch,), -9, dtype=torch.int32, device=DEV),
            torch.full((batch, k), -9, dtype=torch.int32, device=DEV),
            torch.full((batch * k,), -9, dtype=torch.int32, device=DEV))


def _both(batch, k, vocab, tree, seed):
    print(f"no-alloc accept batch={batch} k={k} vocab={vocab} tree={tree}", flush=True)
    tokens, parent, logits = _case(batch, k, vocab, tree, seed)
    ws = tv.workspace(tv.spec_accept_workspace_bytes(batch, k, vocab), DEV)
    ref = _outs(batch, k)
    tv.spec_accept(logits, tokens, parent, batch, k, vocab, *ref[:3], ws, greedy=ref[3])
    got = _outs(batch, k)
    tv.spec_accept_noalloc(logits, tokens, parent, batch, k, vocab, *got[:3], greedy=got[3])
    torch.cuda.synchronize()
    for r, g, name in zip(ref, got, ("accepted_len", "bonus", "path", "greedy")):
        assert torch.equal(r, g), name
    acc = got[0].cpu().numpy()
    assert acc[-1] == -1 and (acc[:-1] >= 0).all()


def test_noalloc_matches_workspace_entry_point_twice():
    _both(48, 64, 151936, True, 1)      # 3072 rows, near the row limit
    _both(3, 5, 1000, False, 2)         # smaller, over the scratch the first call left


def test_noalloc_rejects_sizes_past_the_scratch():
    tokens, parent, logits = _case(2, 4, 1024, False, 3)
    outs = _outs(2, 4)
    with pytest.raises(RuntimeError, match="scratch"):
        tv.spec_accept_noalloc(logits, tokens, parent, 4097, 1, 1024, *outs[:3])
    with pytest.raises(RuntimeError, match="scratch"):
        tv.spec_accept_noalloc(logits, tokens, parent, 1, 4, tv.SPEC_NOALLOC_MAX_VOCAB + 64, *outs[:3])
