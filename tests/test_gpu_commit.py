"""The KV commit on the GPU where rows really move, checked bit for bit over the whole cache.

Only the accepted root path becomes context [SpecPilot digest, airadar.tv — "Risks"], and a
tree node's K/V row belongs to its own root path [JetSpec article, seventnews.com — "Technical
architecture"]. After spec_verify wrote node i's row into slot ctx + i, spec_commit_kv must move
the accepted path's rows to slots ctx .. ctx + a: slot ctx + t <- slot ctx + path[t]. In a
breadth-first tree the node at depth t usually has an id above t, so these moves are real
(overlapping) copies, unlike a chain where path[t] = t.

Checks:
  * a batch of five requests with k = 64: two trees whose greedy paths are planted along
    branches (path[t] > t), a 64-chain accepted whole (a = k - 1), a request that fails in
    verify (a = -1) and one that accepts nothing; every byte of both pools after the commit
    equals the pools before it with exactly the documented moves applied;
  * the contexts advance by a + 1, the failed request's does not;
  * a second verify over the committed cache meets the oracle's verify over the oracle's
    committed cache (the fixed tolerance; acceptance exact up to logged near-ties);
  * caller-supplied invalid commits (accepted_len past k, a path that does not start at the
    root, a node id below its depth or past k, a context past the pages) leave the request's
    rows and context untouched while valid requests beside them commit.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
import tree_verification_skinny_amd as tv

from helpers import (bits, check_accept, check_logits, device_weights, make_kv, oracle_model_from,
                     run_verify, upload_context)
from test_gpu_parity import planted_tree

pytestmark = pytest.mark.gpu
DEV = "cuda"


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tv.lib()


def _slot(table: np.ndarray, b: int, pos: int):
    return int(table[b, pos // 16]), pos % 16


def expected_pools(k_pool: np.ndarray, v_pool: np.ndarray, table: np.ndarray, ctx, acc, path, k):
    """The pools after the documented moves, applied on host copies (uint16 bits).
    k_pool [L][pages][nkv][16][d], v_pool [L][pages][nkv][d][16]."""
    ke, ve = k_pool.copy(), v_pool.copy()
    for b, a in enumerate(acc):
        if a < 0:
            continue
        for t in range(a + 1):
            sp, ss = _slot(table, b, ctx[b] + int(path[b][t]))
            dp, ds = _slot(table, b, ctx[b] + t)
            ke[:, dp, :, ds, :] = k_pool[:, sp, :, ss, :]
            ve[:, dp, :, :, ds] = v_pool[:, sp, :, :, ss]
    return ke, ve


def _pool_bits(kv):
    return bits(kv.k_pool), bits(kv.v_pool)


def _context(ctx, seed, b):
    kvs = [synth.kv_context(synth.TINY, ctx, seed, l, request=b) for l in range(2)]
    return [np.ascontiguousarray(bits(x)) for x, _ in kvs], [np.ascontiguousarray(bits(y)) for _, y in kvs]


def _greedy_chain(w, m, kc, vc, ctx, K, seed):
    """A K-chain the GPU pass accepts whole: the oracle's greedy continuation of a random root,
    with every token where the GPU's greedy choice differs (a near-tie the pass inverts: the
    oracle's top-2 margin is below the GPU's logit error) replaced by the GPU's choice, position
    by position until the chain is consistent. The oracle check of the batched pass still holds
    the GPU to the near-tie rule at those nodes."""
    root = int(synth.uniform_tokens(1, 1024, seed, "chain")[0])
    cont, _, _, _ = oracle.ar_greedy(m, kc, vc, root, K - 1)
    tok = np.concatenate([[root], cont]).astype(np.int32)
    weights = device_weights(synth.TINY, w, DEV)
    kv = make_kv(synth.TINY, [ctx], K, seed, DEV)
    upload_context(kv, 0, kc, vc)
    for _ in range(K):
        out = run_verify(weights, kv, tok[None], None, [ctx], want_logits=False)
        g = out.greedy[0]
        diff = np.nonzero(g[:-1] != tok[1:])[0]
        if diff.size == 0:
            return tok
        tok[diff[0] + 1] = g[diff[0]]
    raise AssertionError("greedy chain did not settle")


def test_batched_tree_commit_moves_rows_and_second_verify_meets_oracle():
    K = 64
    seed = 4242
    w = synth.model_weights(synth.TINY, seed)
    m = oracle_model_from(synth.TINY, w)
    ctxs = [100, 37, 50, 130, 16]
    B = len(ctxs)
    cases, toks, pars = [], [], []
    for b, ctx in enumerate(ctxs):
        kc, vc = _context(ctx, seed, b)
        if b in (0, 3):          # trees, greedy paths planted along branches
            tok, par = planted_tree(m, kc, vc, K, seed + b, p_follow=0.9 if b == 0 else 0.6)
        elif b == 1:             # the pass's own greedy continuation: accepted whole
            tok, par = _greedy_chain(w, m, kc, vc, ctx, K, seed), oracle.chain(K)
        else:                    # b = 2 fails in verify (token outside the vocabulary); b = 4 random
            tok, par = synth.uniform_tokens(K, 1024, seed, b).astype(np.int32), oracle.chain(K)
        toks.append(tok)
        pars.append(par)
        cases.append((kc, vc))
    tokens = np.stack(toks).astype(np.int32)
    parent = np.stack(pars).astype(np.int32)
    tokens[2, 7] = 1024
    weights = device_weights(synth.TINY, w, DEV)
    kv = make_kv(synth.TINY, ctxs, K, seed, DEV, extra_pages=1)
    for b in range(B):
        upload_context(kv, b, *cases[b])
    out = run_verify(weights, kv, tokens, parent, ctxs)
    acc, path = out.accepted_len.copy(), out.path.copy()
    results = []
    for b in range(B):
        if b == 2:
            assert acc[b] == -1 and out.bonus[b] == -1
            results.append(None)
            continue
        r = oracle.verify(m, cases[b][0], cases[b][1], tokens[b], parent[b])
        check_logits(out.logits[b], r.logits, f"request {b} logits")
        check_accept(r, tokens[b], parent[b], out.greedy[b], int(acc[b]), int(out.bonus[b]), path[b])
        results.append(r)
    print(f"accepted {list(acc)}; paths {[list(path[b][: acc[b] + 1]) for b in (0, 3)]}")
    # the case must exercise what it is for
    assert acc[1] == K - 1, "the pass's own greedy 64-chain must be accepted whole"
    moved = [b for b in (0, 3) if acc[b] > 0 and np.any(path[b][1: acc[b] + 1] > np.arange(1, acc[b] + 1))]
    assert moved, "no tree path with path[t] > t: the commit would not move a row"

    table = kv.block_table.cpu().numpy()
    k_before, v_before = _pool_bits(kv)
    tv.spec_commit_kv(weights.cfg, kv, out.acc_t, out.path_t, out.ctx, B, K)
    torch.cuda.synchronize()
    k_after, v_after = _pool_bits(kv)
    ke, ve = expected_pools(k_before, v_before, table, ctxs, acc, path, K)
    assert np.array_equal(k_after, ke), "K pool differs from the documented moves"
    assert np.array_equal(v_after, ve), "V pool differs from the documented moves"
    new_ctx = out.ctx.cpu().numpy()
    for b in range(B):
        assert new_ctx[b] == (ctxs[b] if acc[b] < 0 else ctxs[b] + acc[b] + 1), b

    # second step over the committed cache: root = the bonus token, a fresh random block
    K2 = 8
    toks2, cases2 = [], []
    for b in range(B):
        if b == 2:
            kc2, vc2 = cases[b]
            root = 5
        else:
            # the oracle's rows along the path the GPU accepted (the same path unless a logged
            # near-tie moved it)
            r_gpu = dataclasses.replace(results[b], accepted_len=int(acc[b]), path=path[b])
            kc2, vc2 = oracle.commit(cases[b][0], cases[b][1], r_gpu)
            root = int(out.bonus[b])
        t2 = synth.uniform_tokens(K2, 1024, seed + 1, b).astype(np.int32)
        t2[0] = root
        toks2.append(t2)
        cases2.append((kc2, vc2))
    tokens2 = np.stack(toks2)
    # the pages past ctx + 64 were reserved by the first step (extra page covers ctx' + 8)
    out2 = run_verify(weights, kv, tokens2, None, [int(c) for c in new_ctx])
    for b in range(B):
        r2 = oracle.verify(m, cases2[b][0], cases2[b][1], tokens2[b])
        check_logits(out2.logits[b], r2.logits, f"second step, request {b}")
        check_accept(r2, tokens2[b], None, out2.greedy[b], int(out2.accepted_len[b]),
                     int(out2.bonus[b]), out2.path[b])


def test_invalid_commits_leave_requests_untouched():
    """Caller-supplied accepted paths: the invalid requests keep every row and their context,
    valid requests beside them commit (bit for bit against the documented moves)."""
    K, B = 12, 7
    seed = 77
    ctxs = [20, 33, 5, 64, 90, 0, 40]
    kv = make_kv(synth.TINY, ctxs, K, seed, DEV, extra_pages=0)
    g = torch.Generator(device="cpu").manual_seed(seed)
    kv.k_pool.copy_(torch.randn(kv.k_pool.shape, generator=g).to(torch.bfloat16))
    kv.v_pool.copy_(torch.randn(kv.v_pool.shape, generator=g).to(torch.bfloat16))
    acc = np.asarray([3, K, 2, 2, 4, 5, 1], np.int32)
    path = np.full((B, K), -1, np.int32)
    path[0, :4] = [0, 2, 5, 9]          # valid, rows move
    path[1, :] = np.arange(K)           # accepted_len = K: invalid
    path[2, :3] = [3, 4, 5]             # does not start at the root: invalid
    path[3, :3] = [0, 2, 1]             # node id below its depth: invalid
    path[4, :5] = [0, 1, 2, 3, K]       # node id past the tree: invalid
    path[5, :6] = [0, 1, 4, 6, 8, 11]   # valid, from an empty context
    path[6, :2] = [0, 1]                # valid, but its context is pushed past its pages below
    ctx_dev = list(ctxs)
    ctx_dev[6] = kv.max_pages * 16 - K + 1
    table = kv.block_table.cpu().numpy()
    cfg = tv.ModelCfg.of(synth.TINY)
    t_acc = torch.from_numpy(acc).to(DEV)
    t_path = torch.from_numpy(path).to(DEV)
    t_ctx = torch.tensor(ctx_dev, dtype=torch.int32, device=DEV)
    k_before, v_before = _pool_bits(kv)
    tv.spec_commit_kv(cfg, kv, t_acc, t_path, t_ctx, B, K)
    torch.cuda.synchronize()
    k_after, v_after = _pool_bits(kv)
    valid = np.asarray([1, 0, 0, 0, 0, 1, 0], bool)
    eff = np.where(valid, acc, -1)
    ke, ve = expected_pools(k_before, v_before, table, ctx_dev, eff, path, K)
    assert np.array_equal(k_after, ke) and np.array_equal(v_after, ve)
    new_ctx = t_ctx.cpu().numpy()
    for b in range(B):
        assert new_ctx[b] == (ctx_dev[b] + acc[b] + 1 if valid[b] else ctx_dev[b]), b
