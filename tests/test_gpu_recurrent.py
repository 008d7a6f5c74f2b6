"""Parity of the recurrent-layer tree pass and state commit (spec_rec_tree_verify,
spec_rec_commit) against the CPU oracle, which walks every node's root path token by token in
float64 [SpecPilot digest, airadar.tv — "Reasons": tree verification for targets with recurrent
layers; the recurrence S <- exp(g) S + k v^T, o = S^T q is this library's reading].

Bound. The GPU evaluates the closed form o_i = e^{c_i} q_i^T S0 + sum_j e^{c_i - c_j}
(q_i . k_j) v_j with fp32 accumulation (path sums c in float64, rounded to fp32 before exp). The
fp32 state and the fp32 weights enter the bf16 matrix core as three bf16 parts each (exact to
2^-27 relative), so one output accumulates 3 D + 3 K products; with u = 2^-24 and each
exponential good to (|c| + 3) u, to first order
    |o_gpu - o_64| <= (3 D + 3 K + max|c| + 16) u * (e^{c_i} |q_i|^T |S0| + sum_j e^{c_i - c_j} |q_i . k_j|_abs |v_j|),
with |q . k|_abs = sum_r |q_r k_r|. The commit runs on the vector units, n path tokens in a
plain fp32 sum: (n + max|c| + 16) u times its own magnitude.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import tree_verification_skinny_amd as tv

from helpers import bits

pytestmark = pytest.mark.gpu
DEV = "cuda"
U32 = 2.0 ** -24


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _inputs(B, K, H, D, seed):
    S0, q, k, v, g = synth.rec_inputs(B, K, H, D, D, seed, DEV, "gpu")
    return S0, q, k, v, g


def _T(S):
    """The library's state layout: S transposed, [B][H][dv][dk]."""
    return S.transpose(-1, -2).contiguous()


def _host(S0, q, k, v, g):
    return S0.cpu().numpy(), bits(q), bits(k), bits(v), g.cpu().numpy()


def _paths(parent, K):
    par = np.arange(-1, K - 1) if parent is None else parent
    anc = []
    for i in range(K):
        p, j = [], i
        while j != -1:
            p.append(j)
            j = par[j]
        anc.append(p[::-1])
    return anc


def _tree_bound(S0, q, k, v, g, parents, K, D):
    B, _, H, _ = q.shape
    qf, kf, vf = (np.abs(oracle.from_bf16(x).astype(np.float64)) for x in (q, k, v))
    S = np.abs(S0.astype(np.float64))
    bound = np.zeros((B, K, H, D))
    for b in range(B):
        paths = _paths(None if parents is None else parents[b], K)
        for h in range(H):
            gg = g[b, :, h].astype(np.float64)
            for i, path in enumerate(paths):
                c = np.cumsum(gg[path])
                ci = c[-1]
                mag = np.exp(ci) * (qf[b, i, h] @ S[b, h])
                for t, j in enumerate(path):
                    mag += np.exp(ci - c[t]) * (qf[b, i, h] @ kf[b, j, h]) * vf[b, j, h]
                cmax = np.abs(c).max()
                bound[b, i, h] = (3 * D + 3 * K + cmax + 16) * U32 * mag
    return bound


def _run_tree(state_t, q, k, v, g, parent):
    """state_t: the state in the library's (transposed) layout."""
    B, K, H, D = q.shape
    out = torch.full((B, K, H, D), float("nan"), device=DEV)
    status = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    tv.spec_rec_tree_verify(state_t, q, k, v, g, parent, out, status)
    torch.cuda.synchronize()
    return out.cpu().numpy(), status.cpu().numpy()


@pytest.mark.parametrize("B,K,H,D,tree", [(2, 64, 3, 128, True), (3, 16, 2, 64, False),
                                          (2, 33, 2, 128, True), (1, 1, 4, 64, False),
                                          (2, 7, 5, 128, True), (1, 64, 2, 64, False),
                                          (1, 17, 1, 128, True), (3, 48, 1, 64, True)])
def test_tree_pass_matches_oracle(B, K, H, D, tree):
    print(f"rec tree B={B} K={K} H={H} D={D} tree={tree}", flush=True)
    S0, q, k, v, g = _inputs(B, K, H, D, K * 7 + D)
    parents = None
    pt = None
    if tree:
        parents = np.stack([synth.random_tree(K, 10, K, "rec", b) for b in range(B)]).astype(np.int32)
        pt = torch.from_numpy(parents).to(DEV)
    state_t = _T(S0)
    before = state_t.clone()
    o, st = _run_tree(state_t, q, k, v, g, pt)
    assert torch.equal(state_t.view(torch.int32), before.view(torch.int32))   # read only
    hs = _host(S0, q, k, v, g)
    ref, st_ref = oracle.rec_tree(*hs, parents)
    assert list(st) == list(st_ref) == [0] * B
    bound = _tree_bound(*hs, parents, K, D)
    err = np.abs(o - ref)
    assert np.all(err <= bound), (err.max(), float((err / np.maximum(bound, 1e-300)).max()))


def test_malformed_tree_flags_only_its_request():
    B, K, H, D = 3, 12, 2, 64
    S0, q, k, v, g = _inputs(B, K, H, D, 99)
    parents = np.stack([synth.random_tree(K, 5, 99, b) for b in range(B)]).astype(np.int32)
    parents[1, 6] = 9          # a parent after its child
    o, st = _run_tree(_T(S0), q, k, v, g, torch.from_numpy(parents).to(DEV))
    assert list(st) == [0, 1, 0]
    assert not o[1].any()
    ref, st_ref = oracle.rec_tree(*_host(S0, q, k, v, g), parents)
    assert list(st_ref) == [0, 1, 0]
    bound = _tree_bound(*_host(S0, q, k, v, g), parents, K, D)
    for b in (0, 2):
        assert np.all(np.abs(o[b] - ref[b]) <= bound[b])


@pytest.mark.parametrize("B,K,H,D", [(4, 64, 3, 128), (3, 16, 2, 64)])
def test_commit_matches_oracle(B, K, H, D):
    print(f"rec commit B={B} K={K} H={H} D={D}", flush=True)
    S0, q, k, v, g = _inputs(B, K, H, D, 5 * K + D)
    parents = np.stack([synth.random_tree(K, 10, K, "rc", b) for b in range(B)]).astype(np.int32)
    rng = np.random.default_rng(K + D)
    acc = np.zeros(B, np.int32)
    path = np.zeros((B, K), np.int32)
    for b in range(B):
        node = int(rng.integers(0, K)) if b != 1 else K - 1
        p = _paths(parents[b], K)[node]
        acc[b] = len(p) - 1
        path[b, :len(p)] = p
    acc[B - 1] = -1                          # a failed request keeps its state
    hs = _host(S0, q, k, v, g)
    state = _T(S0)
    tv.spec_rec_commit(state, k, v, g, torch.from_numpy(acc).to(DEV), torch.from_numpy(path).to(DEV))
    torch.cuda.synchronize()
    got = state.transpose(-1, -2).cpu().numpy()
    ref = oracle.rec_commit(*hs[:1], *hs[2:], acc, path)
    assert np.array_equal(got[B - 1], hs[0][B - 1])
    kf, vf = (np.abs(oracle.from_bf16(x).astype(np.float64)) for x in (hs[2], hs[3]))
    for b in range(B - 1):
        n = acc[b] + 1
        for h in range(H):
            gg = hs[4][b, path[b, :n], h].astype(np.float64)
            suf = np.concatenate([np.cumsum(gg[::-1])[::-1][1:], [0.0]])   # decay after node t
            mag = np.exp(gg.sum()) * np.abs(hs[0][b, h].astype(np.float64))
            for t in range(n):
                mag += np.exp(suf[t]) * np.outer(kf[b, path[b, t], h], vf[b, path[b, t], h])
            bound = (n + np.abs(np.cumsum(gg)).max() + 16) * U32 * mag
            assert np.all(np.abs(got[b, h] - ref[b, h]) <= bound), (b, h)


def test_commit_rejects_invalid_paths():
    """accepted_len >= k, or a path node id outside [0, k): no accepted path to apply, so the
    state stays bit-identical (as the oracle says); a valid request beside them commits."""
    B, K, H, D = 4, 16, 2, 128
    print(f"rec commit invalid paths B={B} K={K} H={H} D={D}", flush=True)
    S0, q, k, v, g = _inputs(B, K, H, D, 99)
    acc = np.asarray([3, K, 2, -1], np.int32)
    path = np.zeros((B, K), np.int32)
    path[0, :4] = [0, 1, 2, 3]
    path[1, :] = np.arange(K)
    path[2, :3] = [0, 1, K + 5]
    hs = _host(S0, q, k, v, g)
    state = _T(S0)
    tv.spec_rec_commit(state, k, v, g, torch.from_numpy(acc).to(DEV), torch.from_numpy(path).to(DEV))
    torch.cuda.synchronize()
    got = state.transpose(-1, -2).cpu().numpy()
    ref = oracle.rec_commit(*hs[:1], *hs[2:], acc, path)
    for b in (1, 2, 3):
        assert np.array_equal(got[b], hs[0][b]), b
        assert np.array_equal(ref[b], hs[0][b].astype(np.float64)), b
    assert not np.array_equal(got[0], hs[0][0])
    np.testing.assert_allclose(got[0], ref[0], rtol=1e-5, atol=1e-5)


def test_commit_then_pass_equals_child_in_tree():
    """After committing root -> best, a one-token pass from the new state gives what the tree pass
    gave the same token placed under best (within both bounds)."""
    B, K, H, D = 1, 10, 2, 128
    S0, q, k, v, g = _inputs(B, K, H, D, 1234)
    parents = np.asarray([[-1, 0, 1, 1, 0, 3, 5, 2, 6, 6]], np.int32)
    o, _ = _run_tree(_T(S0), q, k, v, g, torch.from_numpy(parents).to(DEV))
    state = _T(S0)
    path = np.zeros((1, K), np.int32)
    path[0, :5] = [0, 1, 3, 5, 6]
    tv.spec_rec_commit(state, k, v, g, torch.tensor([4], dtype=torch.int32, device=DEV),
                       torch.from_numpy(path).to(DEV))
    o1, _ = _run_tree(state, q[:, 8:9].contiguous(), k[:, 8:9].contiguous(), v[:, 8:9].contiguous(),
                      g[:, 8:9].contiguous(), None)
    b1 = _tree_bound(*_host(S0, q, k, v, g), parents, K, D)
    assert np.all(np.abs(o1[0, 0] - o[0, 8]) <= 4 * b1[0, 8])


def test_full_size_sampled_against_oracle():
    """32 requests x 64-node trees x 32 heads of 128: the launch the benchmark times, checked on
    sampled (request, head) pairs that the oracle computes alone (each pair depends only on its
    own inputs)."""
    B, K, H, D = 32, 64, 32, 128
    print(f"rec full size B={B} K={K} H={H} D={D}", flush=True)
    S0, q, k, v, g = _inputs(B, K, H, D, 2026)
    parents = np.stack([synth.random_tree(K, 10, 2026, "full", b) for b in range(B)]).astype(np.int32)
    o, st = _run_tree(_T(S0), q, k, v, g, torch.from_numpy(parents).to(DEV))
    assert not st.any()
    for b, h in [(0, 0), (13, 31), (31, 7)]:
        S = S0[b:b + 1, h:h + 1].contiguous()
        sl = lambda t: t[b:b + 1, :, h:h + 1].contiguous()
        sub = _host(S, sl(q), sl(k), sl(v), g[b:b + 1, :, h:h + 1].contiguous())
        ref, _ = oracle.rec_tree(*sub, parents[b:b + 1])
        bound = _tree_bound(*sub, parents[b:b + 1], K, D)
        assert np.all(np.abs(o[b:b + 1, :, h:h + 1] - ref) <= bound), (b, h)


@pytest.mark.parametrize("D", [64, 128])
def test_commit_deep_chain_paths(D):
    """Accepted paths longer than the 16 tokens the commit keeps in registers and LDS (41 and all
    64 nodes of a chain): the deeper tokens come from memory and must give the same state."""
    B, K, H = 2, 64, 2
    print(f"rec commit deep chain D={D}", flush=True)
    S0, q, k, v, g = _inputs(B, K, H, D, 77 + D)
    acc = np.asarray([40, 63], np.int32)
    path = np.tile(np.arange(K, dtype=np.int32), (B, 1))
    hs = _host(S0, q, k, v, g)
    state = _T(S0)
    tv.spec_rec_commit(state, k, v, g, torch.from_numpy(acc).to(DEV), torch.from_numpy(path).to(DEV))
    torch.cuda.synchronize()
    got = state.transpose(-1, -2).cpu().numpy()
    ref = oracle.rec_commit(hs[0], hs[2], hs[3], hs[4], acc, path)
    kf, vf = (np.abs(oracle.from_bf16(x).astype(np.float64)) for x in (hs[2], hs[3]))
    for b in range(B):
        n = acc[b] + 1
        for h in range(H):
            gg = hs[4][b, :n, h].astype(np.float64)
            suf = np.concatenate([np.cumsum(gg[::-1])[::-1][1:], [0.0]])
            mag = np.exp(gg.sum()) * np.abs(hs[0][b, h].astype(np.float64))
            for t in range(n):
                mag += np.exp(suf[t]) * np.outer(kf[b, t, h], vf[b, t, h])
            bound = (n + np.abs(np.cumsum(gg)).max() + 16) * U32 * mag
            assert np.all(np.abs(got[b, h] - ref[b, h]) <= bound), (b, h)
