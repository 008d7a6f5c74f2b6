"""Pins of the recurrent-layer oracle (tree verification for a hybrid target).

The pages name tree verification for targets with recurrent layers [SpecPilot digest,
airadar.tv — "Reasons"] and give no recurrence; the reading is a scalar-gated linear recurrence
per head, S <- exp(g) S + k v^T and o = S^T q, every tree node continuing its parent's state.
The oracle walks each node's root path token by token. It is pinned here by:
  * hand-worked values of a 3-node tree, a chain and a commit (tests/golden/rec_tree_tiny.json);
  * the parallel (masked-matrix) form of the same recurrence on chains, a different formula;
  * tree = the chain over each node's own root path (path conditioning);
  * a zero gate forgets everything before it;
  * commit followed by a one-token pass = the same token as a child in the tree pass;
  * malformed trees and failed requests.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden", "rec_tree_tiny.json")


def _np_bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _case(B, K, H, dk, dv, seed):
    S0, q, k, v, g = synth.rec_inputs(B, K, H, dk, dv, seed, "cpu", "pin")
    return S0.numpy(), _np_bits(q), _np_bits(k), _np_bits(v), g.numpy()


def _golden():
    with open(GOLD) as f:
        d = json.load(f)
    bf = lambda x: oracle.to_bf16(np.asarray(x, np.float32))
    S0 = np.asarray(d["S0"], np.float32)[None, None]
    q = bf(d["q"])[None, :, None]
    k = bf(d["k"])[None, :, None]
    v = bf(d["v"])[None, :, None]
    g = np.full((1, 3, 1), np.log(np.float32(d["a"])), np.float32)
    return d, S0, q, k, v, g


def test_golden_tree_chain_commit():
    d, S0, q, k, v, g = _golden()
    par = np.asarray(d["parent"], np.int32)[None]
    o, st = oracle.rec_tree(S0, q, k, v, g, par)
    assert st[0] == 0
    np.testing.assert_allclose(o[0, :, 0], d["out_tree"], rtol=1e-7, atol=1e-7)
    o, st = oracle.rec_tree(S0, q, k, v, g, None)
    np.testing.assert_allclose(o[0, :, 0], d["out_chain"], rtol=1e-7, atol=1e-7)
    S = oracle.rec_commit(S0, k, v, g, np.asarray([d["accepted_len"]], np.int32),
                          np.asarray(d["accepted_path"], np.int32)[None])
    np.testing.assert_allclose(S[0, 0], d["state_commit"], rtol=1e-7, atol=1e-7)


@pytest.mark.parametrize("seed", [0, 1])
def test_chain_equals_parallel_form(seed):
    """o_i = exp(c_i) q_i^T S0 + sum_{j <= i} exp(c_i - c_j) (q_i . k_j) v_j with c the running
    sum of the log-gates: the masked-matrix form of the recurrence, evaluated in float64."""
    B, K, H, dk, dv = 2, 12, 2, 16, 8
    S0, q, k, v, g = _case(B, K, H, dk, dv, seed)
    o, st = oracle.rec_tree(S0, q, k, v, g, None)
    assert not st.any()
    qf, kf, vf = (oracle.from_bf16(x).astype(np.float64) for x in (q, k, v))
    for b in range(B):
        for h in range(H):
            c = np.cumsum(g[b, :, h].astype(np.float64))
            L = np.tril(np.exp(c[:, None] - c[None, :]))
            Q, Kt, V = qf[b, :, h], kf[b, :, h], vf[b, :, h]
            ref = np.exp(c)[:, None] * (Q @ S0[b, h].astype(np.float64)) + (L * (Q @ Kt.T)) @ V
            np.testing.assert_allclose(o[b, :, h], ref, rtol=1e-10, atol=1e-12)


def test_tree_equals_chain_over_each_path():
    B, K, H, dk, dv = 1, 20, 2, 8, 8
    S0, q, k, v, g = _case(B, K, H, dk, dv, 7)
    par = synth.random_tree(K, 6, 7, "rec")[None].astype(np.int32)
    o, st = oracle.rec_tree(S0, q, k, v, g, par)
    assert st[0] == 0
    for i in range(K):
        path = []
        j = i
        while j != -1:
            path.append(j)
            j = par[0, j]
        path = path[::-1]
        oc, _ = oracle.rec_tree(S0, q[:, path], k[:, path], v[:, path], g[:, path], None)
        assert np.array_equal(o[0, i], oc[0, -1])


def test_zero_gate_forgets_the_past():
    B, K, H, dk, dv = 1, 8, 1, 8, 4
    S0, q, k, v, g = _case(B, K, H, dk, dv, 3)
    g[0, 4, 0] = -np.inf
    o1, _ = oracle.rec_tree(S0, q, k, v, g, None)
    S0b, _, k2, v2, _ = _case(B, K, H, dk, dv, 4)
    k2[:, 4:], v2[:, 4:] = k[:, 4:], v[:, 4:]
    o2, _ = oracle.rec_tree(S0b, q, k2, v2, g, None)
    assert np.array_equal(o1[0, 4:], o2[0, 4:])
    assert not np.allclose(o1[0, :4], o2[0, :4])


def test_commit_then_one_token_equals_child_in_tree():
    """Commit the path root -> best, then pass one more token from that state: its output equals
    the same token placed under best in the tree pass (up to the fp32 rounding of the state)."""
    B, K, H, dk, dv = 1, 10, 2, 8, 8
    S0, q, k, v, g = _case(B, K, H, dk, dv, 11)
    par = np.asarray([[-1, 0, 1, 1, 0, 3, 5, 2, 6, 6]], np.int32)
    path = [0, 1, 3, 5, 6]
    o, _ = oracle.rec_tree(S0, q, k, v, g, par)
    ap = np.zeros((1, K), np.int32)
    ap[0, :5] = path
    S1 = oracle.rec_commit(S0, k, v, g, np.asarray([4], np.int32), ap)
    o1, _ = oracle.rec_tree(S1.astype(np.float32), q[:, [8]], k[:, [8]], v[:, [8]], g[:, [8]], None)
    scale = np.abs(S1).max() * 4
    np.testing.assert_allclose(o1[0, 0], o[0, 8], rtol=0, atol=scale * 2.0 ** -23)


def test_malformed_tree_and_failed_commit():
    B, K, H, dk, dv = 2, 6, 1, 4, 4
    S0, q, k, v, g = _case(B, K, H, dk, dv, 5)
    par = np.asarray([[-1, 0, 1, 5, 2, 3], [-1, 0, 0, 1, 1, 2]], np.int32)
    o, st = oracle.rec_tree(S0, q, k, v, g, par)
    assert list(st) == [1, 0]
    assert not o[0].any() and o[1].any()
    S = oracle.rec_commit(S0, k, v, g, np.asarray([-1, 0], np.int32), np.zeros((B, K), np.int32))
    assert np.array_equal(S[0], S0[0].astype(np.float64))
    ref = np.exp(np.float64(g[1, 0, 0])) * S0[1, 0].astype(np.float64) + np.outer(
        oracle.from_bf16(k[1, 0, 0]).astype(np.float64), oracle.from_bf16(v[1, 0, 0]).astype(np.float64))
    np.testing.assert_allclose(S[1, 0], ref, rtol=1e-15, atol=1e-15)


def test_commit_rejects_out_of_range_requests():
    """A request with accepted_len >= K, or whose accepted path names a node outside [0, K),
    has no accepted path to apply and keeps its committed state bit for bit; a valid request
    beside them is committed as usual (the state after its path tokens, worked in float64)."""
    B, K, H, dk, dv = 4, 5, 2, 4, 4
    S0, q, k, v, g = _case(B, K, H, dk, dv, 21)
    al = np.asarray([K, 2, 1, 0], np.int32)
    ap = np.full((B, K), -1, np.int32)
    ap[0] = [0, 1, 2, 3, 4]
    ap[1, :3] = [0, 1, K]          # node id past the tree
    ap[2, :2] = [0, -3]            # negative node id
    ap[3, :1] = [0]
    S = oracle.rec_commit(S0, k, v, g, al, ap)
    for b in (0, 1, 2):
        assert np.array_equal(S[b], S0[b].astype(np.float64)), b
    for h in range(H):
        ref = np.exp(np.float64(g[3, 0, h])) * S0[3, h].astype(np.float64) + np.outer(
            oracle.from_bf16(k[3, 0, h]).astype(np.float64),
            oracle.from_bf16(v[3, 0, h]).astype(np.float64))
        np.testing.assert_allclose(S[3, h], ref, rtol=1e-15, atol=1e-15)
