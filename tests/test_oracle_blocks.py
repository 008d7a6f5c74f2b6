"""Pins of the CPU oracle's building blocks against things other than itself: torch's own bf16
conversion, float64 references with a classical rounding-error bound, closed forms
(complex rotation, one-key and equal-score attention), torch's scaled_dot_product_attention in
float64, numpy.argmax, and brute force over root paths."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

U32 = 2.0 ** -24          # unit roundoff of binary32
BF16_REL = 2.0 ** -8      # one bf16 ulp, relative (a rounding is within half of it)


def bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def f64(h: np.ndarray) -> np.ndarray:
    return oracle.from_bf16(h).astype(np.float64)


def rand_bf16(shape, std, seed):
    return bits(synth.randn_bf16(shape, std, "cpu", "test", seed))


# ------------------------------------------------------------------------------------------
# bf16 conversion: torch's float32 -> bfloat16 cast is round-to-nearest-even
# ------------------------------------------------------------------------------------------

def test_bf16_rounding_matches_torch():
    g = torch.Generator().manual_seed(1)
    x = torch.randn(100000, generator=g) * torch.exp2(torch.randint(-130, 120, (100000,), generator=g).float())
    edge = torch.tensor([0.0, -0.0, 1.0, -1.0, float("inf"), float("-inf"), 3.4e38, -3.4e38, 1e-40,
                         -1e-40, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20,
                         1.0 + 2 ** -9, 1.00390625, 2.0 ** -126, 2.0 ** -133])
    # exact ties: low 16 bits == 0x8000 with even and odd kept parts
    ties = torch.tensor(np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x7F7F8000], np.uint32).view(np.float32))
    x = torch.cat([x, edge, ties]).float()
    got = oracle.to_bf16(x.numpy())
    want = bits(x.to(torch.bfloat16))
    assert np.array_equal(got, want)
    assert np.array_equal(oracle.from_bf16(want), x.to(torch.bfloat16).float().numpy())


def test_bf16_nan_stays_nan():
    x = np.array([np.nan, -np.nan], np.float32)
    assert np.all(np.isnan(oracle.from_bf16(oracle.to_bf16(x))))


# ------------------------------------------------------------------------------------------
# linear: float64 product of the same bf16 operands, within the fp32 summation bound
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("m,kd,n", [(1, 32, 16), (5, 256, 48), (16, 704, 40), (3, 1000, 7)])
def test_linear_within_summation_bound(m, kd, n):
    x = rand_bf16((m, kd), 1.0, ("lx", m, kd))
    w = rand_bf16((n, kd), 0.02, ("lw", m, kd))
    y = oracle.linear(x, w).astype(np.float64)
    ref = f64(x) @ f64(w).T
    gamma = kd * U32 / (1 - kd * U32)
    bound = gamma * (np.abs(f64(x)) @ np.abs(f64(w)).T)
    assert np.all(np.abs(y - ref) <= bound + 1e-30)
    # a transposed or shifted operand would be far outside the bound
    assert np.max(np.abs(ref)) > 100 * np.max(bound)


def test_linear_exact_on_small_integers():
    x = np.arange(-8, 8, dtype=np.float32).reshape(2, 8)
    w = np.array([[1, 0, 0, 0, 0, 0, 0, 2], [0, 1, -1, 0, 3, 0, 0, 0], [1] * 8], np.float32)
    y = oracle.linear(oracle.to_bf16(x), oracle.to_bf16(w))
    assert np.array_equal(y, (x @ w.T).astype(np.float32))


# ------------------------------------------------------------------------------------------
# RMSNorm
# ------------------------------------------------------------------------------------------

def test_rmsnorm_float64_reference_and_gain():
    x = rand_bf16((7, 256), 1.0, "nx")
    g = rand_bf16((256,), 1.0, "ng")
    out = f64(oracle.rmsnorm(x, g, 1e-6))
    xf, gf = f64(x), f64(g)
    ref = xf / np.sqrt(np.mean(xf ** 2, axis=1, keepdims=True) + 1e-6) * gf
    assert np.all(np.abs(out - ref) <= BF16_REL * np.abs(ref) + 1e-6)


def test_rmsnorm_unit_rms_and_scale_invariance():
    x = rand_bf16((4, 5120), 3.0, "nx2")
    g = oracle.to_bf16(np.ones(5120, np.float32))
    out = f64(oracle.rmsnorm(x, g, 1e-6))
    rms = np.sqrt(np.mean(out ** 2, axis=1))
    assert np.all(np.abs(rms - 1) < 2e-3)
    x4 = oracle.to_bf16(oracle.from_bf16(x) * 4.0)          # exact in bf16
    out4 = f64(oracle.rmsnorm(x4, g, 1e-6))
    assert np.max(np.abs(out4 - out)) <= 2 * BF16_REL * np.max(np.abs(out))


# ------------------------------------------------------------------------------------------
# RoPE: rotate-half == multiplication of z_j = t[j] + i t[j + d/2] by exp(i pos theta^(-2j/d))
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("d", [64, 128])
def test_rope_matches_complex_rotation(d):
    t = rand_bf16((6, 3, d), 1.0, ("rt", d))
    pos = np.array([0, 1, 7, 128, 4095, 8200], np.int32)
    out = f64(oracle.rope(t, pos, 1e4))
    tf = f64(t)
    half = d // 2
    z = tf[..., :half] + 1j * tf[..., half:]
    freq = 1e4 ** (-2.0 * np.arange(half) / d)
    zr = z * np.exp(1j * pos[:, None, None] * freq[None, None, :])
    ref = np.concatenate([zr.real, zr.imag], axis=-1)
    assert np.all(np.abs(out - ref) <= BF16_REL * np.abs(ref) + 4 * U32 * np.abs(z).repeat(2, -1).reshape(ref.shape) + 1e-7)


def test_rope_position_zero_is_identity():
    t = rand_bf16((3, 5, 128), 1.0, "r0")
    assert np.array_equal(oracle.rope(t, np.zeros(3, np.int32), 1e4), t)


def test_rope_relative_position_property():
    q = rand_bf16((1, 1, 128), 1.0, "rq")
    k = rand_bf16((1, 1, 128), 1.0, "rk")

    def dot(mq, nk):
        a = f64(oracle.rope(q, np.array([mq], np.int32), 1e4))
        b = f64(oracle.rope(k, np.array([nk], np.int32), 1e4))
        return float(np.sum(a * b))

    base = dot(10, 3)
    for shift in (1, 100, 3000):
        assert abs(dot(10 + shift, 3 + shift) - base) < 0.08   # bf16 rounding of both operands
    assert abs(dot(10, 3) - dot(3, 10)) > 1e-3                  # depends on the sign of m - n


# ------------------------------------------------------------------------------------------
# attention
# ------------------------------------------------------------------------------------------

def _sdpa_ref(q, k_ctx, v_ctx, k_new, v_new, parent):
    """float64 torch SDPA with an explicit visibility mask: context keys visible to all, node j
    visible to node i iff j lies on i's root path (found by following parents)."""
    m, nq, d = q.shape
    nkv = k_new.shape[1]
    ctx = k_ctx.shape[0]
    keys = np.concatenate([f64(k_ctx), f64(k_new)], 0)        # [ctx+m][nkv][d]
    vals = np.concatenate([f64(v_ctx), f64(v_new)], 0)
    mask = np.zeros((m, ctx + m), bool)
    mask[:, :ctx] = True
    for i in range(m):
        node = i
        while node >= 0:
            mask[i, ctx + node] = True
            node = int(parent[node])
    rep = nq // nkv
    K = torch.tensor(keys).permute(1, 0, 2).repeat_interleave(rep, 0)   # [nq][keys][d]
    V = torch.tensor(vals).permute(1, 0, 2).repeat_interleave(rep, 0)
    Q = torch.tensor(f64(q)).permute(1, 0, 2)                           # [nq][m][d]
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=torch.tensor(mask))
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("ctx,m,tree", [(0, 1, False), (5, 8, False), (37, 12, True), (200, 16, True)])
def test_attention_matches_sdpa_float64(ctx, m, tree):
    nq, nkv, d = 4, 2, 64
    q = rand_bf16((m, nq, d), 1.0, ("aq", ctx, m))
    kc = rand_bf16((ctx, nkv, d), 1.0, ("akc", ctx, m))
    vc = rand_bf16((ctx, nkv, d), 1.0, ("avc", ctx, m))
    kn = rand_bf16((m, nkv, d), 1.0, ("akn", ctx, m))
    vn = rand_bf16((m, nkv, d), 1.0, ("avn", ctx, m))
    parent = synth.random_tree(m, 4, "atree", m) if tree else oracle.chain(m)
    o = f64(oracle.attention(q, kc, vc, kn, vn, parent))
    ref = _sdpa_ref(q, kc, vc, kn, vn, parent)
    assert np.all(np.abs(o - ref) <= BF16_REL * np.abs(ref) + 1e-5)


def test_attention_single_key_returns_value_exactly():
    q = rand_bf16((1, 4, 64), 1.0, "sq")
    kn = rand_bf16((1, 2, 64), 1.0, "sk")
    vn = rand_bf16((1, 2, 64), 1.0, "sv")
    empty = np.zeros((0, 2, 64), np.uint16)
    o = oracle.attention(q, empty, empty, kn, vn, np.array([-1], np.int32))
    assert np.array_equal(o, vn[:, [0, 0, 1, 1], :])       # heads 0,1 -> kv 0; heads 2,3 -> kv 1


def test_attention_equal_scores_average_and_unit_weights():
    nkv, d = 2, 64
    kc = np.tile(rand_bf16((1, nkv, d), 1.0, "ek"), (50, 1, 1))
    vc = rand_bf16((50, nkv, d), 1.0, "ev")
    q = rand_bf16((1, 4, d), 1.0, "eq")
    kn = kc[:1].copy()
    vn = rand_bf16((1, nkv, d), 1.0, "evn")
    o = f64(oracle.attention(q, kc, vc, kn, vn, np.array([-1], np.int32)))
    mean = (f64(vc).sum(0) + f64(vn)[0]) / 51
    assert np.all(np.abs(o[0] - mean[[0, 0, 1, 1]]) <= BF16_REL * np.abs(mean[[0, 0, 1, 1]]) + 1e-6)
    # all values 1: the normalised weights sum to exactly one
    ones = oracle.to_bf16(np.ones((50, nkv, d), np.float32))
    o1 = oracle.attention(q, rand_bf16((50, nkv, d), 1.0, "ek2"), ones, kn, ones[:1], np.array([-1], np.int32))
    assert np.all(oracle.from_bf16(o1) == 1.0)


# ------------------------------------------------------------------------------------------
# SwiGLU, argmax, tree depth, acceptance
# ------------------------------------------------------------------------------------------

def test_swiglu_float64_reference():
    gate = rand_bf16((5000,), 3.0, "sg")
    up = rand_bf16((5000,), 1.0, "su")
    out = f64(oracle.swiglu(gate, up))
    gf, uf = f64(gate), f64(up)
    ref = gf / (1 + np.exp(-gf)) * uf
    assert np.all(np.abs(out - ref) <= BF16_REL * np.abs(ref) + 1e-30)


def test_argmax_matches_numpy_first_occurrence():
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((40, 1537)).astype(np.float32)
    for i in range(0, 40, 3):                       # planted ties: lowest index must win
        j1, j2 = sorted(rng.choice(1537, 2, replace=False))
        lg[i, j1] = lg[i, j2] = lg[i].max() + 1
    arg, margin = oracle.argmax(lg)
    assert np.array_equal(arg, np.argmax(lg, axis=1).astype(np.int32))
    s = np.sort(lg, axis=1)
    assert np.array_equal(margin, (s[:, -1] - s[:, -2]).astype(np.float32))


def test_tree_depth_and_malformed_trees():
    assert list(oracle.tree_depth(np.array([-1, 0, 0, 1, 3, 2]))) == [0, 1, 1, 2, 3, 2]
    for bad in ([0, 0], [-1, 1], [-1, 0, 5], [-1, -1], [-1, 0, 2]):
        assert oracle.tree_depth(np.array(bad)) is None
        a, b, path = oracle.accept(np.zeros(len(bad)), np.array(bad), np.zeros(len(bad)))
        assert (a, b) == (-1, -1) and np.all(path == -1)


def _brute_force_accept(tokens, parent, arg):
    """Enumerate every node's root path; a node is accepted iff every token on its path (root
    excluded) is the greedy choice of its parent. Deepest accepted node, lowest id on ties."""
    k = len(tokens)
    best, best_path = 0, [0]
    for i in range(k):
        path = []
        node = i
        while node >= 0:
            path.append(node)
            node = int(parent[node])
        path.reverse()
        if all(tokens[path[t + 1]] == arg[path[t]] for t in range(len(path) - 1)):
            if len(path) - 1 > len(best_path) - 1:
                best, best_path = i, path
    return len(best_path) - 1, int(arg[best]), best_path


@pytest.mark.parametrize("k,kind", [(1, "chain"), (2, "chain"), (8, "chain"), (16, "chain"),
                                    (64, "chain"), (12, "tree"), (64, "tree")])
@pytest.mark.parametrize("seed", range(12))
def test_accept_planted_closed_form_and_brute_force(k, kind, seed):
    vocab = 1024
    if kind == "chain":
        parent = oracle.chain(k)
        tokens = synth.uniform_tokens(k, vocab, seed, "acc", k)
    else:
        parent = synth.random_tree(k, 10, seed, "acc", k)
        tokens = synth.tree_tokens(parent, vocab, seed, "acc", k)
    g = synth.geometric(0.25, seed, "acc", k, kind)
    lg, path = synth.planted_logits(tokens, parent, vocab, g, seed, "acc", k, kind)
    arg, _ = oracle.argmax(lg)
    a, b, got_path = oracle.accept(tokens, parent, arg)
    ea, eb, epath = _brute_force_accept(tokens, parent, np.argmax(lg, axis=1))
    assert (a, b) == (ea, eb)
    assert list(got_path[: a + 1]) == epath and np.all(got_path[a + 1:] == -1)
    if kind == "chain":                      # closed form for a planted chain
        assert a == min(g, k - 1)
        assert list(got_path[: a + 1]) == list(range(a + 1))
        assert b == int(np.argmax(lg[a]))
    else:
        assert a >= min(g, len(path) - 1)    # the planted path is accepted at least this far


def test_geometric_law_mean():
    draws = [synth.geometric(0.3, "gl", i) for i in range(20000)]
    assert abs(np.mean(draws) - 0.7 / 0.3) < 0.06
    assert min(draws) == 0


def test_random_tree_shape():
    for seed in range(20):
        p = synth.random_tree(64, 10, seed)
        depth = oracle.tree_depth(p)
        assert depth is not None and depth.max() == 10
        assert all(depth[i] <= depth[i + 1] for i in range(63))        # breadth-first ids
        assert all(depth[p[i]] == depth[i] - 1 for i in range(1, 64))


def test_accept_equal_depth_tie_takes_lowest_node_id():
    """Duplicate sibling tokens can accept two nodes at the same depth; the lower id wins."""
    parent = np.array([-1, 0, 0, 1, 2], np.int32)      # two branches of depth 2
    tokens = np.array([7, 5, 5, 9, 9], np.int32)       # nodes 1 and 2 (and 3 and 4) duplicate
    arg = np.array([5, 9, 9, 1, 2], np.int32)
    assert oracle.accept(tokens, parent, arg)[:2] == (2, 1)
    assert list(oracle.accept(tokens, parent, arg)[2][:3]) == [0, 1, 3]
    assert _brute_force_accept(tokens, parent, arg)[2] == [0, 1, 3]
    arg2 = np.array([5, 9, 9, 1, 4], np.int32)
    parent2 = np.array([-1, 0, 0, 2, 1], np.int32)     # deeper node 3 under the higher id
    a, b, path = oracle.accept(tokens, parent2, arg2)
    assert (a, b, list(path[:3])) == (2, 1, [0, 2, 3])
