"""The lossless 12-bit weight path (W12) on the GPU, through the C ABI.

W12 is lossless, so a pass over W12 weights must give exactly what the same pass over the bf16
weights gives: the packed layout is checked against the oracle's definition of the format, the
projection kernel's partial sums against the bf16 kernel's bit for bit, and whole verify passes
against both the bf16 GPU pass with the same launch plan (one kernel per step, the plan W12 runs;
bit for bit) and the CPU oracle (the usual tolerance and exact acceptance)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tree_verification_skinny_amd as tv

from helpers import (bits, check_accept, check_logits, make_kv, oracle_model_from, run_verify,
                     tiny_case, upload_context)
from test_gpu_parity import planted_tree

pytestmark = pytest.mark.gpu
DEV = "cuda"
U32 = 2.0 ** -24


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tv.lib()


def with_exceptions(w: torch.Tensor, seed, frac=0.01, big=9.5) -> torch.Tensor:
    """A copy with a share of the values moved outside the window that holds the N(0, 0.02)
    rest: zeros, +-big, tiny normals and subnormals."""
    w = w.clone()
    g = torch.Generator().manual_seed(synth.seed_of(seed, "exc") % (1 << 62))
    n = w.numel()
    idx = torch.randperm(n, generator=g)[:max(1, int(n * frac))]
    kinds = torch.randint(0, 4, (idx.numel(),), generator=g)
    vals = torch.tensor([0.0, big, 1e-30, -3e-39], dtype=torch.float32)[kinds]
    vals = vals * torch.where(torch.rand(idx.numel(), generator=g) < 0.5, -1.0, 1.0)
    flat = w.view(-1)
    flat[idx.to(w.device)] = vals.to(torch.bfloat16).to(w.device)
    return w


def unpack_w12(m: tv.W12Matrix) -> oracle.W12:
    """The logical planes and exception list of a W12 matrix, read back from the layout the
    header documents (fragment order, 12 bytes per slot: two dwords of low bytes, one of
    nibbles)."""
    n, kd = m.n, m.kd
    S, T = kd // 32, n // 16
    plan = m.plan.cpu().numpy()
    words = m.planes.cpu().numpy().view(np.uint32).reshape(T, S, 64, 3).transpose(0, 1, 3, 2)
    lo = np.empty((n, kd), np.uint8)
    nib = np.empty((n, kd), np.uint8)
    lane = np.arange(64)
    rows = (np.arange(T)[:, None, None] * 16 + (lane % 16)[None, None, :])          # [T][1][64]
    cols0 = (np.arange(S)[None, :, None] * 32 + 8 * (lane // 16)[None, None, :])    # [1][S][64]
    rows = np.broadcast_to(rows, (T, S, 64))
    cols0 = np.broadcast_to(cols0, (T, S, 64))
    for j in range(8):
        word = words[:, :, 0 if j < 4 else 1, :]
        lo[rows, cols0 + j] = (word >> np.uint32(8 * (j % 4))) & np.uint32(0xFF)
        sh = 16 + 4 * (j >> 1) if j & 1 else 4 * (j >> 1)
        nib[rows, cols0 + j] = (words[:, :, 2, :] >> np.uint32(sh)) & np.uint32(0xF)
    exc = m.exc.cpu().numpy()[:2 * m.n_exc].reshape(-1, 2)
    offs = plan[2:2 + T + 1]
    assert offs[0] == 0 and offs[-1] == m.n_exc == plan[1] and np.all(np.diff(offs) >= 0)
    idx = np.empty(m.n_exc, np.int64)
    for t in range(T):
        e = exc[offs[t]:offs[t + 1]]
        pos = e[:, 0].astype(np.int64)
        assert np.all(np.diff(pos) > 0)                 # sorted by position within the tile
        s, l, j = pos >> 9, (pos >> 3) & 63, pos & 7
        assert np.all(s < S)
        idx[offs[t]:offs[t + 1]] = (16 * t + l % 16) * kd + 32 * s + 8 * (l // 16) + j
    order = np.argsort(idx)
    return oracle.W12(int(plan[0]), lo.reshape(-1), nib.reshape(-1), idx[order],
                      (exc[:, 1][order] & 0xFFFF).astype(np.uint16))


@pytest.mark.parametrize("n,kd,frac", [(64, 256, 0.0), (64, 256, 0.01), (1408, 256, 0.002),
                                       (32, 17408, 0.0005)])
def test_w12_layout_matches_oracle_definition(n, kd, frac):
    w = synth.randn_bf16((n, kd), 0.02, DEV, "w12l", n, kd)
    if frac:
        w = with_exceptions(w, (n, kd), frac)
    m = tv.W12Matrix(w)
    torch.cuda.synchronize()
    wb = bits(w.cpu()).reshape(-1)
    ref = oracle.w12_encode(wb)
    got = unpack_w12(m)
    assert got.base == ref.base == oracle.w12_base(wb)
    np.testing.assert_array_equal(got.esc_idx, ref.esc_idx)
    np.testing.assert_array_equal(got.esc_val, ref.esc_val)
    np.testing.assert_array_equal(got.lo, ref.lo)
    np.testing.assert_array_equal(got.nib, ref.nib)
    np.testing.assert_array_equal(oracle.w12_decode(got), wb)
    assert m.planes.numel() == n * kd * 3 // 2


@pytest.mark.parametrize("m,n,kd,frac", [(16, 7168, 5120, 0.0), (16, 5120, 17408, 1e-4),
                                         (16, 5120, 5120, 0.01), (1, 34816, 5120, 0.0),
                                         (8, 1408, 256, 0.02), (7, 512, 256, 0.3), (3, 64, 32, 0.5),
                                         (16, 1024, 8192, 0.05), (5, 2048, 4096, 0.2)])
def test_w12_gemm_bit_identical_to_bf16(m, n, kd, frac):
    """Includes K splits that start thousands of exceptions into a tile (the cursor search)."""
    x = synth.randn_bf16((m, kd), 1.0, DEV, "w12x", m, n, kd)
    w = synth.randn_bf16((n, kd), 0.02, DEV, "w12w", m, n, kd)
    if frac:
        w = with_exceptions(w, (m, n, kd), frac)
    q = tv.W12Matrix(w)
    nb = tv.spec_skinny_gemm_bytes(m, n, kd)
    p16 = torch.full((nb // 4,), float("nan"), device=DEV)
    p12 = torch.full((nb // 4,), float("nan"), device=DEV)
    s16 = tv.spec_skinny_gemm(x, tv.spec_pack_weight(w), p16)
    s12 = tv.spec_skinny_gemm_w12(x, q, p12)
    torch.cuda.synchronize()
    assert s16 == s12
    a, b = p16[:s16 * m * n], p12[:s12 * m * n]
    assert torch.equal(a.view(torch.int32), b.view(torch.int32)), \
        (q.n_exc, (a - b).abs().max().item())


@pytest.mark.parametrize("m,n,kd", [(17, 1024, 2048), (40, 7168, 5120), (64, 5120, 17408), (33, 64, 96)])
def test_w12_gemm_many_rows_bit_identical_to_bf16(m, n, kd):
    """17..64 rows: both formats run the wide kernel (or the skinny one where N does not split
    into its 128-column groups) with the same plan, so the partials agree bit for bit; they also
    meet the classical fp32 summation bound against float64."""
    x = synth.randn_bf16((m, kd), 1.0, DEV, "w12xm", m, n)
    w = with_exceptions(synth.randn_bf16((n, kd), 0.02, DEV, "w12wm", m, n), (m, n), 0.001)
    q = tv.W12Matrix(w)
    nb = tv.spec_skinny_gemm_bytes(m, n, kd)
    p16 = torch.full((nb // 4,), float("nan"), device=DEV)
    part = torch.full((nb // 4,), float("nan"), device=DEV)
    s16 = tv.spec_skinny_gemm(x, tv.spec_pack_weight(w), p16)
    s = tv.spec_skinny_gemm_w12(x, q, part)
    torch.cuda.synchronize()
    assert s == s16
    assert torch.equal(p16[:s * m * n].view(torch.int32), part[:s * m * n].view(torch.int32))
    p = part[:s * m * n].view(s, m, n).cpu().numpy()
    y = p[0].copy()
    for i in range(1, s):
        y += p[i]
    xf = x.float().cpu().numpy().astype(np.float64)
    wf = w.float().cpu().numpy().astype(np.float64)
    ref = xf @ wf.T
    gamma = kd * U32 / (1 - kd * U32)
    bound = gamma * (np.abs(xf) @ np.abs(wf).T) + s * U32 * np.abs(ref)
    assert np.all(np.abs(y - ref) <= bound)


def tiny_weights(w: dict, w12: bool) -> tv.Weights:
    dev = {k: w[k].to(DEV) for k in ("embed", "final_norm", "lm_head")}
    layers = [{k: v.to(DEV) for k, v in lw.items()} for lw in w["layers"]]
    return tv.Weights(tv.ModelCfg.of(synth.TINY), dev["embed"], dev["final_norm"], dev["lm_head"],
                      layers, w12=w12)


def test_w12_tiny_block_equals_bf16_and_oracle():
    near = 0
    for seed in range(12):
        w, m, kc, vc, tokens, G = tiny_case(seed)
        if seed % 3 == 1:              # exceptions in every projection and the output head
            w = dict(w)
            w["lm_head"] = with_exceptions(w["lm_head"], (seed, "lm"), 0.01, big=0.5)
            w["layers"] = [{k: (with_exceptions(v, (seed, l, k), 0.01, big=0.5) if k.startswith("w_") else v)
                            for k, v in lw.items()} for l, lw in enumerate(w["layers"])]
            m = oracle_model_from(synth.TINY, w)
        k = tokens.size
        r = oracle.verify(m, kc, vc, tokens)
        outs = []
        for fmt in (False, True):
            kv = make_kv(synth.TINY, [128], k, seed, DEV)
            upload_context(kv, 0, kc, vc)
            outs.append(run_verify(tiny_weights(w, fmt), kv, tokens[None], None, [128], path="steps"))
        b16, b12 = outs
        assert np.array_equal(b16.logits.view(np.int32), b12.logits.view(np.int32)), seed
        assert np.array_equal(b16.greedy, b12.greedy)
        assert (b16.accepted_len[0], b16.bonus[0]) == (b12.accepted_len[0], b12.bonus[0])
        assert np.array_equal(b16.path, b12.path)
        check_logits(b12.logits[0], r.logits, f"seed {seed} logits")
        near += check_accept(r, tokens, None, b12.greedy[0], int(b12.accepted_len[0]),
                             int(b12.bonus[0]), b12.path[0])
    assert near <= 3


@pytest.mark.parametrize("k", [12, 40, 64])
def test_w12_tiny_tree_equals_bf16_and_oracle(k):
    """Trees of 12 (skinny kernel) and 40 or 64 nodes (wide kernel): the W12 pass is
    bit-identical to the bf16 pass and meets the oracle."""
    near = 0
    for seed in range(3):
        w = synth.model_weights(synth.TINY, 900 + seed)
        m = oracle_model_from(synth.TINY, w)
        ctx = 50 + 41 * seed
        ctxs = [synth.kv_context(synth.TINY, ctx, seed, l) for l in range(2)]
        kc = [np.ascontiguousarray(bits(x)) for x, _ in ctxs]
        vc = [np.ascontiguousarray(bits(y)) for _, y in ctxs]
        tokens, parent = planted_tree(m, kc, vc, k, seed)
        r = oracle.verify(m, kc, vc, tokens, parent)
        outs = []
        for fmt in (False, True):
            kv = make_kv(synth.TINY, [ctx], k, seed, DEV)
            upload_context(kv, 0, kc, vc)
            outs.append(run_verify(tiny_weights(w, fmt), kv, tokens[None], parent[None], [ctx], path="steps"))
        b16, out = outs
        assert np.array_equal(b16.logits.view(np.int32), out.logits.view(np.int32)), seed
        assert np.array_equal(b16.path, out.path) and np.array_equal(b16.greedy, out.greedy)
        check_logits(out.logits[0], r.logits)
        near += check_accept(r, tokens, parent, out.greedy[0], int(out.accepted_len[0]),
                             int(out.bonus[0]), out.path[0])
    assert near <= 1


def test_w12_root_only_pass_equals_bf16():
    """A one-node pass (k = 1: the root alone, M = 1 row) over W12 and over bf16."""
    w, m, kc, vc, tokens, G = tiny_case(5)
    outs = []
    for fmt in (False, True):
        kv = make_kv(synth.TINY, [128], 1, 5, DEV)
        upload_context(kv, 0, kc, vc)
        outs.append(run_verify(tiny_weights(w, fmt), kv, tokens[None, :1], None, [128], path="steps"))
    assert np.array_equal(outs[0].logits.view(np.int32), outs[1].logits.view(np.int32))
    assert outs[0].accepted_len[0] == outs[1].accepted_len[0] == 0
    assert outs[0].bonus[0] == outs[1].bonus[0]


@pytest.mark.parametrize("m,n,kd", [(130, 1024, 512), (200, 384, 96)])
def test_w12_gemm_beyond_128_rows_in_chunks(m, n, kd):
    """From 128 rows the W12 projection runs 64-row chunks (the wide or skinny kernel per chunk)
    where bf16 switches to its matrix-core tile kernel: checked against float64 within the fp32
    summation bound, with exceptions planted."""
    x = synth.randn_bf16((m, kd), 1.0, DEV, "w12xc", m, n)
    w = with_exceptions(synth.randn_bf16((n, kd), 0.02, DEV, "w12wc", m, n), (m, n, "c"), 0.01)
    q = tv.W12Matrix(w)
    part = torch.full((tv.spec_skinny_gemm_bytes(m, n, kd) // 4,), float("nan"), device=DEV)
    s = tv.spec_skinny_gemm_w12(x, q, part)
    torch.cuda.synchronize()
    p = part[:s * m * n].view(s, m, n).cpu().numpy()
    y = p[0].copy()
    for i in range(1, s):
        y += p[i]
    xf = x.float().cpu().numpy().astype(np.float64)
    wf = w.float().cpu().numpy().astype(np.float64)
    ref = xf @ wf.T
    gamma = kd * U32 / (1 - kd * U32)
    bound = gamma * (np.abs(xf) @ np.abs(wf).T) + s * U32 * np.abs(ref)
    assert np.all(np.abs(y - ref) <= bound)
