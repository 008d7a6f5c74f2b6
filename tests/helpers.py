"""Shared test plumbing: seeded cases, moving tensors between the oracle (numpy bf16 bits) and
the HIP library (torch device tensors), and the parity rules.

Parity rules (the tolerance is the one the target states; the near-tie rule follows the pages'
caveat that a different order of computation may invert near-ties [SpecPilot digest,
airadar.tv — "Risks"]):
  * logits: |gpu - oracle| <= 2e-2 + 1e-2 |oracle| for every element;
  * greedy token per node: equal wherever the oracle's top-2 margin is >= 1e-2;
  * acceptance: the GPU's (accepted_len, bonus, path) equals the oracle walk applied to the
    GPU's own greedy tokens, and equals the oracle's result outright unless a node of the
    oracle's accepted set has margin < 1e-2 (a logged near-tie).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth
import tree_verification_skinny_amd as tv
from tree_verification_skinny_amd import kvlayout

ATOL, RTOL, NEAR_TIE = 2e-2, 1e-2, 1e-2
# check_as_exact: how much farther from the exact (float64) evaluation than the oracle the GPU may
# be. The GPU's blocked sums keep it closer to the exact values than the oracle's sequential ones
# on the 27B block (0.1x to 1.1x by layer); planted kernel mistakes (a dropped K step, wrong RoPE
# pairs or position, swapped kv heads, a 1 % softmax scale error) measure far more
# (tests/test_oracle_27b_criterion.py).
EXACT_FACTOR = 1.25


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def from_bits(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def oracle_cfg(shape: synth.Shape) -> oracle.Cfg:
    return oracle.Cfg(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads,
                      shape.head_dim, shape.ffn, shape.vocab, shape.rms_eps, shape.rope_theta)


def oracle_model_from(shape: synth.Shape, w: dict) -> oracle.Model:
    layers = [{k: bits(v) for k, v in lw.items()} for lw in w["layers"]]
    return oracle.Model(oracle_cfg(shape), bits(w["embed"]), bits(w["final_norm"]),
                        bits(w["lm_head"]), layers)


def device_weights(shape: synth.Shape, w: dict, device) -> tv.Weights:
    dev = {k: w[k].to(device) for k in ("embed", "final_norm", "lm_head")}
    layers = [{k: v.to(device) for k, v in lw.items()} for lw in w["layers"]]
    return tv.Weights(tv.ModelCfg.of(shape), dev["embed"], dev["final_norm"], dev["lm_head"], layers)


def pages_for(ctx_lens, k, extra_pages=0):
    return [int((c + k + 15) // 16) + extra_pages for c in ctx_lens]


def make_kv(shape: synth.Shape, ctx_lens, k, seed, device, shuffle=True, extra_pages=0):
    table, n_pages = synth.page_table(len(ctx_lens), pages_for(ctx_lens, k, extra_pages), seed,
                                      shuffle=shuffle)
    return tv.PagedKV.empty(tv.ModelCfg.of(shape), n_pages, torch.from_numpy(table), device)


def upload_context(kv: tv.PagedKV, b: int, k_ctx, v_ctx):
    """k_ctx/v_ctx: per layer numpy bf16 bits [ctx][nkv][d]."""
    dev = kv.k_pool.device
    for l in range(len(k_ctx)):
        if k_ctx[l].shape[0]:
            kvlayout.write_context(kv, l, b, from_bits(k_ctx[l], dev), from_bits(v_ctx[l], dev))


class VerifyOut:
    pass


def run_verify(weights: tv.Weights, kv: tv.PagedKV, tokens: np.ndarray, parent, ctx_lens,
               want_hidden=False, want_logits=True, path: str = "auto", ws_fill=None):
    """tokens [B][K] int32; parent [B][K] or None. Returns numpy outputs. ws_fill: a byte
    value written over the whole workspace first (e.g. 0xFF: NaN floats, -1 integers)."""
    dev = kv.k_pool.device
    B, K = tokens.shape
    cfg = weights.cfg
    M = B * K
    ws = tv.workspace(tv.spec_workspace_bytes(cfg, B, K, kv.max_pages), dev)
    if ws_fill is not None:
        ws.fill_(ws_fill)
    t_tok = torch.from_numpy(np.ascontiguousarray(tokens, np.int32)).to(dev)
    t_par = None if parent is None else torch.from_numpy(np.ascontiguousarray(parent, np.int32)).to(dev)
    t_ctx = torch.tensor(list(ctx_lens), dtype=torch.int32, device=dev)
    acc = torch.full((B,), -7, dtype=torch.int32, device=dev)
    bonus = torch.full((B,), -7, dtype=torch.int32, device=dev)
    path_t = torch.full((B, K), -7, dtype=torch.int32, device=dev)
    greedy = torch.full((M,), -7, dtype=torch.int32, device=dev)
    logits = torch.full((M, cfg.vocab), float("nan"), device=dev) if want_logits else None
    hidden = (torch.empty((cfg.n_layers + 1, M, cfg.hidden), dtype=torch.bfloat16, device=dev)
              if want_hidden else None)
    tv.spec_verify(weights, kv, t_tok, t_par, t_ctx, B, K, acc, bonus, path_t, ws, logits=logits,
                   greedy=greedy, hidden=hidden, path=path)
    torch.cuda.synchronize()
    o = VerifyOut()
    o.accepted_len = acc.cpu().numpy()
    o.bonus = bonus.cpu().numpy()
    o.path = path_t.cpu().numpy()
    o.greedy = greedy.cpu().numpy().reshape(B, K)
    o.logits = None if logits is None else logits.cpu().numpy().reshape(B, K, cfg.vocab)
    o.hidden = None if hidden is None else hidden
    o.ctx = t_ctx
    o.acc_t, o.path_t = acc, path_t
    return o


def check_logits(gpu: np.ndarray, orc: np.ndarray, what: str = "logits"):
    err = np.abs(gpu.astype(np.float64) - orc.astype(np.float64))
    lim = ATOL + RTOL * np.abs(orc.astype(np.float64))
    bad = err > lim
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; "
                           f"max err {err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}")
    return float(err.max())


def bf16_ulp(v: float) -> float:
    """Spacing of bf16 values (8 significant bits) at magnitude v."""
    v = abs(float(v))
    if v < 2.0 ** -126:
        return 2.0 ** -133
    return 2.0 ** (np.floor(np.log2(v)) - 7)


def check_as_exact(gpu, orc, ref, what: str = "", factor: float = EXACT_FACTOR):
    """Parity where summation order alone exceeds the fixed tolerance (the 27B-class shape with
    random weights: an exact float64 evaluation of the same model and storage points already
    differs from the oracle by more than 2e-2 + 1e-2|x| in a few elements). Both the GPU and the
    oracle are fp32 evaluations of the same storage points, so each is measured against the exact
    one: the GPU's max and mean deviation from it, and its share of elements outside the fixed
    tolerance around it, must be within `factor` of the oracle's. (Measured against the oracle
    instead, a correct GPU inherits the oracle's own rounding on top of its own, up to sqrt(2)
    times the exact evaluation's distance, so no tight factor holds there.) The max of bf16
    outputs moves in whole ULPs of the largest elements (one rounding flip at magnitude 64 turns
    0.25 into 0.5), so it may exceed `factor` times the oracle's by one bf16 ULP of the worst
    element's own magnitude; mean and out-of-tolerance share carry no such slack."""
    ref = np.asarray(ref, np.float64)
    orc = np.asarray(orc, np.float64)
    eg = np.abs(np.asarray(gpu, np.float64) - ref)
    eo = np.abs(orc - ref)
    lim = ATOL + RTOL * np.abs(ref)
    fg, fo = float(np.mean(eg > lim)), float(np.mean(eo > lim))
    d = np.abs(np.asarray(gpu, np.float64) - orc)
    msg = (f"{what}: gpu-vs-exact max {eg.max():.3e} mean {eg.mean():.3e} out-of-tol {fg:.4f}; "
           f"oracle-vs-exact max {eo.max():.3e} mean {eo.mean():.3e} out-of-tol {fo:.4f}; "
           f"gpu-vs-oracle max {d.max():.3e} mean {d.mean():.3e}")
    worst = float(np.abs(ref.reshape(-1)[int(np.argmax(eg))]))
    assert eg.max() <= factor * max(eo.max(), 1e-6) + bf16_ulp(worst), msg
    assert eg.mean() <= factor * max(eo.mean(), 1e-7), msg
    assert fg <= factor * fo + 1e-3, msg
    return msg


def check_accept(r: oracle.VerifyResult, tokens, parent, gpu_greedy, gpu_a, gpu_b, gpu_path,
                 near_tie: float = NEAR_TIE):
    """Returns True when the case was a logged near-tie (compared loosely), else False.
    `near_tie` is the top-2 margin below which a flipped greedy choice is a near-tie inversion;
    it is 1e-2 except where the exact evaluation itself moves logits by more (see
    check_as_exact), where it is EXACT_FACTOR times that movement."""
    k = len(tokens)
    par = oracle.chain(k) if parent is None else np.asarray(parent, np.int32)
    firm = r.margin >= near_tie
    assert np.array_equal(gpu_greedy[firm], r.arg[firm]), (
        f"greedy differs at firm nodes {np.nonzero((gpu_greedy != r.arg) & firm)[0]}")
    a2, b2, p2 = oracle.accept(tokens, par, gpu_greedy)
    assert (gpu_a, gpu_b) == (a2, b2) and np.array_equal(gpu_path, p2), "walk inconsistent"
    accepted = [i for i in range(k) if i == 0 or _on_accepted(i, tokens, par, r.arg)]
    near = any(r.margin[i] < near_tie for i in accepted)
    if not near:
        assert (gpu_a, gpu_b) == (r.accepted_len, r.bonus)
        assert np.array_equal(gpu_path, r.path)
    return near


def _on_accepted(i, tokens, par, arg):
    node = i
    while node > 0:
        if tokens[node] != arg[par[node]]:
            return False
        node = par[node]
    return True


def tiny_case(seed: int, k: int = 8, p: float = 0.3, prompt_len: int = 128):
    """Tiny decoder, prompt prefilled by the oracle, draft = oracle greedy continuation with one
    token replaced at position 1 + G, G ~ Geometric(p) on {0, 1, ...} (no replacement when
    1 + G >= k). Returns (weights dict, oracle model, k_ctx, v_ctx, tokens, G)."""
    shape = synth.TINY
    w = synth.model_weights(shape, seed)
    m = oracle_model_from(shape, w)
    prompt = synth.uniform_tokens(prompt_len, shape.vocab, seed, "prompt")
    kc, vc, last = oracle.prefill(m, prompt)
    g1 = int(np.argmax(last))
    cont, _, _, _ = oracle.ar_greedy(m, kc, vc, g1, k - 1)
    tokens = np.concatenate([[g1], cont]).astype(np.int32)
    G = synth.geometric(p, seed, "replace")
    if 1 + G < k:
        tokens[1 + G] = synth.other_token(int(tokens[1 + G]), shape.vocab, seed, "replace")
    return w, m, kc, vc, tokens, G
