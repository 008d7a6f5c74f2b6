"""No step of spec_verify reads workspace memory that the same call has not written: each launch
plan runs once over a workspace filled with 0xFF bytes (NaN in every float slot, -1 in every
integer slot, NaN bf16) and once over a zeroed one, and every output must be bit-identical
(logits, greedy tokens, accepted lengths, bonus tokens, paths, the per-layer residual stream).
Plans: the per-step skinny kernels (a block of 8), the persistent kernel (same block), a 13-node
tree, the wide kernels (4 x 16 rows), the tile kernels (32 x 16 rows), W12 weights, a hybrid
target."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tree_verification_skinny_amd as tv

from helpers import device_weights, make_kv, run_verify
from test_gpu_hybrid import build as hybrid_build

pytestmark = pytest.mark.gpu
DEV = "cuda"


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tv.lib()


def _same(a, b, what):
    for name in ("logits", "greedy", "accepted_len", "bonus", "path"):
        x, y = getattr(a, name), getattr(b, name)
        assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8)), f"{what}: {name} differs"
    if a.hidden is not None:
        assert torch.equal(a.hidden.view(torch.int16), b.hidden.view(torch.int16)), f"{what}: hidden differs"


def _fill_context(kv, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    kv.k_pool.normal_(generator=g)
    kv.v_pool.normal_(generator=g)


@pytest.mark.parametrize("case", ["block-steps", "block-persistent", "tree", "wide", "tile", "w12"])
def test_poisoned_workspace_changes_nothing(case):
    shape = synth.TINY
    w = synth.model_weights(shape, 88)
    weights = (tv.Weights(tv.ModelCfg.of(shape), w["embed"].to(DEV), w["final_norm"].to(DEV), w["lm_head"].to(DEV),
                          [{k: v.to(DEV) for k, v in lw.items()} for lw in w["layers"]], w12=True)
               if case == "w12" else device_weights(shape, w, DEV))
    path = "persistent" if case == "block-persistent" else "steps"
    if case in ("block-steps", "block-persistent", "w12"):
        B, k, parent = 1, 8, None
    elif case == "tree":
        B, k = 1, 13
        parent = synth.random_tree(k, 5, 88, "poison")[None]
    elif case == "wide":
        B, k, parent = 4, 16, None
    else:
        B, k, parent = 32, 16, None
    rng = np.random.default_rng(88)
    ctxs = [int(c) for c in rng.integers(1, 300, B)]
    kv = make_kv(shape, ctxs, k, 88, DEV)
    _fill_context(kv, 88)
    tokens = np.stack([synth.uniform_tokens(k, shape.vocab, 88, case, b) for b in range(B)]).astype(np.int32)
    print(f"case {case}: B={B} k={k}", flush=True)
    outs = [run_verify(weights, kv, tokens, parent, ctxs, want_hidden=True, path=path, ws_fill=fill)
            for fill in (0xFF, 0x00)]
    _same(outs[0], outs[1], case)
    assert np.isfinite(outs[0].logits).all()


def test_poisoned_workspace_hybrid():
    c = hybrid_build(89, [17, 40], 8)
    tokens = np.stack([synth.uniform_tokens(8, synth.HYBRID_TINY.vocab, 89, "hp", b) for b in range(2)]).astype(np.int32)
    outs = [run_verify(c.weights, c.kv, tokens, None, c.ctxs, want_hidden=True, ws_fill=fill) for fill in (0xFF, 0x00)]
    _same(outs[0], outs[1], "hybrid")
    assert np.isfinite(outs[0].logits).all()
