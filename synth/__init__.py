"""Seeded synthetic inputs for the verification step: model weights, committed KV contexts,
draft blocks and trees, planted logits.

This module only draws numbers and places them; it holds none of the method's arithmetic
(no norm, projection, attention, argmax or acceptance). The CPU oracle and the HIP library both
consume what it makes. Every draw comes from a ``torch.Generator`` seeded by a stable hash of
(base seed, tensor name, layer), so a tensor is reproducible on its own without generating the
ones before it.

Shapes: the pages fix no model; the two shapes used are a tiny decoder (2 layers, hidden 256,
4 q / 2 kv heads of dim 64, MLP 704, vocab 1024) and a 27B-class dense decoder (64 layers,
hidden 5120, 40 q / 8 kv heads of dim 128, MLP 17408, vocab 151936). Linear and embedding
weights ~ N(0, 0.02) rounded to bf16; RMSNorm gains 1.0; context K/V ~ N(0, 1) bf16.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, replace
from typing import Dict, List, Optional, Tuple

import numpy as np
import torch


@dataclass(frozen=True)
class Shape:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float = 1e-6
    rope_theta: float = 1e4

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    def layer_shapes(self) -> Dict[str, Tuple[int, ...]]:
        H, F, d = self.hidden, self.ffn, self.head_dim
        return {
            "attn_norm": (H,),
            "w_qkv": (self.qkv_rows, H),
            "w_o": (H, self.n_q_heads * d),
            "mlp_norm": (H,),
            "w_gate_up": (2 * F, H),
            "w_down": (H, F),
        }

    def layer_params(self) -> int:
        return sum(int(np.prod(s)) for s in self.layer_shapes().values())

    def with_layers(self, n: int) -> "Shape":
        return replace(self, n_layers=n)

    def with_vocab(self, v: int) -> "Shape":
        return replace(self, vocab=v)


TINY = Shape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=704, vocab=1024)
DENSE_27B = Shape(n_layers=64, hidden=5120, n_q_heads=40, n_kv_heads=8, head_dim=128, ffn=17408,
                  vocab=151936)

LAYER_KEYS = ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate_up", "w_down")


def seed_of(*parts) -> int:
    """Stable 63-bit seed from any printable parts."""
    h = hashlib.blake2b("/".join(str(p) for p in parts).encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(*parts))
    return g


def randn_bf16(shape, std: float, device, *parts) -> torch.Tensor:
    """N(0, std^2) drawn in fp32 from a generator on ``device``, rounded to bf16 (RNE)."""
    g = _gen(device, *parts)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch.bfloat16)


def layer_weights(shape: Shape, seed: int, layer: int, device="cpu", std: float = 0.02):
    out = {}
    for name, shp in shape.layer_shapes().items():
        if name.endswith("norm"):
            out[name] = torch.ones(shp, dtype=torch.bfloat16, device=device)
        else:
            out[name] = randn_bf16(shp, std, device, seed, "layer", layer, name)
    return out


def model_weights(shape: Shape, seed: int, device="cpu", std: float = 0.02,
                  layers: Optional[int] = None):
    """dict with 'embed' [V][H], 'final_norm' [H], 'lm_head' [V][H], 'layers' (list of dicts)."""
    n = shape.n_layers if layers is None else layers
    return {
        "embed": randn_bf16((shape.vocab, shape.hidden), std, device, seed, "embed"),
        "final_norm": torch.ones(shape.hidden, dtype=torch.bfloat16, device=device),
        "lm_head": randn_bf16((shape.vocab, shape.hidden), std, device, seed, "lm_head"),
        "layers": [layer_weights(shape, seed, l, device, std) for l in range(n)],
    }


# A hybrid target: the tiny shape with 4 layers, attention and recurrent layers alternating.
HYBRID_TINY = TINY.with_layers(4)
HYBRID_KINDS = (0, 1, 0, 1)          # 0: attention layer, 1: recurrent layer


def rec_layer_weights(shape: Shape, seed: int, layer: int, device="cpu", std: float = 0.02,
                      gate_std: float = 0.2, pad16: bool = False):
    """A recurrent layer's weights: w_qkv has 3 nh d q/k/v rows (nh = n_q_heads, d = head_dim)
    ~ N(0, std^2) and nh gate rows ~ N(0, gate_std^2) (with a unit-RMS operand the gate input then
    spreads over about +-6, decays from ~1 to ~e^-6 per token); with pad16 zero rows follow up to
    a multiple of 16 (the packed layout). The other matrices as an attention layer's."""
    H, F, nh, d = shape.hidden, shape.ffn, shape.n_q_heads, shape.head_dim
    out = {}
    for name, shp in shape.layer_shapes().items():
        if name.endswith("norm"):
            out[name] = torch.ones(shp, dtype=torch.bfloat16, device=device)
        elif name == "w_qkv":
            qkv = randn_bf16((3 * nh * d, H), std, device, seed, "rec_layer", layer, "w_qkv")
            gate = randn_bf16((nh, H), gate_std, device, seed, "rec_layer", layer, "w_gate")
            rows = [qkv, gate]
            n = 3 * nh * d + nh
            if pad16 and n % 16:
                rows.append(torch.zeros((16 - n % 16, H), dtype=torch.bfloat16, device=device))
            out[name] = torch.cat(rows, 0)
        else:
            out[name] = randn_bf16(shp, std, device, seed, "rec_layer", layer, name)
    return out


def rec_state(shape: Shape, seed: int, layer: int, requests: int = 1, device="cpu"):
    """Committed state of a recurrent layer, fp32 [requests][nh][d][d] ~ N(0, 1/4)."""
    g = _gen(device, seed, "rec_layer_state", layer)
    nh, d = shape.n_q_heads, shape.head_dim
    return torch.randn((requests, nh, d, d), generator=g, device=device, dtype=torch.float32).mul_(0.5)


def kv_context(shape: Shape, ctx: int, seed: int, layer: int, device="cpu", request: int = 0):
    """Committed K and V for one layer of one request: [ctx][n_kv][head_dim], N(0, 1) bf16."""
    s = (ctx, shape.n_kv_heads, shape.head_dim)
    return (randn_bf16(s, 1.0, device, seed, "kctx", request, layer),
            randn_bf16(s, 1.0, device, seed, "vctx", request, layer))


def uniform_tokens(n: int, vocab: int, seed, *parts) -> np.ndarray:
    g = _gen("cpu", seed, "tokens", *parts)
    return torch.randint(0, vocab, (n,), generator=g, dtype=torch.int64).numpy().astype(np.int32)


def geometric(p: float, seed, *parts) -> int:
    """G in {0, 1, 2, ...} with P(G = g) = (1 - p)^g p (failures before the first success)."""
    rng = np.random.default_rng(seed_of(seed, "geom", *parts))
    return int(rng.geometric(p)) - 1


def other_token(tok: int, vocab: int, seed, *parts) -> int:
    """A token drawn uniformly from the vocab - 1 values other than ``tok``."""
    rng = np.random.default_rng(seed_of(seed, "other", *parts))
    r = int(rng.integers(0, vocab - 1))
    return r if r < tok else r + 1


def random_tree(k: int, max_depth: int, seed, *parts) -> np.ndarray:
    """Parent array of a k-node draft tree (node 0 the root, parent -1) with depth <= max_depth.

    The k - 1 non-root nodes are split over depths 1..D, D = min(max_depth, k - 1), by a uniform
    random composition (D - 1 distinct cut points among 1..k-2), so every depth holds at least
    one node. Node ids run level by level (breadth-first), and each node's parent is drawn
    uniformly among the nodes one level up."""
    rng = np.random.default_rng(seed_of(seed, "tree", *parts))
    parent = np.full(k, -1, dtype=np.int32)
    if k == 1:
        return parent
    D = min(max_depth, k - 1)
    cuts = np.sort(rng.choice(np.arange(1, k - 1), size=D - 1, replace=False)) if D > 1 else []
    bounds = [0] + list(cuts) + [k - 1]
    sizes = [int(bounds[i + 1] - bounds[i]) for i in range(D)]
    prev = [0]
    nxt = 1
    for s in sizes:
        level = list(range(nxt, nxt + s))
        for node in level:
            parent[node] = prev[int(rng.integers(0, len(prev)))]
        prev = level
        nxt += s
    return parent


def tree_tokens(parent: np.ndarray, vocab: int, seed, *parts) -> np.ndarray:
    """Uniform random tokens for a draft tree, distinct among the children of any one node."""
    rng = np.random.default_rng(seed_of(seed, "treetok", *parts))
    k = parent.size
    tok = np.empty(k, np.int32)
    used: Dict[int, set] = {}
    for i in range(k):
        s = used.setdefault(int(parent[i]), set())
        while True:
            t = int(rng.integers(0, vocab))
            if t not in s:
                break
        s.add(t)
        tok[i] = t
    return tok


def planted_logits(tokens: np.ndarray, parent: np.ndarray, vocab: int, g: int, seed, *parts):
    """fp32 [k][vocab] logits whose greedy choices accept the draft along one root path for g
    steps and then stop.

    Base values N(0, 1). The accepted path is node 0 -> the deepest chain of first children (for
    a chain block: nodes 0..k-1). On the path's first g parent rows the child's token is planted
    at row max + 0.5; on the next path row (if any) the next node's token is forced below that
    row's maximum, so acceptance stops there. Returns (logits, path_nodes)."""
    gen = _gen("cpu", seed, "planted", *parts)
    lg = torch.randn((tokens.size, vocab), generator=gen, dtype=torch.float32).numpy()
    k = tokens.size
    first_child = {}
    for i in range(1, k):
        first_child.setdefault(int(parent[i]), i)
    path = [0]
    while path[-1] in first_child:
        path.append(first_child[path[-1]])
    for step in range(len(path) - 1):
        row, child = path[step], path[step + 1]
        t = int(tokens[child])
        if step < g:
            lg[row, t] = lg[row].max() + 0.5
        else:
            others = np.delete(lg[row], t)
            lg[row, t] = others.max() - 0.5
            break
    return lg, np.array(path, np.int32)


def page_table(n_requests: int, pages_per_request: List[int], seed, shuffle: bool = True):
    """Block table [B][max_pages] (-1 padded) over a pool of sum(pages) pages, the pool order
    randomly permuted when ``shuffle``. Returns (table, n_pages)."""
    total = int(sum(pages_per_request))
    ids = np.arange(total, dtype=np.int32)
    if shuffle:
        np.random.default_rng(seed_of(seed, "pages")).shuffle(ids)
    mp = max(pages_per_request)
    table = np.full((n_requests, mp), -1, dtype=np.int32)
    o = 0
    for b, n in enumerate(pages_per_request):
        table[b, :n] = ids[o:o + n]
        o += n
    return table, total


def rec_inputs(B: int, K: int, H: int, dk: int, dv: int, seed, device="cpu", *parts):
    """Seeded inputs of a recurrent layer's tree pass: state S0 fp32 [B][H][dk][dv] ~ N(0, 1/4);
    q, k bf16 [B][K][H][dk] ~ N(0, 1/dk); v bf16 [B][K][H][dv] ~ N(0, 1); log-gates g fp32
    [B][K][H] ~ U(log 0.6, 0), i.e. per-token decays between 0.6 and 1."""
    gs = _gen(device, seed, "rec_state", *parts)
    S0 = torch.randn((B, H, dk, dv), generator=gs, device=device, dtype=torch.float32).mul_(0.5)
    q = randn_bf16((B, K, H, dk), dk ** -0.5, device, seed, "rec_q", *parts)
    k = randn_bf16((B, K, H, dk), dk ** -0.5, device, seed, "rec_k", *parts)
    v = randn_bf16((B, K, H, dv), 1.0, device, seed, "rec_v", *parts)
    gg = _gen(device, seed, "rec_gate", *parts)
    g = torch.rand((B, K, H), generator=gg, device=device, dtype=torch.float32).mul_(float(np.log(0.6)))
    return S0, q, k, v, g
