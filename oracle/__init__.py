"""CPU oracle for the verification step of lossless greedy speculative decoding.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package. The product library never loads it, and the two share
no code: the arithmetic lives in ``specverify_oracle.c`` (plain C, fp32 sums in index order,
bf16 storage points) and this module only marshals numpy arrays into it and sequences the
steps of the definition:

* verify: one target pass over a block or tree of draft tokens, then the greedy acceptance
  walk. A drafter's tokens are all checked in one pass [JetSpec article, seventnews.com —
  opening section]; tree tokens are conditioned on their own path [JetSpec article —
  "Technical architecture"]; every accepted token is the target's greedy choice
  [SpecPilot digest, airadar.tv — "Risks"].
* ar_greedy: plain one-token-at-a-time greedy decoding, the result verification must equal.
* commit: the accepted path's K/V rows appended to the committed context.
* rec_tree / rec_commit: a recurrent layer of a hybrid target verified over a draft tree (every
  node continues its parent's state) and its state after acceptance; the recurrence is a
  reading, since the pages only name tree verification for such targets [SpecPilot digest,
  airadar.tv — "Reasons"].

Arrays: bf16 tensors travel as ``numpy.uint16`` bit patterns. K/V caches are per layer,
``[positions][n_kv][head_dim]``.

Parity status: every function here is pinned by ``tests/test_oracle_*.py`` against float64
references, library routines, closed forms and brute force; see each test's docstring.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Callable, List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "specverify_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_i32p = ctypes.POINTER(ctypes.c_int32)


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                               "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Cfg(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int), ("hidden", ctypes.c_int), ("n_q_heads", ctypes.c_int),
                ("n_kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int), ("ffn", ctypes.c_int),
                ("vocab", ctypes.c_int), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_double)]


class _LayerW(ctypes.Structure):
    _fields_ = [(n, _u16p) for n in ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate_up", "w_down")]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        L.orc_max_threads.restype = ctypes.c_int
        L.orc_set_threads.argtypes = [ctypes.c_int]
        _u8p = ctypes.POINTER(ctypes.c_uint8)
        _i64p = ctypes.POINTER(ctypes.c_int64)
        L.orc_w12_base.argtypes = [_u16p, ctypes.c_int64]
        L.orc_w12_base.restype = ctypes.c_int
        L.orc_w12_encode.argtypes = [_u16p, ctypes.c_int64, ctypes.c_int, _u8p, _u8p, _u8p]
        L.orc_w12_encode.restype = ctypes.c_int64
        L.orc_w12_decode.argtypes = [_u8p, _u8p, ctypes.c_int64, ctypes.c_int, _i64p, _u16p,
                                     ctypes.c_int64, _u16p]
        L.orc_f32_to_bf16.argtypes = [_f32p, _u16p, ctypes.c_int64]
        L.orc_bf16_to_f32.argtypes = [_u16p, _f32p, ctypes.c_int64]
        L.orc_tree_depth.argtypes = [_i32p, ctypes.c_int, _i32p]
        L.orc_tree_depth.restype = ctypes.c_int
        L.orc_rmsnorm.argtypes = [_u16p, _u16p, ctypes.c_int, ctypes.c_int, ctypes.c_float, _u16p]
        L.orc_linear.argtypes = [_u16p, ctypes.c_int, ctypes.c_int, _u16p, ctypes.c_int, _f32p]
        L.orc_rope.argtypes = [_u16p, _i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double]
        L.orc_attention.argtypes = [_u16p, _u16p, _u16p, ctypes.c_int, _u16p, _u16p, _i32p,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _u16p]
        L.orc_swiglu.argtypes = [_u16p, _u16p, ctypes.c_int64, _u16p]
        L.orc_layer_forward.argtypes = [ctypes.POINTER(_Cfg), ctypes.POINTER(_LayerW), _u16p, _u16p,
                                        ctypes.c_int, _i32p, ctypes.c_int, _u16p, _u16p, _u16p]
        L.orc_layer_forward.restype = ctypes.c_int
        L.orc_embed.argtypes = [_u16p, ctypes.c_int, ctypes.c_int, _i32p, ctypes.c_int, _u16p]
        L.orc_embed.restype = ctypes.c_int
        L.orc_logits.argtypes = [ctypes.POINTER(_Cfg), _u16p, _u16p, _u16p, ctypes.c_int, _f32p]
        L.orc_argmax.argtypes = [_f32p, ctypes.c_int, ctypes.c_int, _i32p, _f32p]
        L.orc_accept.argtypes = [_i32p, _i32p, _i32p, ctypes.c_int, _i32p, _i32p, _i32p]
        L.orc_accept.restype = ctypes.c_int
        _f64p = ctypes.POINTER(ctypes.c_double)
        L.orc_rec_tree.argtypes = [_f32p, _u16p, _u16p, _u16p, _f32p, _i32p, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _f64p, _i32p]
        L.orc_rec_commit.argtypes = [_f32p, _u16p, _u16p, _f32p, _i32p, _i32p, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _f64p]
        L.orc_rec_layer_forward.argtypes = [ctypes.POINTER(_Cfg), ctypes.POINTER(_LayerW), _f32p, _i32p,
                                            ctypes.c_int, _u16p, _u16p, _u16p, _f32p]
        L.orc_rec_layer_forward.restype = ctypes.c_int
        _lib = L
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _p(a: Optional[np.ndarray], ptype):
    if a is None:
        return ctypes.cast(None, ptype)
    return a.ctypes.data_as(ptype)


def threads() -> int:
    """OpenMP threads the oracle's loops use on this host."""
    return int(lib().orc_max_threads())


def set_threads(n: int) -> None:
    """Threads of the oracle's following parallel loops (for timing at one thread or all cores)."""
    lib().orc_set_threads(int(n))


# ---------------------------------------------------------------------------------------------
# bf16 helpers
# ---------------------------------------------------------------------------------------------

def to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_f32_to_bf16(_p(x, _f32p), _p(out, _u16p), x.size)
    return out


def from_bf16(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 (exact)."""
    h = _c(h, np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib().orc_bf16_to_f32(_p(h, _u16p), _p(out, _f32p), h.size)
    return out


# ---------------------------------------------------------------------------------------------
# model
# ---------------------------------------------------------------------------------------------

@dataclass
class Cfg:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float = 1e-6
    rope_theta: float = 1e4

    def c(self) -> _Cfg:
        return _Cfg(self.n_layers, self.hidden, self.n_q_heads, self.n_kv_heads, self.head_dim,
                    self.ffn, self.vocab, self.rms_eps, self.rope_theta)


LAYER_KEYS = ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate_up", "w_down")


ATTENTION, RECURRENT = 0, 1


class Model:
    """Weights as numpy uint16 (bf16 bits). ``layer_fn(l)`` returns layer l's dict, so a large
    model can be streamed one layer at a time instead of held whole. ``kinds``: per layer,
    ATTENTION (default) or RECURRENT (a hybrid target; see rec_layer_forward)."""

    def __init__(self, cfg: Cfg, embed: np.ndarray, final_norm: np.ndarray, lm_head: np.ndarray,
                 layers: Optional[Sequence[dict]] = None,
                 layer_fn: Optional[Callable[[int], dict]] = None,
                 kinds: Optional[Sequence[int]] = None):
        self.cfg = cfg
        self.kinds = [ATTENTION] * cfg.n_layers if kinds is None else [int(k) for k in kinds]
        self.embed = _c(embed, np.uint16)
        self.final_norm = _c(final_norm, np.uint16)
        self.lm_head = _c(lm_head, np.uint16)
        self._layers = None if layers is None else [
            {k: _c(v, np.uint16) for k, v in lw.items()} for lw in layers]
        self._layer_fn = layer_fn

    def layer(self, l: int) -> dict:
        if self._layers is not None:
            return self._layers[l]
        return {k: _c(v, np.uint16) for k, v in self._layer_fn(l).items()}


def _layer_struct(lw: dict) -> _LayerW:
    return _LayerW(*[_p(lw[k], _u16p) for k in LAYER_KEYS])


def tree_depth(parent: np.ndarray) -> Optional[np.ndarray]:
    parent = _c(parent, np.int32)
    depth = np.zeros(parent.shape, dtype=np.int32)
    rc = lib().orc_tree_depth(_p(parent, _i32p), parent.size, _p(depth, _i32p))
    return None if rc != 0 else depth


def chain(k: int) -> np.ndarray:
    """Parent array of a linear block: node i's parent is node i - 1."""
    return np.arange(-1, k - 1, dtype=np.int32)


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    x = _c(x, np.uint16)
    g = _c(g, np.uint16)
    rows, h = x.reshape(-1, x.shape[-1]).shape
    out = np.empty_like(x)
    lib().orc_rmsnorm(_p(x, _u16p), _p(g, _u16p), rows, h, eps, _p(out, _u16p))
    return out


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """fp32 [m][n] = x [m][kd] . w[n][kd]^T (bf16 operands)."""
    x = _c(x, np.uint16)
    w = _c(w, np.uint16)
    m, kd = x.shape
    n = w.shape[0]
    assert w.shape[1] == kd
    y = np.empty((m, n), dtype=np.float32)
    lib().orc_linear(_p(x, _u16p), m, kd, _p(w, _u16p), n, _p(y, _f32p))
    return y


def rope(t: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half RoPE of t [m][nh][d] (bf16 bits) at positions pos [m]; returns a copy."""
    t = np.array(t, dtype=np.uint16, copy=True, order="C")
    pos = _c(pos, np.int32)
    m, nh, d = t.shape
    lib().orc_rope(_p(t, _u16p), _p(pos, _i32p), m, nh, d, theta)
    return t


def attention(q, k_ctx, v_ctx, k_new, v_new, parent) -> np.ndarray:
    """q [m][nq][d]; k_ctx/v_ctx [ctx][nkv][d]; k_new/v_new [m][nkv][d]; parent [m]."""
    q = _c(q, np.uint16)
    m, nq, d = q.shape
    nkv = k_new.shape[1]
    k_ctx = _c(k_ctx, np.uint16).reshape(-1, nkv, d)
    v_ctx = _c(v_ctx, np.uint16).reshape(-1, nkv, d)
    k_new = _c(k_new, np.uint16)
    v_new = _c(v_new, np.uint16)
    parent = _c(parent, np.int32)
    o = np.empty_like(q)
    lib().orc_attention(_p(q, _u16p), _p(k_ctx, _u16p), _p(v_ctx, _u16p), k_ctx.shape[0],
                        _p(k_new, _u16p), _p(v_new, _u16p), _p(parent, _i32p), m, nq, nkv, d,
                        _p(o, _u16p))
    return o


def swiglu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    gate = _c(gate, np.uint16)
    up = _c(up, np.uint16)
    out = np.empty_like(gate)
    lib().orc_swiglu(_p(gate, _u16p), _p(up, _u16p), gate.size, _p(out, _u16p))
    return out


def embed(model: Model, tokens: np.ndarray) -> np.ndarray:
    tokens = _c(tokens, np.int32)
    x = np.empty((tokens.size, model.cfg.hidden), dtype=np.uint16)
    rc = lib().orc_embed(_p(model.embed, _u16p), model.cfg.vocab, model.cfg.hidden,
                         _p(tokens, _i32p), tokens.size, _p(x, _u16p))
    if rc != 0:
        raise ValueError("token out of range")
    return x


def layer_forward(cfg: Cfg, lw: dict, k_ctx: np.ndarray, v_ctx: np.ndarray, parent: np.ndarray,
                  x: np.ndarray):
    """One decoder layer over the m nodes of a draft tree. Returns (x_out, k_new, v_new)."""
    nkv, d = cfg.n_kv_heads, cfg.head_dim
    k_ctx = _c(k_ctx, np.uint16).reshape(-1, nkv, d)
    v_ctx = _c(v_ctx, np.uint16).reshape(-1, nkv, d)
    parent = _c(parent, np.int32)
    x = np.array(x, dtype=np.uint16, copy=True, order="C")
    m = x.shape[0]
    k_new = np.empty((m, nkv, d), dtype=np.uint16)
    v_new = np.empty((m, nkv, d), dtype=np.uint16)
    c = cfg.c()
    s = _layer_struct(lw)
    rc = lib().orc_layer_forward(ctypes.byref(c), ctypes.byref(s), _p(k_ctx, _u16p),
                                 _p(v_ctx, _u16p), k_ctx.shape[0], _p(parent, _i32p), m,
                                 _p(x, _u16p), _p(k_new, _u16p), _p(v_new, _u16p))
    if rc != 0:
        raise ValueError("malformed draft tree")
    return x, k_new, v_new


def rec_layer_forward(cfg: Cfg, lw: dict, S0: np.ndarray, parent: np.ndarray, x: np.ndarray):
    """One recurrent layer of a hybrid target over the m nodes of a draft tree (the reading is
    written out in specverify_oracle.c): lw["w_qkv"] holds 3 nh d + nh rows (q, k, v heads, then
    one gate row per head; nh = n_q_heads), S0 the committed state fp32 [nh][d][d]. Returns
    (x_out, k [m][nh][d] bf16 bits, v [m][nh][d], g [m][nh] fp32 log-gates)."""
    nh, d = cfg.n_q_heads, cfg.head_dim
    S0 = _c(S0, np.float32).reshape(nh, d, d)
    parent = _c(parent, np.int32)
    x = np.array(x, dtype=np.uint16, copy=True, order="C")
    m = x.shape[0]
    k = np.empty((m, nh, d), np.uint16)
    v = np.empty((m, nh, d), np.uint16)
    g = np.empty((m, nh), np.float32)
    c = cfg.c()
    s = _layer_struct(lw)
    rc = lib().orc_rec_layer_forward(ctypes.byref(c), ctypes.byref(s), _p(S0, _f32p), _p(parent, _i32p), m,
                                     _p(x, _u16p), _p(k, _u16p), _p(v, _u16p), _p(g, _f32p))
    if rc != 0:
        raise ValueError("malformed draft tree")
    return x, k, v, g


def logits(model: Model, x: np.ndarray) -> np.ndarray:
    x = _c(x, np.uint16)
    m = x.shape[0]
    out = np.empty((m, model.cfg.vocab), dtype=np.float32)
    c = model.cfg.c()
    lib().orc_logits(ctypes.byref(c), _p(model.final_norm, _u16p), _p(model.lm_head, _u16p),
                     _p(x, _u16p), m, _p(out, _f32p))
    return out


def argmax(lg: np.ndarray):
    """Lowest index of each row's maximum, and the top-1 minus top-2 margin."""
    lg = _c(lg, np.float32)
    m, v = lg.shape
    arg = np.empty(m, dtype=np.int32)
    margin = np.empty(m, dtype=np.float32)
    lib().orc_argmax(_p(lg, _f32p), m, v, _p(arg, _i32p), _p(margin, _f32p))
    return arg, margin


def accept(tokens: np.ndarray, parent: np.ndarray, arg: np.ndarray):
    """Greedy acceptance walk. Returns (accepted_len, bonus, path[k]); -1s for a bad tree."""
    tokens = _c(tokens, np.int32)
    parent = _c(parent, np.int32)
    arg = _c(arg, np.int32)
    k = tokens.size
    a = np.zeros(1, np.int32)
    b = np.zeros(1, np.int32)
    path = np.empty(k, np.int32)
    lib().orc_accept(_p(tokens, _i32p), _p(parent, _i32p), _p(arg, _i32p), k, _p(a, _i32p),
                     _p(b, _i32p), _p(path, _i32p))
    return int(a[0]), int(b[0]), path


# ---------------------------------------------------------------------------------------------
# whole steps
# ---------------------------------------------------------------------------------------------

@dataclass
class VerifyResult:
    logits: np.ndarray          # fp32 [k][vocab]
    arg: np.ndarray             # int32 [k]
    margin: np.ndarray          # fp32 [k]
    accepted_len: int
    bonus: int
    path: np.ndarray            # int32 [k], -1 after the end
    k_new: List[np.ndarray]     # per layer [k][nkv][d] (recurrent layers: [k][nh][d])
    v_new: List[np.ndarray]
    hidden: List[np.ndarray]    # residual stream entering each layer, and after the last
    g_new: Optional[List] = None   # per layer: recurrent log-gates [k][nh] fp32, else None


def verify(model: Model, k_ctx: Sequence[np.ndarray], v_ctx: Sequence[np.ndarray],
           tokens: np.ndarray, parent: Optional[np.ndarray] = None,
           keep_hidden: bool = False, state: Optional[Sequence] = None) -> VerifyResult:
    """One verification pass of one request: the draft tree (node 0 = root, the last committed
    token) scored in one target pass over the committed context, then the acceptance walk.
    ``k_ctx[l]``/``v_ctx[l]``: layer l's committed cache [ctx][nkv][d]; for a recurrent layer
    of a hybrid target ``state[l]`` is its committed state fp32 [nh][d][d] instead."""
    cfg = model.cfg
    tokens = _c(tokens, np.int32)
    parent = chain(tokens.size) if parent is None else _c(parent, np.int32)
    x = embed(model, tokens)
    hidden = [x.copy()] if keep_hidden else []
    k_new, v_new, g_new = [], [], []
    for l in range(cfg.n_layers):
        if model.kinds[l] == RECURRENT:
            x, kn, vn, gn = rec_layer_forward(cfg, model.layer(l), state[l], parent, x)
        else:
            x, kn, vn = layer_forward(cfg, model.layer(l), k_ctx[l], v_ctx[l], parent, x)
            gn = None
        k_new.append(kn)
        v_new.append(vn)
        g_new.append(gn)
        if keep_hidden:
            hidden.append(x.copy())
    lg = logits(model, x)
    arg, margin = argmax(lg)
    a, b, path = accept(tokens, parent, arg)
    return VerifyResult(lg, arg, margin, a, b, path, k_new, v_new, hidden, g_new)


def prefill(model: Model, prompt: np.ndarray, k_ctx=None, v_ctx=None):
    """Run the prompt through the target as a chain over an (optionally empty) cache. Returns
    the new caches (committed context plus the prompt) and the last row's fp32 logits."""
    cfg = model.cfg
    nkv, d = cfg.n_kv_heads, cfg.head_dim
    if k_ctx is None:
        k_ctx = [np.zeros((0, nkv, d), np.uint16) for _ in range(cfg.n_layers)]
        v_ctx = [np.zeros((0, nkv, d), np.uint16) for _ in range(cfg.n_layers)]
    r = verify(model, k_ctx, v_ctx, prompt, chain(len(prompt)))
    k_out = [np.concatenate([k_ctx[l], r.k_new[l]], 0) for l in range(cfg.n_layers)]
    v_out = [np.concatenate([v_ctx[l], r.v_new[l]], 0) for l in range(cfg.n_layers)]
    return k_out, v_out, r.logits[-1]


def commit(k_ctx, v_ctx, r: VerifyResult):
    """Append the accepted path's K/V rows (root first) to each attention layer's committed
    cache (a recurrent layer's cache, which holds no rows, is left as it is; see commit_rec)."""
    if r.accepted_len < 0:
        return list(k_ctx), list(v_ctx)
    sel = r.path[: r.accepted_len + 1]
    rec = [r.g_new is not None and r.g_new[l] is not None for l in range(len(k_ctx))]
    k_out = [k_ctx[l] if rec[l] else np.concatenate([k_ctx[l], r.k_new[l][sel]], 0) for l in range(len(k_ctx))]
    v_out = [v_ctx[l] if rec[l] else np.concatenate([v_ctx[l], r.v_new[l][sel]], 0) for l in range(len(v_ctx))]
    return k_out, v_out


def commit_rec(model: Model, state: Sequence, r: VerifyResult) -> list:
    """Each recurrent layer's committed state after the accepted path (root first) of ``r``,
    stored in fp32 as the state is kept between passes; unchanged for a failed request (None
    for attention layers)."""
    out = []
    K = r.path.size
    al = np.array([r.accepted_len], np.int32)
    ap = np.array(r.path, np.int32).reshape(1, K)
    for l in range(model.cfg.n_layers):
        if model.kinds[l] != RECURRENT:
            out.append(None)
            continue
        nh, d = model.cfg.n_q_heads, model.cfg.head_dim
        S0 = _c(state[l], np.float32).reshape(1, nh, d, d)
        S = rec_commit(S0, r.k_new[l][None], r.v_new[l][None], r.g_new[l][None], al, ap)
        out.append(S[0].astype(np.float32))
    return out


def ar_greedy_hybrid(model: Model, k_ctx, v_ctx, state, first_token: int, n: int):
    """Greedy decoding of a hybrid target one token per pass, each pass committing its token:
    the K/V row of every attention layer, the fp32 state of every recurrent layer. Returns the n
    greedy tokens after ``first_token``, the logits of each pass, and the caches and states."""
    toks, lgs = [], []
    tok = int(first_token)
    k_ctx, v_ctx, state = list(k_ctx), list(v_ctx), list(state)
    for _ in range(n):
        r = verify(model, k_ctx, v_ctx, np.array([tok], np.int32), np.array([-1], np.int32), state=state)
        st = commit_rec(model, state, r)
        for l in range(model.cfg.n_layers):
            if model.kinds[l] == RECURRENT:
                state[l] = st[l]
            else:
                k_ctx[l] = np.concatenate([k_ctx[l], r.k_new[l]], 0)
                v_ctx[l] = np.concatenate([v_ctx[l], r.v_new[l]], 0)
        lgs.append(r.logits[0])
        tok = int(r.arg[0])
        toks.append(tok)
    return np.array(toks, np.int32), np.stack(lgs), k_ctx, v_ctx, state


def ar_greedy(model: Model, k_ctx, v_ctx, first_token: int, n: int):
    """Plain greedy decoding: feed ``first_token`` (whose K/V is not cached yet), then each
    greedy choice in turn, one token per pass. Returns the n greedy tokens that follow
    ``first_token``, the logits of each pass, and the caches after the n passes."""
    toks, lgs = [], []
    tok = int(first_token)
    k_ctx, v_ctx = list(k_ctx), list(v_ctx)
    for _ in range(n):
        r = verify(model, k_ctx, v_ctx, np.array([tok], np.int32), np.array([-1], np.int32))
        k_ctx = [np.concatenate([k_ctx[l], r.k_new[l]], 0) for l in range(len(k_ctx))]
        v_ctx = [np.concatenate([v_ctx[l], r.v_new[l]], 0) for l in range(len(v_ctx))]
        lgs.append(r.logits[0])
        tok = int(r.arg[0])
        toks.append(tok)
    return np.array(toks, np.int32), np.stack(lgs), k_ctx, v_ctx


# ---- W12: lossless 12-bit weight storage ---------------------------------------------------------
# The SpecPilot digest (airadar.tv — "Reasons") names a lossless 12-bit format that splits each
# bf16 weight into three 4-bit planes reassembled in the GEMM's registers. The reading (the planes'
# contents, the per-matrix exponent window, the exception list) is written out in
# specverify_oracle.c.

@dataclass
class W12:
    base: int                 # even exponent-window base b: fields b..b+15 fit
    lo: np.ndarray            # uint8 [n]: planes 1 and 0 (the value's low byte)
    nib: np.ndarray           # uint8 [n]: plane 2, (sign, (e - b) >> 1); 0 for an exception
    esc_idx: np.ndarray       # int64 [n_esc]: flat indices of the exceptions, ascending
    esc_val: np.ndarray       # uint16 [n_esc]: their bf16 bit patterns


def w12_base(w: np.ndarray) -> int:
    w = _c(w.reshape(-1), np.uint16)
    return int(lib().orc_w12_base(_p(w, _u16p), w.size))


def w12_encode(w: np.ndarray, base: Optional[int] = None) -> W12:
    """Planes and exception list of a bf16 array (uint16 bit patterns), flattened in C order."""
    w = _c(w.reshape(-1), np.uint16)
    b = w12_base(w) if base is None else int(base)
    u8 = ctypes.POINTER(ctypes.c_uint8)
    lo = np.empty(w.size, np.uint8)
    nib = np.empty(w.size, np.uint8)
    esc = np.empty(w.size, np.uint8)
    lib().orc_w12_encode(_p(w, _u16p), w.size, b, lo.ctypes.data_as(u8), nib.ctypes.data_as(u8),
                         esc.ctypes.data_as(u8))
    idx = np.flatnonzero(esc).astype(np.int64)
    return W12(b, lo, nib, idx, w[idx].copy())


def w12_decode(c: W12) -> np.ndarray:
    """The bf16 bit patterns (flat, uint16) the planes and exceptions stand for."""
    u8 = ctypes.POINTER(ctypes.c_uint8)
    lo = _c(c.lo, np.uint8)
    nib = _c(c.nib, np.uint8)
    idx = _c(c.esc_idx, np.int64)
    val = _c(c.esc_val, np.uint16)
    out = np.empty(lo.size, np.uint16)
    lib().orc_w12_decode(lo.ctypes.data_as(u8), nib.ctypes.data_as(u8), lo.size, c.base,
                         idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _p(val, _u16p), idx.size,
                         _p(out, _u16p))
    return out


# ---------------------------------------------------------------------------------------------
# recurrent layers of a hybrid target
# ---------------------------------------------------------------------------------------------
# Reading (the pages name tree verification for targets with recurrent layers [SpecPilot digest,
# airadar.tv — "Reasons"] but give no recurrence): per head, a scalar-gated linear recurrence
# S <- exp(g) S + k v^T, o = S^T q, the node's state continuing its parent's, the root's the
# committed state. Computed by walking each node's root path token by token, in float64.

def rec_tree(S0: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray,
             parent: Optional[np.ndarray]):
    """Outputs [B][K][H][dv] (float64) and status [B] (1 = malformed tree, outputs zero).

    S0 fp32 [B][H][dk][dv]; q, k bf16 bits [B][K][H][dk]; v bf16 bits [B][K][H][dv];
    g fp32 [B][K][H]; parent int32 [B][K] or None for chains."""
    B, H, dk, dv = S0.shape
    K = q.shape[1]
    S0 = _c(S0, np.float32)
    q, k, v = _c(q, np.uint16), _c(k, np.uint16), _c(v, np.uint16)
    g = _c(g, np.float32)
    par = None if parent is None else _c(parent, np.int32)
    out = np.empty((B, K, H, dv), np.float64)
    st = np.empty(B, np.int32)
    f64 = ctypes.POINTER(ctypes.c_double)
    lib().orc_rec_tree(_p(S0, _f32p), _p(q, _u16p), _p(k, _u16p), _p(v, _u16p), _p(g, _f32p),
                       _p(par, _i32p), B, K, H, dk, dv, out.ctypes.data_as(f64), _p(st, _i32p))
    return out, st


def rec_commit(S0: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray,
               accepted_len: np.ndarray, accepted_path: np.ndarray) -> np.ndarray:
    """State [B][H][dk][dv] (float64) after the accepted root path; S0 for a request with
    accepted_len < 0 or >= K, or a path node id outside [0, K)."""
    B, H, dk, dv = S0.shape
    K = k.shape[1]
    S0 = _c(S0, np.float32)
    k, v = _c(k, np.uint16), _c(v, np.uint16)
    g = _c(g, np.float32)
    al = _c(accepted_len, np.int32)
    ap = _c(accepted_path, np.int32)
    out = np.empty((B, H, dk, dv), np.float64)
    lib().orc_rec_commit(_p(S0, _f32p), _p(k, _u16p), _p(v, _u16p), _p(g, _f32p), _p(al, _i32p),
                         _p(ap, _i32p), B, K, H, dk, dv, out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    return out
