"""Python binding of libspecverify, the MI355X (gfx950) verification step of lossless greedy
speculative decoding.

Argument marshalling only: every step of the pass runs in the library's HIP kernels, called
through its C ABI (``include/specverify.h``) with ``ctypes``. PyTorch supplies device memory
and the current HIP stream. There is no fallback: if the built library is missing, importing
the entry points raises.

Entry points (same names as the C ABI): ``spec_workspace_bytes``, ``spec_verify``,
``spec_commit_kv``, ``spec_accept_workspace_bytes``, ``spec_accept``,
``spec_pack_weight``, ``spec_skinny_gemm_bytes``, ``spec_skinny_gemm``, ``spec_strerror``.

``Weights`` takes row-major bf16 tensors and packs the projection matrices once
(``spec_pack_weight``) into buffers it owns; ``Weights.from_packed`` takes matrices already
packed.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SPEC_OK = 0
SPEC_EINVAL = -1
SPEC_EUNSUPPORTED = -2
SPEC_EWORKSPACE = -3
SPEC_EHIP = -4
SPEC_ESCRATCH = -5
SPEC_NOALLOC_MAX_ROWS = 4096
SPEC_NOALLOC_MAX_VOCAB = 262144
PAGE_SIZE = 16
MAX_K = 64
LAYER_KEYS = ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate_up", "w_down")


class SpecError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {spec_strerror(code)} ({code})")
        self.code = code


class ModelCfgC(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int), ("hidden", ctypes.c_int), ("n_q_heads", ctypes.c_int),
                ("n_kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int), ("ffn", ctypes.c_int),
                ("vocab", ctypes.c_int), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_double)]


class LayerWeightsC(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in LAYER_KEYS]


class W12MatrixC(ctypes.Structure):
    _fields_ = [("planes", ctypes.c_void_p), ("plan", ctypes.c_void_p), ("exc", ctypes.c_void_p)]


class W12LayerC(ctypes.Structure):
    _fields_ = [(k, W12MatrixC) for k in ("w_qkv", "w_o", "w_gate_up", "w_down")]


class WeightsC(ctypes.Structure):
    _fields_ = [("cfg", ModelCfgC), ("layers", ctypes.POINTER(LayerWeightsC)),
                ("embed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("lm_head", ctypes.c_void_p), ("w12_layers", ctypes.POINTER(W12LayerC)),
                ("w12_lm_head", W12MatrixC), ("layer_kind", ctypes.c_void_p)]


class KVCacheC(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("n_pages", ctypes.c_int),
                ("max_pages_per_req", ctypes.c_int), ("rec_state", ctypes.c_void_p),
                ("rec_k", ctypes.c_void_p), ("rec_v", ctypes.c_void_p), ("rec_g", ctypes.c_void_p)]


class ExtrasC(ctypes.Structure):
    _fields_ = [("logits", ctypes.c_void_p), ("greedy", ctypes.c_void_p), ("hidden", ctypes.c_void_p),
                ("gate_up_events", ctypes.c_void_p), ("path", ctypes.c_int),
                ("layer_events", ctypes.c_void_p), ("phase_trace", ctypes.c_void_p)]


SPEC_PATH_AUTO, SPEC_PATH_STEPS, SPEC_PATH_PERSISTENT = 0, 1, 2
PATHS = {"auto": SPEC_PATH_AUTO, "steps": SPEC_PATH_STEPS, "persistent": SPEC_PATH_PERSISTENT}


_lib = None


def lib() -> ctypes.CDLL:
    """Load the built library (fails loudly when it is absent)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                              "python tree_verification_skinny_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.spec_strerror.argtypes = [i32]
        L.spec_strerror.restype = ctypes.c_char_p
        L.spec_workspace_bytes.argtypes = [ctypes.POINTER(ModelCfgC), i32, i32, i32, ctypes.POINTER(sz)]
        L.spec_verify.argtypes = [ctypes.POINTER(WeightsC), ctypes.POINTER(KVCacheC), vp, vp, vp, i32, i32,
                                  vp, vp, vp, ctypes.POINTER(ExtrasC), vp, sz, vp]
        L.spec_commit_kv.argtypes = [ctypes.POINTER(ModelCfgC), ctypes.POINTER(KVCacheC), vp, vp, vp,
                                     i32, i32, vp]
        L.spec_accept_workspace_bytes.argtypes = [i32, i32, i32, ctypes.POINTER(sz)]
        L.spec_accept.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
        L.spec_accept_noalloc.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp]
        L.spec_pack_weight.argtypes = [vp, i32, i32, vp, vp]
        L.spec_skinny_gemm_bytes.argtypes = [i32, i32, i32, ctypes.POINTER(sz)]
        L.spec_skinny_gemm.argtypes = [vp, i32, i32, vp, i32, vp, sz, ctypes.POINTER(i32), vp]
        L.spec_read_probe.argtypes = [vp, sz, vp, vp]
        L.spec_w12_plan_ints.argtypes = [i32, i32, ctypes.POINTER(sz)]
        L.spec_w12_plan.argtypes = [vp, i32, i32, vp, vp]
        L.spec_w12_pack.argtypes = [vp, i32, i32, vp, vp, vp, vp]
        L.spec_skinny_gemm_w12.argtypes = [vp, i32, i32, ctypes.POINTER(W12MatrixC), i32, vp, sz,
                                           ctypes.POINTER(i32), vp]
        L.spec_prefill_workspace_bytes.argtypes = [ctypes.POINTER(ModelCfgC), i32, i32, i32,
                                                   ctypes.POINTER(sz)]
        L.spec_prefill.argtypes = [ctypes.POINTER(WeightsC), ctypes.POINTER(KVCacheC), vp, vp, i32, i32,
                                   vp, vp, vp, sz, vp]
        L.spec_rec_tree_verify.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp]
        L.spec_rec_commit.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp]
        for f in (L.spec_prefill_workspace_bytes, L.spec_prefill, L.spec_rec_tree_verify,
                  L.spec_rec_commit, L.spec_accept_noalloc):
            f.restype = i32
        for f in (L.spec_workspace_bytes, L.spec_verify, L.spec_commit_kv,
                  L.spec_accept_workspace_bytes, L.spec_accept, L.spec_skinny_gemm_bytes,
                  L.spec_skinny_gemm, L.spec_pack_weight, L.spec_read_probe, L.spec_w12_plan_ints,
                  L.spec_w12_plan, L.spec_w12_pack, L.spec_skinny_gemm_w12):
            f.restype = i32
        _lib = L
    return _lib


EXPORTED = ("spec_workspace_bytes", "spec_verify", "spec_commit_kv", "spec_accept_workspace_bytes",
            "spec_accept", "spec_pack_weight", "spec_skinny_gemm_bytes", "spec_skinny_gemm",
            "spec_read_probe", "spec_w12_plan_ints", "spec_w12_plan", "spec_w12_pack",
            "spec_skinny_gemm_w12", "spec_prefill_workspace_bytes", "spec_prefill",
            "spec_rec_tree_verify", "spec_rec_commit", "spec_accept_noalloc", "spec_strerror")


def spec_strerror(code: int) -> str:
    return lib().spec_strerror(int(code)).decode()


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libspecverify must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, where: str):
    if rc != SPEC_OK:
        raise SpecError(rc, where)


@dataclass(frozen=True)
class ModelCfg:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float = 1e-6
    rope_theta: float = 1e4

    def c(self) -> ModelCfgC:
        return ModelCfgC(self.n_layers, self.hidden, self.n_q_heads, self.n_kv_heads, self.head_dim,
                         self.ffn, self.vocab, self.rms_eps, self.rope_theta)

    @staticmethod
    def of(shape) -> "ModelCfg":
        return ModelCfg(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads,
                        shape.head_dim, shape.ffn, shape.vocab, shape.rms_eps, shape.rope_theta)


PACKED_KEYS = ("w_qkv", "w_o", "w_gate_up", "w_down")


def spec_pack_weight(w: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Packed copy of a row-major bf16 [n][kd] projection matrix (same shape and size)."""
    if out is None:
        out = torch.empty_like(w)
    n, kd = w.shape
    _check(lib().spec_pack_weight(_ptr(w), n, kd, _ptr(out), _stream(stream)), "spec_pack_weight")
    return out


class W12Matrix:
    """One projection matrix in the library's lossless 12-bit layout (spec_w12_plan, then
    spec_w12_pack): planes (uint8, n*kd*3/2), plan (int32) and exceptions (int32 pairs)."""

    def __init__(self, w: torch.Tensor, stream=None):
        n, kd = w.shape
        ints = ctypes.c_size_t(0)
        _check(lib().spec_w12_plan_ints(n, kd, ctypes.byref(ints)), "spec_w12_plan_ints")
        self.n, self.kd = n, kd
        self.plan = torch.empty(ints.value, dtype=torch.int32, device=w.device)
        _check(lib().spec_w12_plan(_ptr(w), n, kd, _ptr(self.plan), _stream(stream)), "spec_w12_plan")
        self.n_exc = int(self.plan[1].item())          # waits for the plan
        self.exc = torch.empty(max(2 * self.n_exc, 2), dtype=torch.int32, device=w.device)
        self.planes = torch.empty(n * kd * 3 // 2, dtype=torch.uint8, device=w.device)
        _check(lib().spec_w12_pack(_ptr(w), n, kd, _ptr(self.plan), _ptr(self.planes), _ptr(self.exc),
                                   _stream(stream)), "spec_w12_pack")
        self.c = W12MatrixC(_ptr(self.planes), _ptr(self.plan), _ptr(self.exc))

    def nbytes(self) -> int:
        """Bytes a pass streams: the planes, the per-tile offsets and the exceptions."""
        return self.planes.numel() + 4 * (self.n // 16 + 1) + 8 * self.n_exc


def spec_skinny_gemm_w12(x: torch.Tensor, w: W12Matrix, partials: torch.Tensor, stream=None) -> int:
    """spec_skinny_gemm over a W12 matrix; returns the split count."""
    m, kd = x.shape
    splits = ctypes.c_int(0)
    rc = lib().spec_skinny_gemm_w12(_ptr(x), m, kd, ctypes.byref(w.c), w.n, _ptr(partials),
                                    partials.numel() * partials.element_size(), ctypes.byref(splits),
                                    _stream(stream))
    _check(rc, "spec_skinny_gemm_w12")
    return splits.value


class Weights:
    """Device weights and the C struct that points at them. The constructor takes row-major
    bf16 tensors and packs the projection matrices (and the output head) once; with
    ``drop_rowmajor`` the row-major projection tensors are released after packing. With
    ``w12`` the projections and the output head are stored in the lossless 12-bit layout
    instead (W12Matrix) and no bf16 copy of them is kept."""

    def __init__(self, cfg: ModelCfg, embed: torch.Tensor, final_norm: torch.Tensor,
                 lm_head: torch.Tensor, layers: Sequence[dict], packed: bool = False,
                 drop_rowmajor: bool = False, w12: bool = False, kinds: Optional[Sequence[int]] = None):
        if len(layers) != cfg.n_layers:
            raise ValueError("need one weight dict per layer")
        self.cfg = cfg
        # hybrid targets: SPEC_LAYER_ATTENTION / SPEC_LAYER_RECURRENT per layer (host array)
        self.kinds = None if kinds is None else (ctypes.c_int32 * cfg.n_layers)(*[int(k) for k in kinds])
        self.rowmajor = None
        self.w12 = None
        self._w12_layers = None
        w12_head = W12MatrixC(None, None, None)
        if w12:
            if packed:
                raise ValueError("W12 weights are built from row-major tensors")
            if not drop_rowmajor:
                self.rowmajor = dict(lm_head=lm_head, layers=list(layers))
            self.w12 = dict(lm_head=W12Matrix(lm_head),
                            layers=[{k: W12Matrix(lw[k]) for k in PACKED_KEYS} for lw in layers])
            self._w12_layers = (W12LayerC * cfg.n_layers)(
                *[W12LayerC(*[m[k].c for k in PACKED_KEYS]) for m in self.w12["layers"]])
            w12_head = self.w12["lm_head"].c
            lm_head = None
            layers = [{k: v for k, v in lw.items() if k not in PACKED_KEYS} for lw in layers]
        elif not packed:
            if not drop_rowmajor:
                self.rowmajor = dict(lm_head=lm_head, layers=list(layers))
            lm_head = spec_pack_weight(lm_head)
            layers = [{k: (spec_pack_weight(v) if k in PACKED_KEYS else v) for k, v in lw.items()}
                      for lw in layers]
        self.tensors = dict(embed=embed, final_norm=final_norm, lm_head=lm_head, layers=list(layers))
        self._layers = (LayerWeightsC * cfg.n_layers)(
            *[LayerWeightsC(*[_ptr(lw.get(k)) for k in LAYER_KEYS]) for lw in layers])
        w12p = (ctypes.cast(self._w12_layers, ctypes.POINTER(W12LayerC)) if self._w12_layers is not None
                else None)
        self.c = WeightsC(cfg.c(), ctypes.cast(self._layers, ctypes.POINTER(LayerWeightsC)),
                          _ptr(embed), _ptr(final_norm), _ptr(lm_head), w12p, w12_head,
                          None if self.kinds is None else ctypes.cast(self.kinds, ctypes.c_void_p))

    @staticmethod
    def from_packed(cfg: ModelCfg, embed, final_norm, lm_head_packed, layers_packed) -> "Weights":
        return Weights(cfg, embed, final_norm, lm_head_packed, layers_packed, packed=True)


class PagedKV:
    """Paged bf16 KV cache in the library's layout (see include/specverify.h):
    k_pool [L][pages][n_kv][16][d], v_pool [L][pages][n_kv][d][16], block_table [B][max_pages]."""

    def __init__(self, k_pool: torch.Tensor, v_pool: torch.Tensor, block_table: torch.Tensor):
        self.k_pool, self.v_pool = k_pool, v_pool
        self.block_table = block_table.to(torch.int32).contiguous()
        self.n_pages = k_pool.shape[1]
        self.max_pages = self.block_table.shape[1]
        self.c = KVCacheC(_ptr(k_pool), _ptr(v_pool), _ptr(self.block_table), self.n_pages, self.max_pages,
                          None, None, None, None)

    def attach_rec(self, cfg: ModelCfg, states: Sequence[Optional[torch.Tensor]], batch: int, k: int):
        """Recurrent layers of a hybrid target: ``states[l]`` layer l's committed state, fp32
        [batch][nq][d][d] with each head's S stored transposed (None for attention layers); the
        buffers spec_verify fills with each pass's keys, values and log-gates and spec_commit_kv
        applies (for this batch and k)."""
        L, nq, d = cfg.n_layers, cfg.n_q_heads, cfg.head_dim
        dev = self.k_pool.device
        self.rec_states = list(states)
        self._rec_ptrs = (ctypes.c_void_p * L)(*[_ptr(t) if t is not None else None for t in states])
        self.rec_k = torch.zeros((L, batch, k, nq, d), dtype=torch.bfloat16, device=dev)
        self.rec_v = torch.zeros((L, batch, k, nq, d), dtype=torch.bfloat16, device=dev)
        self.rec_g = torch.zeros((L, batch, k, nq), dtype=torch.float32, device=dev)
        self.c.rec_state = ctypes.cast(self._rec_ptrs, ctypes.c_void_p)
        self.c.rec_k, self.c.rec_v, self.c.rec_g = _ptr(self.rec_k), _ptr(self.rec_v), _ptr(self.rec_g)
        return self

    @staticmethod
    def empty(cfg: ModelCfg, n_pages: int, block_table: torch.Tensor, device) -> "PagedKV":
        L, nkv, d = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim
        k = torch.zeros((L, n_pages, nkv, PAGE_SIZE, d), dtype=torch.bfloat16, device=device)
        v = torch.zeros((L, n_pages, nkv, d, PAGE_SIZE), dtype=torch.bfloat16, device=device)
        return PagedKV(k, v, block_table.to(device))


def spec_workspace_bytes(cfg: ModelCfg, batch: int, k: int, max_pages_per_req: int) -> int:
    n = ctypes.c_size_t(0)
    c = cfg.c()
    _check(lib().spec_workspace_bytes(ctypes.byref(c), batch, k, max_pages_per_req, ctypes.byref(n)),
           "spec_workspace_bytes")
    return n.value


def workspace(nbytes: int, device) -> torch.Tensor:
    """A 256-byte aligned device buffer (torch's caching allocator aligns to 512 bytes)."""
    t = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    assert t.data_ptr() % 256 == 0
    return t


def spec_verify(weights: Weights, kv: PagedKV, draft_tokens: torch.Tensor,
                tree_parent: Optional[torch.Tensor], ctx_len: torch.Tensor, batch: int, k: int,
                accepted_len: torch.Tensor, bonus_token: torch.Tensor, accepted_path: torch.Tensor,
                ws: torch.Tensor, logits: Optional[torch.Tensor] = None,
                greedy: Optional[torch.Tensor] = None, hidden: Optional[torch.Tensor] = None,
                gate_up_events=None, stream=None, path: str = "auto", layer_events=None,
                phase_trace: Optional[torch.Tensor] = None) -> None:
    """gate_up_events: optional ctypes array of 2 * n_layers hipEvent_t handles (e.g. the
    cuda_event handles of torch timing events that have been recorded once), per-step path;
    layer_events: the same, 2 * ceil(n_layers / 16) handles around the persistent launches.
    path: "auto", "steps" or "persistent" (see SPEC_PATH_* in include/specverify.h);
    phase_trace: int64 device tensor [n_layers][compute units][24] (persistent path)."""
    ev = None if gate_up_events is None else ctypes.cast(gate_up_events, ctypes.c_void_p)
    lev = None if layer_events is None else ctypes.cast(layer_events, ctypes.c_void_p)
    extras = ExtrasC(_ptr(logits), _ptr(greedy), _ptr(hidden), ev, PATHS[path], lev, _ptr(phase_trace))
    rc = lib().spec_verify(ctypes.byref(weights.c), ctypes.byref(kv.c), _ptr(draft_tokens),
                           _ptr(tree_parent), _ptr(ctx_len), batch, k, _ptr(accepted_len),
                           _ptr(bonus_token), _ptr(accepted_path), ctypes.byref(extras), _ptr(ws),
                           ws.numel(), _stream(stream))
    _check(rc, "spec_verify")


def spec_prefill_workspace_bytes(cfg: ModelCfg, batch: int, max_pages_per_req: int,
                                 want_logits: bool = False) -> int:
    n = ctypes.c_size_t(0)
    c = cfg.c()
    _check(lib().spec_prefill_workspace_bytes(ctypes.byref(c), batch, max_pages_per_req,
                                              1 if want_logits else 0, ctypes.byref(n)),
           "spec_prefill_workspace_bytes")
    return n.value


def spec_prefill(weights: Weights, kv: PagedKV, prompt: torch.Tensor, ctx_len: torch.Tensor,
                 next_token: torch.Tensor, ws: torch.Tensor, last_logits: Optional[torch.Tensor] = None,
                 stream=None) -> None:
    """Appends prompt [batch][p] (int32, device) to every request's committed context; writes
    next_token [batch] and, if given, last_logits [batch][vocab]."""
    batch, p = prompt.shape
    rc = lib().spec_prefill(ctypes.byref(weights.c), ctypes.byref(kv.c), _ptr(prompt), _ptr(ctx_len),
                            batch, p, _ptr(next_token), _ptr(last_logits), _ptr(ws), ws.numel(),
                            _stream(stream))
    _check(rc, "spec_prefill")


def spec_commit_kv(cfg: ModelCfg, kv: PagedKV, accepted_len: torch.Tensor,
                   accepted_path: torch.Tensor, ctx_len: torch.Tensor, batch: int, k: int,
                   stream=None) -> None:
    c = cfg.c()
    rc = lib().spec_commit_kv(ctypes.byref(c), ctypes.byref(kv.c), _ptr(accepted_len),
                              _ptr(accepted_path), _ptr(ctx_len), batch, k, _stream(stream))
    _check(rc, "spec_commit_kv")


def spec_accept_workspace_bytes(batch: int, k: int, vocab: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().spec_accept_workspace_bytes(batch, k, vocab, ctypes.byref(n)),
           "spec_accept_workspace_bytes")
    return n.value


def spec_accept(logits: torch.Tensor, draft_tokens: torch.Tensor,
                tree_parent: Optional[torch.Tensor], batch: int, k: int, vocab: int,
                accepted_len: torch.Tensor, bonus_token: torch.Tensor,
                accepted_path: torch.Tensor, ws: torch.Tensor,
                greedy: Optional[torch.Tensor] = None, stream=None) -> None:
    rc = lib().spec_accept(_ptr(logits), _ptr(draft_tokens), _ptr(tree_parent), batch, k, vocab,
                           _ptr(accepted_len), _ptr(bonus_token), _ptr(accepted_path), _ptr(greedy),
                           _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "spec_accept")


def spec_accept_noalloc(logits: torch.Tensor, draft_tokens: torch.Tensor,
                        tree_parent: Optional[torch.Tensor], batch: int, k: int, vocab: int,
                        accepted_len: torch.Tensor, bonus_token: torch.Tensor,
                        accepted_path: torch.Tensor, greedy: Optional[torch.Tensor] = None,
                        stream=None) -> None:
    """spec_accept with the library's static per-GPU scratch instead of a workspace."""
    rc = lib().spec_accept_noalloc(_ptr(logits), _ptr(draft_tokens), _ptr(tree_parent), batch, k,
                                   vocab, _ptr(accepted_len), _ptr(bonus_token), _ptr(accepted_path),
                                   _ptr(greedy), _stream(stream))
    _check(rc, "spec_accept_noalloc")


def spec_read_probe(buf: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    """Reads all of buf (a contiguous device tensor, size a multiple of 16 bytes) once as a
    plain stream; out: a device int32/uint32 tensor of at least one element."""
    _check(lib().spec_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out),
                                 _stream(stream)), "spec_read_probe")


def spec_rec_tree_verify(state: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         log_gate: torch.Tensor, tree_parent: Optional[torch.Tensor],
                         out: torch.Tensor, status: torch.Tensor, stream=None) -> None:
    """One recurrent layer over draft trees. state fp32 [B][H][D][D], S transposed ([dv][dk]);
    q, k, v bf16 [B][K][H][D];
    log_gate fp32 [B][K][H]; tree_parent int32 [B][K] or None (chains); out fp32 [B][K][H][D];
    status int32 [B] (1 = malformed tree)."""
    B, K, H, D = q.shape
    for t in (state, q, k, v, log_gate, out, status) + ((tree_parent,) if tree_parent is not None else ()):
        if not t.is_contiguous():
            raise ValueError("spec_rec_tree_verify: tensors must be contiguous")
    if (tuple(state.shape) != (B, H, D, D) or tuple(k.shape) != (B, K, H, D) or
            tuple(v.shape) != (B, K, H, D) or tuple(log_gate.shape) != (B, K, H) or
            tuple(out.shape) != (B, K, H, D) or status.numel() < B or
            (tree_parent is not None and tuple(tree_parent.shape) != (B, K))):
        raise ValueError("spec_rec_tree_verify: shapes do not match")
    _check(lib().spec_rec_tree_verify(_ptr(state), _ptr(q), _ptr(k), _ptr(v), _ptr(log_gate),
                                      _ptr(tree_parent), B, K, H, D, _ptr(out), _ptr(status),
                                      _stream(stream)), "spec_rec_tree_verify")


def spec_rec_commit(state: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_gate: torch.Tensor,
                    accepted_len: torch.Tensor, accepted_path: torch.Tensor, stream=None) -> None:
    """The accepted node's state written over state (fp32 [B][H][D][D], S transposed) in place; k, v, log_gate
    as passed to spec_rec_tree_verify; accepted_len int32 [B], accepted_path int32 [B][K]."""
    B, K, H, D = k.shape
    for t in (state, k, v, log_gate, accepted_len, accepted_path):
        if not t.is_contiguous():
            raise ValueError("spec_rec_commit: tensors must be contiguous")
    if (tuple(state.shape) != (B, H, D, D) or tuple(v.shape) != (B, K, H, D) or
            tuple(log_gate.shape) != (B, K, H) or accepted_len.numel() < B or
            tuple(accepted_path.shape) != (B, K)):
        raise ValueError("spec_rec_commit: shapes do not match")
    _check(lib().spec_rec_commit(_ptr(state), _ptr(k), _ptr(v), _ptr(log_gate), _ptr(accepted_len),
                                 _ptr(accepted_path), B, K, H, D, _stream(stream)), "spec_rec_commit")


def spec_skinny_gemm_bytes(m: int, n: int, kd: int) -> int:
    nb = ctypes.c_size_t(0)
    _check(lib().spec_skinny_gemm_bytes(m, n, kd, ctypes.byref(nb)), "spec_skinny_gemm_bytes")
    return nb.value


def spec_skinny_gemm(x: torch.Tensor, w: torch.Tensor, partials: torch.Tensor, stream=None) -> int:
    """partials[s][m][n] for x [m][kd] (bf16, row-major), w [n][kd] (bf16, packed by
    spec_pack_weight); returns the split count."""
    m, kd = x.shape
    n = w.shape[0]
    splits = ctypes.c_int(0)
    rc = lib().spec_skinny_gemm(_ptr(x), m, kd, _ptr(w), n, _ptr(partials),
                                partials.numel() * partials.element_size(), ctypes.byref(splits),
                                _stream(stream))
    _check(rc, "spec_skinny_gemm")
    return splits.value

