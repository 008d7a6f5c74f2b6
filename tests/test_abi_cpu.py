"""The C ABI without a GPU: the library loads, exports every function include/specverify.h
declares, sizes workspaces, and rejects bad host-visible arguments before enqueueing anything
(none of these calls reaches the device)."""
import ctypes
import os
import re

import pytest

import tree_verification_skinny_amd as tv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
           if f.endswith(".h")]

TINY = tv.ModelCfg(2, 256, 4, 2, 64, 704, 1024)
D27 = tv.ModelCfg(64, 5120, 40, 8, 128, 17408, 151936)


def declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*(spec_[a-z0-9_]+)\s*\(",
                             text, flags=re.M):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"spec_verify", "spec_commit_kv", "spec_accept", "spec_workspace_bytes",
            "spec_accept_workspace_bytes", "spec_strerror"} <= names
    L = ctypes.CDLL(tv.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert set(tv.EXPORTED) == names


def test_strerror_codes():
    assert tv.spec_strerror(tv.SPEC_OK) == "ok"
    for c in (tv.SPEC_EINVAL, tv.SPEC_EUNSUPPORTED, tv.SPEC_EWORKSPACE, tv.SPEC_EHIP):
        assert tv.spec_strerror(c) not in ("ok", "unknown error")
    assert tv.spec_strerror(12345) == "unknown error"


def test_workspace_sizes_grow_with_batch_and_context():
    a = tv.spec_workspace_bytes(D27, 1, 16, 257)
    b = tv.spec_workspace_bytes(D27, 32, 16, 514)
    c = tv.spec_workspace_bytes(D27, 1, 64, 517)
    assert 0 < a < b and a < c
    assert a % 256 == 0
    assert tv.spec_workspace_bytes(TINY, 1, 8, 9) > 0


@pytest.mark.parametrize("cfg,code", [
    (tv.ModelCfg(2, 256, 4, 2, 96, 704, 1024), tv.SPEC_EUNSUPPORTED),     # head_dim 96
    (tv.ModelCfg(2, 256, 4, 3, 64, 704, 1024), tv.SPEC_EUNSUPPORTED),     # 4 q heads, 3 kv heads
    (tv.ModelCfg(2, 250, 4, 2, 64, 704, 1024), tv.SPEC_EUNSUPPORTED),     # hidden % 32
    (tv.ModelCfg(2, 256, 4, 2, 64, 700, 1024), tv.SPEC_EUNSUPPORTED),     # ffn % 32
    (tv.ModelCfg(2, 256, 4, 2, 64, 704, 1000), tv.SPEC_EUNSUPPORTED),     # vocab % 64
    (tv.ModelCfg(2, 256, 4, 2, 64, 704, 1040), tv.SPEC_EUNSUPPORTED),     # vocab % 64
    (tv.ModelCfg(2, 96, 2, 1, 64, 704, 1024), tv.SPEC_EUNSUPPORTED),      # hidden % 64
    (tv.ModelCfg(0, 256, 4, 2, 64, 704, 1024), tv.SPEC_EINVAL),
    (tv.ModelCfg(2, 256, 4, 2, 64, 704, 1024, rope_theta=-1.0), tv.SPEC_EINVAL),
])
def test_workspace_rejects_bad_shapes(cfg, code):
    with pytest.raises(tv.SpecError) as e:
        tv.spec_workspace_bytes(cfg, 1, 8, 9)
    assert e.value.code == code


def test_workspace_rejects_bad_sizes():
    for batch, k, pages, code in [(0, 8, 9, tv.SPEC_EINVAL), (1, 0, 9, tv.SPEC_EINVAL),
                                  (1, 65, 9, tv.SPEC_EUNSUPPORTED), (1, 8, 0, tv.SPEC_EINVAL)]:
        with pytest.raises(tv.SpecError) as e:
            tv.spec_workspace_bytes(TINY, batch, k, pages)
        assert e.value.code == code


def _raw_verify(weights_c, kv_c, ptrs, batch, k, ws_ptr, ws_bytes):
    L = tv.lib()
    extras = tv.ExtrasC(None, None, None)
    return L.spec_verify(ctypes.byref(weights_c) if weights_c is not None else None,
                         ctypes.byref(kv_c) if kv_c is not None else None,
                         ptrs["tok"], ptrs["par"], ptrs["ctx"], batch, k, ptrs["a"], ptrs["b"],
                         ptrs["p"], ctypes.byref(extras), ws_ptr, ws_bytes, None)


def _fake_structs(cfg, n_layers_ptrs=True):
    fake = 0x10000   # never dereferenced on the host; calls below fail validation first
    layers = (tv.LayerWeightsC * cfg.n_layers)(
        *[tv.LayerWeightsC(*([fake] * 6 if n_layers_ptrs else [fake] * 5 + [None]))
          for _ in range(cfg.n_layers)])
    w = tv.WeightsC(cfg.c(), ctypes.cast(layers, ctypes.POINTER(tv.LayerWeightsC)), fake, fake, fake)
    kv = tv.KVCacheC(fake, fake, fake, 16, 9)
    return w, kv, layers


def test_verify_rejects_host_visible_errors_without_launching():
    w, kv, keep = _fake_structs(TINY)
    fake = 0x10000
    ptrs = dict(tok=fake, par=None, ctx=fake, a=fake, b=fake, p=fake)
    need = tv.spec_workspace_bytes(TINY, 1, 8, 9)
    assert _raw_verify(None, kv, ptrs, 1, 8, 0x100000, need) == tv.SPEC_EINVAL
    assert _raw_verify(w, None, ptrs, 1, 8, 0x100000, need) == tv.SPEC_EINVAL
    for key in ("tok", "ctx", "a", "b", "p"):
        bad = dict(ptrs, **{key: None})
        assert _raw_verify(w, kv, bad, 1, 8, 0x100000, need) == tv.SPEC_EINVAL
    assert _raw_verify(w, kv, ptrs, 1, 8, None, need) == tv.SPEC_EINVAL
    assert _raw_verify(w, kv, ptrs, 1, 8, 0x100000, need - 1) == tv.SPEC_EWORKSPACE
    assert _raw_verify(w, kv, ptrs, 1, 8, 0x100010, need) == tv.SPEC_EINVAL          # unaligned
    assert _raw_verify(w, kv, ptrs, 1, 65, 0x100000, 1 << 40) == tv.SPEC_EUNSUPPORTED
    assert _raw_verify(w, kv, ptrs, 0, 8, 0x100000, need) == tv.SPEC_EINVAL
    w2, kv2, keep2 = _fake_structs(TINY, n_layers_ptrs=False)
    assert _raw_verify(w2, kv2, ptrs, 1, 8, 0x100000, need) == tv.SPEC_EINVAL       # NULL weight
    kv_bad = tv.KVCacheC(fake, fake, fake, 0, 9)
    assert _raw_verify(w, kv_bad, ptrs, 1, 8, 0x100000, need) == tv.SPEC_EINVAL


def test_pack_and_skinny_gemm_reject_bad_arguments():
    L = tv.lib()
    fake = 0x10000
    assert L.spec_pack_weight(None, 64, 64, fake, None) == tv.SPEC_EINVAL
    assert L.spec_pack_weight(fake, 64, 64, fake, None) == tv.SPEC_EINVAL       # in place
    assert L.spec_pack_weight(fake, 20, 64, fake + 4096, None) == tv.SPEC_EUNSUPPORTED
    assert L.spec_pack_weight(fake, 64, 40, fake + 4096, None) == tv.SPEC_EUNSUPPORTED
    assert L.spec_pack_weight(fake + 2, 64, 64, fake + 4096, None) == tv.SPEC_EINVAL    # unaligned
    assert L.spec_pack_weight(fake, 64, 64, fake + 4098, None) == tv.SPEC_EINVAL
    n = ctypes.c_size_t(0)
    assert L.spec_skinny_gemm_bytes(16, 40, 64, ctypes.byref(n)) == tv.SPEC_EUNSUPPORTED
    assert L.spec_skinny_gemm_bytes(16, 48, 40, ctypes.byref(n)) == tv.SPEC_EUNSUPPORTED
    assert L.spec_skinny_gemm_bytes(17, 32, 64, ctypes.byref(n)) == tv.SPEC_OK
    assert L.spec_skinny_gemm_bytes(16, 64, 64, ctypes.byref(n)) == tv.SPEC_OK and n.value > 0
    sp = ctypes.c_int(0)
    assert L.spec_skinny_gemm(fake, 16, 64, fake, 64, fake, 4, ctypes.byref(sp), None) == tv.SPEC_EWORKSPACE


def test_commit_and_accept_reject_bad_arguments():
    L = tv.lib()
    fake = 0x10000
    cfg = TINY.c()
    kv = tv.KVCacheC(fake, fake, fake, 16, 9)
    assert L.spec_commit_kv(ctypes.byref(cfg), ctypes.byref(kv), None, fake, fake, 1, 8, None) == tv.SPEC_EINVAL
    assert L.spec_commit_kv(ctypes.byref(cfg), ctypes.byref(kv), fake, fake, fake, 1, 65, None) == tv.SPEC_EUNSUPPORTED
    assert L.spec_commit_kv(None, ctypes.byref(kv), fake, fake, fake, 1, 8, None) == tv.SPEC_EINVAL
    need = tv.spec_accept_workspace_bytes(2, 16, 151936)
    assert need > 0
    args = [fake, fake, None, 2, 16, 151936, fake, fake, fake, None]
    assert L.spec_accept(*args, 0x100000, need - 1, None) == tv.SPEC_EWORKSPACE
    assert L.spec_accept(None, *args[1:], 0x100000, need, None) == tv.SPEC_EINVAL
    args_k = list(args)
    args_k[4] = 65
    assert L.spec_accept(*args_k, 0x100000, 1 << 30, None) == tv.SPEC_EUNSUPPORTED


def test_w12_entry_points_reject_bad_arguments():
    L = tv.lib()
    fake = 0x10000
    n = ctypes.c_size_t(0)
    assert L.spec_w12_plan_ints(64, 64, ctypes.byref(n)) == tv.SPEC_OK
    assert n.value == 2 + 64 // 16 + 1 + 256
    assert L.spec_w12_plan_ints(20, 64, ctypes.byref(n)) == tv.SPEC_EUNSUPPORTED
    assert L.spec_w12_plan_ints(64, 40, ctypes.byref(n)) == tv.SPEC_EUNSUPPORTED
    assert L.spec_w12_plan_ints(0, 64, ctypes.byref(n)) == tv.SPEC_EINVAL
    assert L.spec_w12_plan(None, 64, 64, fake, None) == tv.SPEC_EINVAL
    assert L.spec_w12_plan(fake, 64, 64, None, None) == tv.SPEC_EINVAL
    assert L.spec_w12_plan(fake + 2, 64, 64, fake, None) == tv.SPEC_EINVAL              # unaligned rows
    assert L.spec_w12_pack(fake + 8, 64, 64, fake, fake, fake, None) == tv.SPEC_EINVAL
    assert L.spec_w12_pack(fake, 64, 64, fake, None, fake, None) == tv.SPEC_EINVAL
    assert L.spec_w12_pack(fake, 64, 64, fake, fake, None, None) == tv.SPEC_EINVAL
    assert L.spec_w12_pack(fake, 64, 64, fake, fake + 4, fake, None) == tv.SPEC_EINVAL   # unaligned planes
    sp = ctypes.c_int(0)
    m = tv.W12MatrixC(fake, fake, None)
    assert L.spec_skinny_gemm_w12(fake, 16, 64, ctypes.byref(m), 64, fake, 1 << 20, ctypes.byref(sp),
                                  None) == tv.SPEC_EINVAL
    m = tv.W12MatrixC(fake, fake, fake)
    assert L.spec_skinny_gemm_w12(fake, 16, 64, ctypes.byref(m), 64, fake, 4, ctypes.byref(sp),
                                  None) == tv.SPEC_EWORKSPACE


def test_verify_w12_rejects_large_batches_and_missing_parts():
    w, kv, keep = _fake_structs(TINY)
    fake = 0x10000
    ptrs = dict(tok=fake, par=None, ctx=fake, a=fake, b=fake, p=fake)
    full = tv.W12MatrixC(fake, fake, fake)
    lay = (tv.W12LayerC * TINY.n_layers)(*[tv.W12LayerC(full, full, full, full)
                                           for _ in range(TINY.n_layers)])
    w.w12_layers = ctypes.cast(lay, ctypes.POINTER(tv.W12LayerC))
    need = tv.spec_workspace_bytes(TINY, 5, 16, 9)
    assert _raw_verify(w, kv, ptrs, 5, 16, 0x100000, need) == tv.SPEC_EUNSUPPORTED   # 80 rows
    lay[1].w_down = tv.W12MatrixC(fake, fake, None)
    need = tv.spec_workspace_bytes(TINY, 1, 8, 9)
    assert _raw_verify(w, kv, ptrs, 1, 8, 0x100000, need) == tv.SPEC_EINVAL
    w.w12_layers = None
    w.w12_lm_head = tv.W12MatrixC(None, fake, fake)   # planes unset: the bf16 head is used
    w.lm_head = None
    assert _raw_verify(w, kv, ptrs, 1, 8, 0x100000, need) == tv.SPEC_EINVAL


def test_prefill_rejects_bad_arguments():
    L = tv.lib()
    w, kv, keep = _fake_structs(TINY)
    fake = 0x10000
    n = ctypes.c_size_t(0)
    c = TINY.c()
    assert L.spec_prefill_workspace_bytes(ctypes.byref(c), 2, 9, 0, ctypes.byref(n)) == tv.SPEC_OK
    need = n.value
    assert need >= tv.spec_workspace_bytes(TINY, 2, 64, 9)
    assert L.spec_prefill_workspace_bytes(ctypes.byref(c), 2, 9, 1, ctypes.byref(n)) == tv.SPEC_OK
    assert n.value == need                     # the logits are written to the caller's buffer
    args = lambda **k: [k.get("w", ctypes.byref(w)), k.get("kv", ctypes.byref(kv)), k.get("prompt", fake),
                        k.get("ctx", fake), k.get("b", 2), k.get("p", 100), k.get("nt", fake), None,
                        k.get("ws", 0x100000), k.get("wsb", need), None]
    assert L.spec_prefill(*args(prompt=None)) == tv.SPEC_EINVAL
    assert L.spec_prefill(*args(ctx=None)) == tv.SPEC_EINVAL
    assert L.spec_prefill(*args(nt=None)) == tv.SPEC_EINVAL
    assert L.spec_prefill(*args(p=0)) == tv.SPEC_EINVAL
    assert L.spec_prefill(*args(b=0)) == tv.SPEC_EINVAL
    assert L.spec_prefill(*args(wsb=need - 1)) == tv.SPEC_EWORKSPACE
    assert L.spec_prefill(*args(ws=0x100010)) == tv.SPEC_EINVAL


def test_recurrent_entries_reject_bad_arguments():
    """Host-detectable errors of the recurrent-layer entries return before any launch."""
    L = tv.lib()
    f = 0x100000
    ok = (f, f + 0x1000, f + 0x2000, f + 0x3000, f + 0x4000, None, 2, 8, 4, 128, f + 0x5000, f + 0x6000, None)
    bad = [((None,) + ok[1:], tv.SPEC_EINVAL),
           ((f + 8,) + ok[1:], tv.SPEC_EINVAL),                       # unaligned state
           (ok[:4] + (None,) + ok[5:], tv.SPEC_EINVAL),               # no gates
           (ok[:6] + (0,) + ok[7:], tv.SPEC_EINVAL),                  # batch 0
           (ok[:7] + (65,) + ok[8:], tv.SPEC_EUNSUPPORTED),           # 65 nodes
           (ok[:8] + (0,) + ok[9:], tv.SPEC_EINVAL),                  # no heads
           (ok[:9] + (96,) + ok[10:], tv.SPEC_EUNSUPPORTED),          # head_dim 96
           (ok[:10] + (None,) + ok[11:], tv.SPEC_EINVAL),             # no output
           (ok[:10] + (f + 0x5004,) + ok[11:], tv.SPEC_EINVAL),       # unaligned output
           (ok[:11] + (None,) + ok[12:], tv.SPEC_EINVAL)]             # no status
    for args, code in bad:
        assert L.spec_rec_tree_verify(*args) == code, args
    c = (f, f + 0x1000, f + 0x2000, f + 0x3000, f + 0x4000, f + 0x5000, 2, 8, 4, 64, None)
    assert L.spec_rec_commit(*((None,) + c[1:])) == tv.SPEC_EINVAL
    assert L.spec_rec_commit(*(c[:4] + (None,) + c[5:])) == tv.SPEC_EINVAL
    assert L.spec_rec_commit(*(c[:7] + (65,) + c[8:])) == tv.SPEC_EUNSUPPORTED
    assert L.spec_rec_commit(*(c[:9] + (32,) + c[10:])) == tv.SPEC_EUNSUPPORTED
    assert L.spec_rec_commit(*(c[:1] + (f + 2,) + c[2:])) == tv.SPEC_EINVAL


def test_noalloc_accept_rejects_sizes_past_its_scratch_on_the_host():
    """spec_accept_noalloc checks its limits before touching a device: SPEC_ESCRATCH for more
    rows or a larger vocabulary than its static scratch holds, SPEC_EINVAL for empty shapes."""
    L = tv.lib()
    for batch, k, vocab, code in [(4097, 1, 1024, tv.SPEC_ESCRATCH), (65, 64, 1024, tv.SPEC_ESCRATCH),
                                  (1, 1, tv.SPEC_NOALLOC_MAX_VOCAB + 1, tv.SPEC_ESCRATCH),
                                  (0, 4, 1024, tv.SPEC_EINVAL), (1, 0, 1024, tv.SPEC_EINVAL)]:
        rc = L.spec_accept_noalloc(None, None, None, batch, k, vocab, None, None, None, None, None)
        assert rc == code, (batch, k, vocab, rc)
    assert "scratch" in tv.spec_strerror(tv.SPEC_ESCRATCH)
