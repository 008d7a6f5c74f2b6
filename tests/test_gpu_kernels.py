"""Kernel-level parity of the weight-streaming projection GEMM (spec_skinny_gemm) against the
CPU oracle's linear layer and a float64 product of the same bf16 operands, at the row counts the
verify pass uses (1 node, a block of 16, a 64-node tree, 32 requests x 16) and ragged shapes.

Bound: the classical one for a sum of kd products in fp32, |y - y64| <= gamma_kd sum|x||w|,
gamma_n = n u / (1 - n u), u = 2^-24. It holds for any order of summation, so it covers both the
GPU's split-K / MFMA order and the oracle's ascending order."""
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


def test_pack_layout_matches_its_definition():
    """Slot l of (tile t, step s) holds w[16t + l%16][32s + 8(l/16) .. +7], tiles outermost."""
    n, kd = 48, 96
    w = synth.randn_bf16((n, kd), 1.0, DEV, "pack")
    p = tv.spec_pack_weight(w)
    torch.cuda.synchronize()
    wb, pb = bits(w), bits(p).reshape(-1)
    k = 0
    for t in range(n // 16):
        for s in range(kd // 32):
            for l in range(64):
                r, c = 16 * t + l % 16, 32 * s + 8 * (l // 16)
                assert np.array_equal(pb[k:k + 8], wb[r, c:c + 8]), (t, s, l)
                k += 8
    assert k == n * kd


@pytest.mark.parametrize("m,n,kd", [(1, 7168, 5120), (16, 7168, 5120), (16, 5120, 17408),
                                    (16, 34816, 5120), (64, 1024, 5120), (8, 1408, 256),
                                    (8, 256, 704), (33, 64, 96), (512, 512, 1024), (3, 64, 32)])
def test_skinny_gemm_within_summation_bound(m, n, kd):
    x = synth.randn_bf16((m, kd), 1.0, DEV, "gx", m, n, kd)
    w = synth.randn_bf16((n, kd), 0.02, DEV, "gw", m, n, kd)
    part = torch.full((tv.spec_skinny_gemm_bytes(m, n, kd) // 4,), float("nan"), device=DEV)
    s = tv.spec_skinny_gemm(x, tv.spec_pack_weight(w), part)
    torch.cuda.synchronize()
    p = part[:s * m * n].view(s, m, n).cpu().numpy()
    y = p[0].copy()
    for i in range(1, s):
        y += p[i]
    xf = x.float().cpu().numpy().astype(np.float64)
    wf = w.float().cpu().numpy().astype(np.float64)
    ref = xf @ wf.T
    gamma = kd * U32 / (1 - kd * U32)
    bound = gamma * (np.abs(xf) @ np.abs(wf).T) + s * U32 * np.abs(ref)   # + adding the splits
    err = np.abs(y - ref)
    assert np.all(err <= bound), (err.max(), bound[err.argmax() // n, err.argmax() % n])
    yo = oracle.linear(bits(x), bits(w))
    assert np.all(np.abs(y - yo) <= 2 * bound)


def test_skinny_gemm_rejects_bad_shapes():
    x = torch.zeros((4, 40), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((64, 40), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(tv.SpecError):
        tv.spec_skinny_gemm(x, w, torch.zeros(1024, device=DEV))
    with pytest.raises(tv.SpecError):
        tv.spec_pack_weight(torch.zeros((20, 64), dtype=torch.bfloat16, device=DEV))


def test_read_probe_runs_and_checks_its_arguments():
    """The streaming-read probe reads its buffer and leaves the output word alone (the fold of
    all-zero data is zero, not the trigger constant); misaligned sizes are rejected."""
    buf = torch.zeros(1 << 20, dtype=torch.int32, device=DEV)
    out = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    tv.spec_read_probe(buf, out)
    torch.cuda.synchronize()
    assert int(out.item()) == 7
    with pytest.raises(RuntimeError):
        tv.spec_read_probe(buf[:3], out)
