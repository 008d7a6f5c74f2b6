"""Benchmark of the verification step on one MI355X.

One step = one spec_verify (target pass over the draft, greedy choice, accepted-path walk) plus
one spec_commit_kv (the accepted path's K/V rows compacted, context advanced), on synthetic
random-init weights of the 27B-class dense shape (64 layers, hidden 5120, 40 q / 8 kv heads of
128, SwiGLU 17408, vocab 151936), bf16, inputs resident in HBM. Steps are replayed from a HIP
graph captured once.

Workloads (--config):
  block   (default) batch 1, linear block of 16 uniform-random draft tokens, context 4096
  tree    batch 1, 64-node draft tree of depth <= 10, context 8192
  batched 32 requests x block of 16, contexts uniform in [512, 8192], shuffled 16-token pages
  prefill (a separate line, its own metric) one 4096-token prompt from an empty context
  rec     (a separate line, its own metric) the recurrent layers of a hybrid target: 32 requests
          x 64-node trees (depth <= 10), 32 heads with 128 x 128 fp32 states, 8 layers; one step
          is the tree pass and the state commit of every layer
--weights w12 stores the projections and the output head in the lossless 12-bit layout (batch-1
workloads only); the results are bit-identical to bf16 and the step streams a quarter fewer
weight bytes. A bf16 run of a batch-1 workload also times the same step over that layout and
reports it in a `w12` object (--no-w12 skips it).

Prints one JSON line: verified draft tokens/s (batch * k / step time), the step's algorithmic
HBM bytes and GB/s, the roofline of the dominant kernel (on the persistent plan of the block
workload the persistent layers kernel, 16 layers per launch; on the per-step plan the gate/up
projection GEMM with its SwiGLU epilogue; each timed per launch with HIP events recorded around
it on the verify stream in eager steps), and the CPU oracle timed on a bounded sample of the same
workload on this host (plus the tiny decoder at one thread and at all cores). The default block
run also times the block step in two more fresh processes (`processes`) and carries `tree` and
`batched` objects: the same measurement on those workloads.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np
import torch

import synth
import tree_verification_skinny_amd as tv

METRIC = "verified tokens/sec + verify-step HBM GB/s (% peak), 27B-shape dense, 1 GPU"

# HBM traffic of one launch of the dominant kernel (the gate/up projection; the recurrent layers'
# tree pass for --config rec), from two rocprofv3 --pmc passes over this script
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch, averaged over the kernel's dispatches), each
# scaled by what the same counter reads for a device-to-device copy of 4 GiB (bytes known). The
# figures hold for the kernel source they were taken on; any other source reports null.
PMC_TRAFFIC = {
    ("block", "bf16"): {"source": "tree_verification_skinny_amd/csrc/k_gemm.hip",
                        "sha256": "c2fa92e2d58b21d61d0784c079436ade6ebe53e9f7cde0eae0ab49c8f6d06c20",
                        "fetch_kib": 175305.2, "write_kib": 2610.0,
                        "fetch_scale": 1.9999676, "write_scale": 1.0},
    ("tree", "bf16"): {"source": "tree_verification_skinny_amd/csrc/k_gemm.hip",
                       "sha256": "c2fa92e2d58b21d61d0784c079436ade6ebe53e9f7cde0eae0ab49c8f6d06c20",
                       "fetch_kib": 178156.6, "write_kib": 6282.0,
                       "fetch_scale": 1.9999670, "write_scale": 1.0},
    ("rec", "bf16"): {"source": "tree_verification_skinny_amd/csrc/k_recurrent.hip",
                      "sha256": "e4a2e4ece68656d8812df5325d9800fc91a7a8825085a9d28257dc3739e862d6",
                      "fetch_kib": 58592.0, "write_kib": 32768.1,
                      "fetch_scale": 1.9999850, "write_scale": 1.0},
    ("block", "w12"): {"source": "tree_verification_skinny_amd/csrc/k_gemm.hip",
                       "sha256": "c2fa92e2d58b21d61d0784c079436ade6ebe53e9f7cde0eae0ab49c8f6d06c20",
                       "fetch_kib": 132094.1, "write_kib": 2610.0,
                       "fetch_scale": 1.9999698, "write_scale": 1.0},
}
# Average duration of one launch of the gate/up projection kernel in a rocprofv3 kernel trace of
# `bench.py --config C` (summaries under profiles/, each with its command). The trace times the
# kernel alone; the bench line's own figure brackets each launch with HIP events on the stream,
# which adds the launch's dispatch. Reported beside it while the kernel's source is unchanged.
PROFILED = {
    ("block", "bf16"): {"source": "tree_verification_skinny_amd/csrc/k_gemm.hip",
                        "sha256": "c2fa92e2d58b21d61d0784c079436ade6ebe53e9f7cde0eae0ab49c8f6d06c20",
                        "kernel": "gemm_kernel<4, 1, 8, 1, false, true>", "avg_us": 56.79,
                        "profile": "profiles/block16_ctx4096_kernels.md"},
    ("tree", "bf16"): {"source": "tree_verification_skinny_amd/csrc/k_gemm.hip",
                       "sha256": "c2fa92e2d58b21d61d0784c079436ade6ebe53e9f7cde0eae0ab49c8f6d06c20",
                       "kernel": "gemm_wide_kernel<4, 1, false, true>", "avg_us": 66.10,
                       "profile": "profiles/tree64_ctx8192_kernels.md"},
    ("batched", "bf16"): {"source": "tree_verification_skinny_amd/csrc/k_gemm_tc.hip",
                          "sha256": "b4b69ebb59847102b35290782bf7e52eadcf557c320954e21a4c734a0e6afac2",
                          "kernel": "gemm_tc_kernel<1>", "avg_us": 214.55,
                          "profile": "profiles/batched32x16_kernels.md"},
}
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0     # dense bf16 matrix-core peak of MI355X
SEED = 20261202


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def workload(name):
    if name == "block":
        return dict(batch=1, k=16, ctx=[4096], tree=False)
    if name == "tree":
        return dict(batch=1, k=64, ctx=[8192], tree=True)
    if name == "batched":
        rng = np.random.default_rng(synth.seed_of(SEED, "ctx"))
        return dict(batch=32, k=16, ctx=[int(c) for c in rng.integers(512, 8193, 32)], tree=False)
    raise ValueError(name)


def build_model(shape, device, w12=False):
    t0 = time.time()
    layers = [synth.layer_weights(shape, SEED, l, device) for l in range(shape.n_layers)]
    embed = synth.randn_bf16((shape.vocab, shape.hidden), 0.02, device, SEED, "embed")
    lm = synth.randn_bf16((shape.vocab, shape.hidden), 0.02, device, SEED, "lm_head")
    fn = torch.ones(shape.hidden, dtype=torch.bfloat16, device=device)
    torch.cuda.synchronize()
    log(f"weights generated on the GPU in {time.time() - t0:.1f}s")
    # packs the projections once (bf16 fragment order, or the lossless 12-bit layout)
    w = tv.Weights(tv.ModelCfg.of(shape), embed, fn, lm, layers, w12=w12)
    torch.cuda.synchronize()
    log(f"projection weights packed ({'W12' if w12 else 'bf16'}) in {time.time() - t0:.1f}s")
    return w


def step_bytes(shape, batch, k, ctx, w12=None):
    """Algorithmic HBM bytes of one verify step: every weight once (embedding rows only for the
    tokens), every context K/V row once per layer, the draft rows' K/V writes. With W12 weights
    (w12: the Weights.w12 dict) the projections and the output head count their W12 bytes:
    12 bits per value, the per-tile exception offsets and the exceptions."""
    H, F, V, L = shape.hidden, shape.ffn, shape.vocab, shape.n_layers
    d, nq, nkv = shape.head_dim, shape.n_q_heads, shape.n_kv_heads
    if w12 is None:
        per_layer_w = 2 * (shape.qkv_rows * H + H * nq * d + 2 * F * H + H * F + 2 * H)
        weights = L * per_layer_w + 2 * (V * H + H) + 2 * batch * k * H
    else:
        proj = sum(m.nbytes() for lw in w12["layers"] for m in lw.values()) + w12["lm_head"].nbytes()
        weights = proj + L * 2 * 2 * H + 2 * H + 2 * batch * k * H
    kv_read = L * sum(c for c in ctx) * nkv * d * 2 * 2
    kv_write = L * batch * k * nkv * d * 2 * 2
    return weights + kv_read + kv_write


def step_flops(shape, batch, k, ctx, depth_mean):
    H, F, V, L = shape.hidden, shape.ffn, shape.vocab, shape.n_layers
    d, nq = shape.head_dim, shape.n_q_heads
    M = batch * k
    gemm = 2 * M * (shape.qkv_rows * H + H * nq * d + 2 * F * H + H * F) * L + 2 * M * V * H
    keys = sum(ctx) * k + batch * k * (depth_mean + 1)
    attn = L * 4 * nq * d * keys
    return gemm + attn


def gate_up_bytes(shape, m, w12=None):
    """Algorithmic HBM bytes of one gate/up projection launch: the packed [2F][H] weight once (its
    W12 bytes, averaged over the layers, with W12 weights), the normalised activations [m][H] in,
    the SwiGLU output [m][F] out (bf16)."""
    H, F = shape.hidden, shape.ffn
    wb = 2 * (2 * F * H) if w12 is None else \
        sum(lw["w_gate_up"].nbytes() for lw in w12["layers"]) / len(w12["layers"])
    return wb + 2 * m * H + 2 * m * F


def time_gate_up(step_with_events, events, n_layers, stream, reps):
    """Per-launch duration of the gate/up projection kernel (the pass's largest), from HIP events
    recorded on the verify stream right before and after each of its launches in `reps` eager
    steps (launched one by one: events captured into a HIP graph are not ordered against the
    graph's kernels, so they cannot time one). The host enqueues far faster than the step runs,
    so the device queue stays full and each pair of events brackets the kernel alone.
    Returns (mean seconds per launch, ms per eager step)."""
    step_with_events()
    stream.synchronize()
    durs = []
    t_step = 0.0
    for _ in range(reps):
        s0 = torch.cuda.Event(enable_timing=True)
        s1 = torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        step_with_events()
        s1.record(stream)
        s1.synchronize()
        t_step += s0.elapsed_time(s1)
        durs.extend(events[2 * l].elapsed_time(events[2 * l + 1]) for l in range(n_layers))
    return float(np.mean(durs)) / 1e3, t_step / reps


def pmc_traffic(config, weights="bf16"):
    """Counter-measured HBM bytes per launch of the workload's dominant kernel (the gate/up
    projection; the tree pass for the recurrent layers), or None when there are no counters for
    this workload and weight layout or the kernel's source has changed since they were taken."""
    import hashlib
    rec = PMC_TRAFFIC.get((config, weights))
    if rec is None or rec["sha256"] is None:
        return None
    with open(os.path.join(ROOT, rec["source"]), "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec["sha256"]:
            return None
    return int(round((rec["fetch_kib"] * rec["fetch_scale"] + rec["write_kib"] * rec["write_scale"]) * 1024))


def profiled(config, weights, work, bound):
    """The kernel-trace figure of the gate/up launch for this workload (see PROFILED): its
    duration and the roofline fraction it gives for `work` (bytes, or flops when bound is mfma),
    or None when there is no trace for it or the kernel's source has changed since."""
    import hashlib
    rec = PROFILED.get((config, weights))
    if rec is None:
        return None
    with open(os.path.join(ROOT, rec["source"]), "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec["sha256"]:
            return None
    s = rec["avg_us"] * 1e-6
    if bound == "mfma":
        ach, unit, peak = work / s / 1e12, "TFLOP/s", MFMA_BF16_PEAK_TFLOPS
    else:
        ach, unit, peak = work / s / 1e9, "GB/s", HBM_PEAK_GBPS
    return {"kernel": rec["kernel"], "us_per_launch": rec["avg_us"], "achieved": round(ach, 1), "unit": unit,
            "frac": round(ach / peak, 4), "profile": rec["profile"]}


def time_w12(weights, shape, kv, t_tok, t_par, t_ctx, ctx0, B, K, ctx, acc, bonus, path, ws, stream,
             steps, warmup):
    """Step time over W12 weights built from the same row-major tensors: graph replays timed with
    events around the whole run, like the main line. Also checks that the first W12 pass gives
    the bf16 pass's logits bit for bit."""
    R = weights.rowmajor
    w = tv.Weights(weights.cfg, weights.tensors["embed"], weights.tensors["final_norm"], R["lm_head"],
                   R["layers"], w12=True)
    lg16 = torch.empty((B * K, shape.vocab), dtype=torch.float32, device=t_tok.device)
    lg12 = torch.empty_like(lg16)
    with torch.cuda.stream(stream):
        # the bf16 reference runs the per-step plan, the one W12 runs
        tv.spec_verify(weights, kv, t_tok, t_par, t_ctx, B, K, acc, bonus, path, ws, logits=lg16, path="steps")
        tv.spec_verify(w, kv, t_tok, t_par, t_ctx, B, K, acc, bonus, path, ws, logits=lg12)
        stream.synchronize()
        same = bool(torch.equal(lg16.view(torch.int32), lg12.view(torch.int32)))

        def step():
            tv.spec_verify(w, kv, t_tok, t_par, t_ctx, B, K, acc, bonus, path, ws)
            tv.spec_commit_kv(w.cfg, kv, acc, path, t_ctx, B, K)

        t_ctx.copy_(ctx0)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        for _ in range(warmup):
            graph.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            graph.replay()
        e1.record(stream)
        e1.synchronize()
    t_ctx.copy_(ctx0)
    ms = e0.elapsed_time(e1) / steps
    nbytes = step_bytes(shape, B, K, ctx, w.w12)
    del graph, w
    torch.cuda.empty_cache()
    return {"ms_per_step": round(ms, 4), "value": round(B * K / (ms / 1e3), 2),
            "unit": "verified tokens/s", "bytes_per_step": int(nbytes),
            "achieved_gbps": round(nbytes / (ms / 1e3) / 1e9, 1),
            "logits_bit_identical_to_bf16": same,
            "note": "same step over the lossless 12-bit layout of the same weights (per-step "
                    "kernels; logits compared with the bf16 per-step plan)"}


def read_probe(device, nbytes=4 << 30):
    """Streaming-read rate: the library's plain grid-stride read of a 4 GiB buffer (HIP events
    on the current stream around 5 launches)."""
    a = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=device)
    a.fill_(1.0)
    out = torch.zeros(1, dtype=torch.int32, device=device)
    for _ in range(2):
        tv.spec_read_probe(a, out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        tv.spec_read_probe(a, out)
    e1.record()
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) / 1e3 / 5
    del a
    return nbytes / s / 1e9


def copy_probe(device, nbytes=4 << 30):
    a = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=device)
    b = torch.empty_like(a)
    a.fill_(1.0)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) / 1e3 / 5
    del a, b
    return 2 * nbytes / s / 1e9


def cpu_baseline(weights, shape, kv, tokens, parent, ctx, budget_s):
    """The CPU oracle as it stands, on a bounded sample of the same workload: request 0's pass
    through the first n layers (n grows until the budget is spent) and the output head, scaled
    to the whole step (per-layer time x 64, plus the head, times the number of requests)."""
    import oracle
    from tree_verification_skinny_amd import kvlayout

    def host(t):
        return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)

    cfg = oracle.Cfg(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads,
                     shape.head_dim, shape.ffn, shape.vocab, shape.rms_eps, shape.rope_theta)
    W = weights.tensors
    R = weights.rowmajor
    model = oracle.Model(cfg, host(W["embed"]), host(W["final_norm"]), host(R["lm_head"]),
                         layer_fn=lambda l: {k: host(v) for k, v in R["layers"][l].items()})
    tok0 = tokens[0]
    par0 = oracle.chain(len(tok0)) if parent is None else parent[0]
    x = oracle.embed(model, tok0)
    spent, n = 0.0, 0
    pos = torch.arange(ctx[0])
    while n < shape.n_layers and spent < budget_s:
        lw = model.layer(n)
        kc, vc = kvlayout.read_rows(kv, n, 0, pos)
        kc, vc = host(kc), host(vc)
        t0 = time.time()
        x, _, _ = oracle.layer_forward(cfg, lw, kc, vc, par0, x)
        spent += time.time() - t0
        n += 1
    t0 = time.time()
    lg = oracle.logits(model, x)
    oracle.argmax(lg)
    head = time.time() - t0
    per_request = spent / n * shape.n_layers + head
    step = per_request * len(tokens)
    k = len(tok0)
    return {"value": len(tokens) * k / step, "unit": "verified tokens/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": (f"request 0 of {len(tokens)}, layers 0..{n - 1} of {shape.n_layers} "
                       f"({spent:.1f}s) + output head ({head:.1f}s), scaled to the full step "
                       f"({step:.1f}s per step)")}


def prefill_flops(shape, P):
    """The method's arithmetic of a P-token prefill from an empty context (multiply-adds count 2):
    every projection for every prompt row, causal attention (row i's scores and weighted sum over
    i + 1 keys for every q head), the output head for the last row only."""
    L, H, F, d = shape.n_layers, shape.hidden, shape.ffn, shape.head_dim
    nq, nkv = shape.n_q_heads, shape.n_kv_heads
    proj = H * (nq + 2 * nkv) * d + nq * d * H + 2 * F * H + F * H
    attn = 4 * d * nq * P * (P + 1) // 2
    return L * (2 * P * proj + attn) + 2 * shape.vocab * H


def prefill_bench(args, shape, device):
    """spec_prefill of one request's prompt from an empty context, replayed from a HIP graph: the
    whole prompt (up to 4096 positions) in one pass over the tile projections, causal attention
    over the cache, the output head for the last position. Prints one JSON line with prompt
    tokens/s and the method's TFLOP/s against the bf16 matrix-core peak."""
    P = args.prompt
    w12 = args.weights == "w12"
    weights = build_model(shape, device, w12)
    pages = (P + 15) // 16
    kv = tv.PagedKV.empty(tv.ModelCfg.of(shape), pages, torch.arange(pages, dtype=torch.int32).view(1, pages),
                          device)
    prompt = torch.from_numpy(synth.uniform_tokens(P, shape.vocab, SEED, "prefill").astype(np.int32)).to(device)
    prompt = prompt.view(1, P)
    ctx = torch.zeros(1, dtype=torch.int32, device=device)
    nt = torch.empty(1, dtype=torch.int32, device=device)
    ws = tv.workspace(tv.spec_prefill_workspace_bytes(weights.cfg, 1, pages), device)
    stream = torch.cuda.Stream()

    def run():
        ctx.zero_()
        tv.spec_prefill(weights, kv, prompt, ctx, nt, ws)

    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        run()
        stream.synchronize()
        assert int(ctx.item()) == P and int(nt.item()) >= 0
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            run()
        for _ in range(max(1, args.warmup // 2)):
            graph.replay()
        reps = max(2, min(args.steps, 5))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            graph.replay()
        e1.record(stream)
        e1.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = prefill_flops(shape, P)
    tflops = flops / (ms / 1e3) / 1e12
    chunk = min(P, 4096)
    result = {
        "metric": "prefill prompt tokens/s, 27B-shape dense, 1 GPU", "value": round(P / (ms / 1e3), 1),
        "unit": "prompt tokens/s", "n_gpus": 1, "steps": reps, "ms_per_prefill": round(ms, 3),
        "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic (seeded random-init weights N(0,0.02), uniform prompt tokens)",
        "config": {"workload": f"27B-shape dense, 64 layers + lm_head, batch 1, prompt {P} from an empty "
                               f"context, passes of up to {chunk} positions",
                   "weights": "W12 (lossless 12-bit)" if w12 else "bf16", "hip_graph": True},
        "mfma": {"flops_per_prefill": int(flops), "achieved_tflops": round(tflops, 1),
                 "peak_tflops": MFMA_BF16_PEAK_TFLOPS, "frac_of_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                 "note": "the method's arithmetic: all projections of every prompt row, causal "
                         "attention, the output head of the last row"},
    }
    log(f"prefill of {P}: {ms:.2f} ms, {P / (ms / 1e3):.0f} tokens/s, {tflops:.1f} TFLOP/s")
    print(json.dumps(result), flush=True)


def rec_bytes(B, K, H, D, accepted_len):
    """Algorithmic bytes of one recurrent tree pass and one state commit (fp32 states, bf16 q, k,
    v, fp32 gates and outputs, int32 parents and path ids)."""
    tree = B * H * (D * D * 4 + 3 * K * D * 2 + 2 * K * 4 + K * D * 4)
    commit = (B * H * (2 * D * D * 4) + int((np.asarray(accepted_len) + 1).sum()) * H * 2 * D * 2 +
              B * H * K * 4)
    return tree, commit


def rec_bench(args, device):
    """Tree pass + state commit of a hybrid target's recurrent layers (spec_rec_tree_verify,
    spec_rec_commit), 8 layers with their own states and inputs (about 1.2 GB per step, beyond
    the memory-side cache), replayed from a HIP graph. Algorithmic bytes of a tree pass, per
    (request, head): the state D*D*4, q, k, v K*D*2 each, gates and parents K*4 each, outputs
    K*D*4; of a commit: the state read and written, the path's k and v rows, and the K path ids
    each (request, head) reads."""
    B, K, H, D, L = 32, 64, 32, 128, 8
    parents = np.stack([synth.random_tree(K, 10, SEED, "rec", b) for b in range(B)]).astype(np.int32)
    par = torch.from_numpy(parents).to(device)
    layers = []
    for l in range(L):
        S0, q, k, v, g = synth.rec_inputs(B, K, H, D, D, SEED, device, "bench", l)
        layers.append((S0.transpose(-1, -2).contiguous(), q, k, v, g))   # the library's layout
    out = torch.empty((B, K, H, D), dtype=torch.float32, device=device)
    status = torch.empty(B, dtype=torch.int32, device=device)
    # accepted path: the root path of a seeded node of each tree (what the greedy walk returns)
    rng = np.random.default_rng(SEED)
    acc = np.zeros(B, np.int32)
    path = np.zeros((B, K), np.int32)
    for b in range(B):
        j, p = int(rng.integers(0, K)), []
        while j != -1:
            p.append(j)
            j = int(parents[b, j])
        p = p[::-1]
        acc[b] = len(p) - 1
        path[b, :len(p)] = p
    acc_t, path_t = torch.from_numpy(acc).to(device), torch.from_numpy(path).to(device)
    stream = torch.cuda.Stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * L)]

    def step(events=False):
        for l, (S0, q, k, v, g) in enumerate(layers):
            if events:
                ev[3 * l].record(stream)
            tv.spec_rec_tree_verify(S0, q, k, v, g, par, out, status)
            if events:
                ev[3 * l + 1].record(stream)
            tv.spec_rec_commit(S0, k, v, g, acc_t, path_t)
            if events:
                ev[3 * l + 2].record(stream)

    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        step()
        stream.synchronize()
        assert not status.cpu().numpy().any()
        # per-launch tree-pass time from events on this stream, eager steps
        durs, cdurs = [], []
        for _ in range(3):
            step(events=True)
            stream.synchronize()
            durs.extend(ev[3 * l].elapsed_time(ev[3 * l + 1]) for l in range(L))
            cdurs.extend(ev[3 * l + 1].elapsed_time(ev[3 * l + 2]) for l in range(L))
        t_tree = float(np.mean(durs)) / 1e3
        t_commit = float(np.mean(cdurs)) / 1e3
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        for _ in range(args.warmup):
            graph.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        e1.record(stream)
        e1.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    copy_gbps = copy_probe(device)     # also the calibration copy of the counter passes
    depth_sum = 0
    for b in range(B):
        d = np.zeros(K, np.int64)
        for i in range(1, K):
            d[i] = d[parents[b, i]] + 1
        depth_sum += int((d + 1).sum())            # path lengths, root .. node
    tree_bytes, commit_bytes = rec_bytes(B, K, H, D, acc)
    step_bytes_ = L * (tree_bytes + commit_bytes)
    gbps = step_bytes_ / (ms / 1e3) / 1e9
    ach = tree_bytes / t_tree / 1e9
    flops = 2 * B * H * K * D * D + 4 * H * depth_sum * D      # state term + path terms
    result = {
        "metric": "hybrid-target recurrent layers: tree-verified node-layers/s, 1 GPU",
        "value": round(B * K * L / (ms / 1e3), 1), "unit": "node-layers/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded states N(0,1/4), q/k N(0,1/d) and v N(0,1) bf16, decays U(0.6,1))",
        "config": {"workload": f"recurrent layers of a hybrid target: {B} requests x {K}-node trees "
                               f"(depth <= 10), {H} heads, {D}x{D} fp32 states, {L} layers; tree pass "
                               f"+ state commit per layer", "hip_graph": True},
        "hbm": {"bytes_per_step": int(step_bytes_), "achieved_gbps": round(gbps, 1),
                "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4), "copy_probe_gbps": round(copy_gbps, 1)},
        "roofline": {"kernel": "rec_tree_kernel<128>", "bound": "hbm", "achieved": round(ach, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
                     "traffic": pmc_traffic("rec"), "us_per_launch": round(t_tree * 1e6, 2),
                     "bytes_per_launch": int(tree_bytes),
                     "fp32_tflops": round(flops / t_tree / 1e12, 2)},
        "commit_kernel": {"kernel": "rec_commit_kernel<128>", "us_per_launch": round(t_commit * 1e6, 2),
                          "bytes_per_launch": int(commit_bytes),
                          "achieved_gbps": round(commit_bytes / t_commit / 1e9, 1)},
    }
    log(f"rec: {ms:.3f} ms per step ({gbps:.0f} GB/s); tree pass {t_tree * 1e6:.1f} us "
        f"({ach:.0f} GB/s, {flops / t_tree / 1e12:.1f} TFLOP/s)")
    if not args.no_cpu_baseline:
        import oracle
        spent, n = 0.0, 0
        bits = lambda t: t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
        while spent < args.cpu_seconds and n < L * B * H:
            l, b, h = n // (B * H), n % B, (n * 7) % H
            S0, q, k, v, g = layers[l]
            sl = lambda t: t[b:b + 1, :, h:h + 1]
            hs = (S0[b:b + 1, h:h + 1].transpose(-1, -2).contiguous().cpu().numpy(), bits(sl(q)), bits(sl(k)),
                  bits(sl(v)), sl(g).contiguous().cpu().numpy())
            t0 = time.time()
            oracle.rec_tree(*hs, parents[b:b + 1])
            oracle.rec_commit(hs[0], hs[2], hs[3], hs[4], acc[b:b + 1], path[b:b + 1])
            spent += time.time() - t0
            n += 1
        per_pair = spent / n
        result["cpu_baseline"] = {"value": round(K / per_pair / H, 2), "unit": "node-layers/s",
                                  "cores": oracle.threads(), "kind": "oracle",
                                  "sample": f"{n} (layer, request, head) tree passes + commits "
                                            f"({spent:.1f}s), scaled to a step's {L * B * H}"}
        log(f"cpu baseline: {result['cpu_baseline']}")
    print(json.dumps(result), flush=True)


WORKLOAD_NAMES = {
    "block": "27B-shape dense, 64 layers + lm_head 151936, batch 1, linear block of 16, context 4096",
    "tree": "27B-shape dense, 64 layers + lm_head, batch 1, 64-node tree (depth<=10), context 8192",
    "batched": "27B-shape dense, 64 layers + lm_head, 32 requests x block of 16, contexts U[512,8192], paged",
}


def setup(name, shape, weights, device, total_steps):
    """Cache, draft and outputs of one workload (inputs resident on the GPU)."""
    wl = workload(name)
    B, K, ctx = wl["batch"], wl["k"], wl["ctx"]
    # cache: room for the context, the draft, and every step's commit (at most K rows each)
    pages = [(c + K + K * total_steps + 15) // 16 for c in ctx]
    table, n_pages = synth.page_table(B, pages, SEED, shuffle=(B > 1))
    kv = tv.PagedKV.empty(tv.ModelCfg.of(shape), n_pages, torch.from_numpy(table), device)
    g = torch.Generator(device=device)
    g.manual_seed(SEED)
    kv.k_pool.normal_(generator=g)
    kv.v_pool.normal_(generator=g)
    if wl["tree"]:
        parent = np.stack([synth.random_tree(K, 10, SEED, b) for b in range(B)]).astype(np.int32)
        tokens = np.stack([synth.tree_tokens(parent[b], shape.vocab, SEED, b) for b in range(B)])
        depths = []
        for b in range(B):
            dep = [0] * K
            for i in range(1, K):
                dep[i] = dep[parent[b][i]] + 1
            depths.extend(dep)
        depth_mean = float(np.mean(depths))
    else:
        parent = None
        tokens = np.stack([synth.uniform_tokens(K, shape.vocab, SEED, b) for b in range(B)])
        depth_mean = (K - 1) / 2
    w = dict(name=name, B=B, K=K, ctx=ctx, kv=kv, tokens=tokens.astype(np.int32), parent=parent,
             depth_mean=depth_mean)
    w["t_tok"] = torch.from_numpy(w["tokens"]).to(device)
    w["t_par"] = None if parent is None else torch.from_numpy(parent).to(device)
    w["ctx0"] = torch.tensor(ctx, dtype=torch.int32, device=device)
    w["t_ctx"] = w["ctx0"].clone()
    w["acc"] = torch.empty(B, dtype=torch.int32, device=device)
    w["bonus"] = torch.empty(B, dtype=torch.int32, device=device)
    w["path"] = torch.empty((B, K), dtype=torch.int32, device=device)
    w["ws"] = tv.workspace(tv.spec_workspace_bytes(weights.cfg, B, K, kv.max_pages), device)
    return w


def make_step(weights, w, path):
    def step(gate_up_events=None, layer_events=None):
        tv.spec_verify(weights, w["kv"], w["t_tok"], w["t_par"], w["t_ctx"], w["B"], w["K"], w["acc"],
                       w["bonus"], w["path"], w["ws"], gate_up_events=gate_up_events,
                       layer_events=layer_events, path=path)
        tv.spec_commit_kv(weights.cfg, w["kv"], w["acc"], w["path"], w["t_ctx"], w["B"], w["K"])
    return step


def time_steps(step, w, stream, steps, warmup, eager):
    """W untimed warm-up steps, then exactly `steps` steps (HIP-graph replays unless eager),
    bracketed by synchronisations; one event between consecutive steps. Returns (ms per step,
    per-step ms array, rows committed over the timed steps)."""
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        step()                              # first launch: module load, checks
        stream.synchronize()
        graph = None
        if not eager:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                step()
        run = graph.replay if graph is not None else step
        for _ in range(warmup):
            run()
        stream.synchronize()
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ctx_before = w["t_ctx"].clone()
        torch.cuda.synchronize()
        marks[0].record(stream)
        for i in range(steps):
            run()
            marks[i + 1].record(stream)
        marks[-1].synchronize()
        torch.cuda.synchronize()
        committed = (w["t_ctx"] - ctx_before).sum().item()
    ms = marks[0].elapsed_time(marks[-1]) / steps
    per_step = np.array([marks[i].elapsed_time(marks[i + 1]) for i in range(steps)])
    del graph
    return ms, per_step, committed


def step_stats(per_step):
    return {"mean": round(float(np.mean(per_step)), 4), "median": round(float(np.median(per_step)), 4),
            "p5": round(float(np.percentile(per_step, 5)), 4),
            "p95": round(float(np.percentile(per_step, 95)), 4),
            "ci95": round(1.96 * float(np.std(per_step, ddof=1)) / len(per_step) ** 0.5, 4)
            if len(per_step) > 1 else None}


def event_pairs(n, stream):
    events = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in events:
        e.record(stream)                     # creates the underlying HIP event
    stream.synchronize()
    return events, (ctypes.c_void_p * n)(*[e.cuda_event for e in events])


def layer_bytes(shape, batch, k, ctx):
    """Algorithmic HBM bytes of one layer of the pass: its weights once, every context K/V row
    of the layer once, the draft rows' K/V writes."""
    H, F = shape.hidden, shape.ffn
    d, nq, nkv = shape.head_dim, shape.n_q_heads, shape.n_kv_heads
    wb = 2 * (shape.qkv_rows * H + H * nq * d + 2 * F * H + H * F + 2 * H)
    return wb + sum(ctx) * nkv * d * 2 * 2 + batch * k * nkv * d * 2 * 2


def persistent_roofline(step, shape, w, stream, reps):
    """Per-launch duration of the persistent layers kernel (16 layers per launch) from HIP
    events recorded on the verify stream right before and after each launch, in eager steps."""
    L = shape.n_layers
    nl = (L + 15) // 16
    events, handles = event_pairs(2 * nl, stream)
    with torch.cuda.stream(stream):
        s_launch, ms_ev = time_gate_up(lambda: step(layer_events=handles), events, nl, stream, reps)
    w["t_ctx"].copy_(w["ctx0"])
    b_launch = layer_bytes(shape, w["B"], w["K"], w["ctx"]) * L / nl
    ach = b_launch / s_launch / 1e9
    return {"kernel": "fused_layers_kernel (the persistent layers kernel, 16 layers per launch)",
            "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": pmc_traffic("block_persistent"),
            "bytes_per_launch": int(b_launch), "us_per_launch": round(s_launch * 1e6, 2),
            "launches_per_step": nl, "ms_per_eager_step_with_events": round(ms_ev, 4)}


def gate_up_roofline(step, shape, w, stream, reps, config, w12):
    """Per-launch duration of the gate/up projection kernel of the per-step plan (events around
    each launch, eager steps); HBM-bound up to 64 rows, matrix-core-bound beyond."""
    L = shape.n_layers
    events, handles = event_pairs(2 * L, stream)
    with torch.cuda.stream(stream):
        s_launch, ms_ev = time_gate_up(lambda: step(gate_up_events=handles), events, L, stream, reps)
    w["t_ctx"].copy_(w["ctx0"])
    B, K = w["B"], w["K"]
    b_launch = gate_up_bytes(shape, B * K, w12)
    if B * K > 64:
        flops = 2 * B * K * (2 * shape.ffn) * shape.hidden
        ach = flops / s_launch / 1e12
        r = {"kernel": "gemm_tc_kernel, SwiGLU epilogue (gate/up projection)", "bound": "mfma",
             "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": pmc_traffic(config),
             "flops_per_launch": int(flops), "bytes_per_launch": int(b_launch)}
    else:
        ach = b_launch / s_launch / 1e9
        kname = "gemm_kernel" if B * K <= 16 or w12 is not None else "gemm_wide_kernel"
        if w12 is not None:
            kname += " over W12 weights"
        r = {"kernel": f"{kname}, SwiGLU epilogue (gate/up projection)", "bound": "hbm",
             "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
             "frac": round(ach / HBM_PEAK_GBPS, 4),
             "traffic": pmc_traffic(config, "w12" if w12 is not None else "bf16"),
             "bytes_per_launch": int(b_launch)}
    r.update({"us_per_launch": round(s_launch * 1e6, 2), "launches_per_step": L,
              "ms_per_eager_step_with_events": round(ms_ev, 4),
              "timing": "HIP events around each launch on the verify stream (dispatch included)",
              "profiled": profiled(config, "w12" if w12 is not None else "bf16",
                                   r.get("flops_per_launch", b_launch), r["bound"])})
    return r


def measure(name, shape, weights, device, stream, args, steps, warmup, path, kernel_timing=True):
    """One workload: the timed steps, the step's bytes and flops, and the dominant kernel's
    roofline. Returns (result dict, workload state)."""
    w = setup(name, shape, weights, device, steps + warmup + 3 + 12)
    step = make_step(weights, w, path)
    ms, per_step, committed = time_steps(step, w, stream, steps, warmup, args.eager)
    B, K, ctx = w["B"], w["K"], w["ctx"]
    w12 = weights.w12
    nbytes = step_bytes(shape, B, K, ctx, w12)
    flops = step_flops(shape, B, K, ctx, w["depth_mean"])
    value = B * K / (ms / 1e3)
    gbps = nbytes / (ms / 1e3) / 1e9
    r = {"ms_per_step": round(ms, 4), "value": round(value, 2), "unit": "verified tokens/s",
         "workload": WORKLOAD_NAMES[name], "batch": B, "k": K, "ctx_mean": float(np.mean(ctx)),
         "hbm": {"bytes_per_step": int(nbytes), "achieved_gbps": round(gbps, 1),
                 "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)},
         "mfma": {"flops_per_step": flops, "tflops": round(flops / (ms / 1e3) / 1e12, 2),
                  "frac_of_bf16_peak": round(flops / (ms / 1e3) / 2.5e15, 5)},
         "step_ms": step_stats(per_step),
         "draft_tokens_per_s": round(B * (K - 1) / (ms / 1e3), 2),
         "committed_tokens_per_s": round(committed / steps / (ms / 1e3), 2),
         "ctx_after": w["t_ctx"].cpu().tolist()[:4]}
    log(f"{name}: step {ms:.3f} ms  {value:.1f} verified tok/s  {gbps:.0f} GB/s "
        f"({gbps / HBM_PEAK_GBPS:.1%} of peak)")
    if kernel_timing:
        reps = max(3, min(steps, 10))
        persistent = path == "persistent"
        if persistent:
            r["roofline"] = persistent_roofline(step, shape, w, stream, reps)
        else:
            r["roofline"] = gate_up_roofline(step, shape, w, stream, reps, name, w12)
        r["roofline"]["share_of_step"] = round(
            r["roofline"]["us_per_launch"] * r["roofline"]["launches_per_step"] / 1e3 / ms, 4)
        log(f"{name}: {r['roofline']['kernel']}: {r['roofline']['achieved']} {r['roofline']['unit']} "
            f"per launch ({r['roofline']['us_per_launch']} us)")
    w["t_ctx"].copy_(w["ctx0"])
    return r, w


def child_repeat(args):
    """A fresh process: the block workload's step time only (repeats of the headline across
    processes: the confidence interval covers start-up state, not only step-to-step noise)."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--child", "--steps", str(args.steps),
           "--warmup", str(args.warmup), "--path", args.path]
    if args.eager:
        cmd.append("--eager")
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        log(f"repeat process failed ({r.returncode}): {r.stderr[-500:]}")
        return None
    return json.loads(r.stdout.strip().splitlines()[-1])["ms_per_step"]


def cpu_baseline_tiny(budget_s=4.0):
    """The oracle on the tiny decoder's verify step (block of 8 over a 128-token context), at one
    thread and at all of this host's cores."""
    import oracle
    from tree_verification_skinny_amd import kvlayout  # noqa: F401  (same imports as the GPU side)
    shape = synth.TINY

    def host(t):
        return t.detach().contiguous().view(torch.int16).numpy().view(np.uint16)

    w = synth.model_weights(shape, SEED)
    cfg = oracle.Cfg(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads,
                     shape.head_dim, shape.ffn, shape.vocab, shape.rms_eps, shape.rope_theta)
    model = oracle.Model(cfg, host(w["embed"]), host(w["final_norm"]), host(w["lm_head"]),
                         [{k: host(v) for k, v in lw.items()} for lw in w["layers"]])
    kc = [host(synth.kv_context(shape, 128, SEED, l)[0]) for l in range(shape.n_layers)]
    vc = [host(synth.kv_context(shape, 128, SEED, l)[1]) for l in range(shape.n_layers)]
    tokens = synth.uniform_tokens(8, shape.vocab, SEED, "tiny")
    out = {}
    n_all = oracle.threads()
    for label, n in (("threads_1", 1), ("threads_all", n_all)):
        oracle.set_threads(n)
        oracle.verify(model, kc, vc, tokens)
        reps, t0 = 0, time.time()
        while time.time() - t0 < budget_s / 2:
            oracle.verify(model, kc, vc, tokens)
            reps += 1
        out[label] = {"ms_per_step": round((time.time() - t0) / reps * 1e3, 3), "threads": n}
    oracle.set_threads(n_all)
    return {"workload": "tiny decoder (2 layers, hidden 256), block of 8, context 128",
            "kind": "oracle", **out}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="block", choices=["block", "tree", "batched", "prefill", "rec"])
    ap.add_argument("--path", default="auto", choices=["auto", "steps", "persistent"],
                    help="launch plan of spec_verify (auto: persistent where it applies)")
    ap.add_argument("--prompt", type=int, default=4096, help="prompt length of --config prefill")
    ap.add_argument("--eager", action="store_true", help="launch every step instead of a HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--no-w12", action="store_true",
                    help="skip the extra timing of the same step over lossless 12-bit weights")
    ap.add_argument("--no-sub", action="store_true",
                    help="skip the tree and batched sub-objects of the default block run")
    ap.add_argument("--processes", type=int, default=3,
                    help="fresh processes that time the block step (this one included)")
    ap.add_argument("--child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--weights", default="bf16", choices=["bf16", "w12"],
                    help="projection weight storage: bf16, or the lossless 12-bit layout (W12)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the verify step of "
              "this build runs on a single MI355X).", file=sys.stderr)
        sys.exit(2)
    # repeats in fresh processes run first, before this process touches the GPU
    repeats = []
    if not args.child and args.config == "block" and args.weights == "bf16" and args.processes > 1:
        for i in range(args.processes - 1):
            log(f"repeat process {i + 1} of {args.processes - 1}")
            ms = child_repeat(args)
            if ms is not None:
                repeats.append(ms)
    if not torch.cuda.is_available():
        print("bench.py needs the GPU", file=sys.stderr)
        sys.exit(2)
    device = "cuda"
    shape = synth.DENSE_27B
    if args.config == "prefill":
        prefill_bench(args, shape, device)
        return
    if args.config == "rec":
        rec_bench(args, device)
        return
    w12 = args.weights == "w12"
    if w12 and args.config == "batched":
        print("W12 weights serve passes of at most 64 rows (batch 1); use --weights bf16 for the "
              "batched workload", file=sys.stderr)
        sys.exit(2)
    weights = build_model(shape, device, w12)
    stream = torch.cuda.Stream()
    if args.child:
        r, w = measure(args.config, shape, weights, device, stream, args, args.steps, args.warmup,
                       args.path, kernel_timing=False)
        print(json.dumps({"ms_per_step": r["ms_per_step"]}), flush=True)
        return

    main_r, w = measure(args.config, shape, weights, device, stream, args, args.steps, args.warmup,
                        args.path, kernel_timing=not args.no_kernel_timing)
    ms = main_r["ms_per_step"]
    result = {
        "metric": METRIC, "value": main_r["value"], "unit": "verified tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded random-init weights N(0,0.02), context K/V N(0,1))",
        "config": {"workload": WORKLOAD_NAMES[args.config], "batch": main_r["batch"], "k": main_r["k"],
                   "ctx_mean": main_r["ctx_mean"], "layers": shape.n_layers, "vocab": shape.vocab,
                   "hip_graph": not args.eager, "parallelism": "single GPU",
                   "weights": "W12 (lossless 12-bit)" if w12 else "bf16",
                   "launch_plan": "persistent" if args.path == "persistent" else "per-step kernels"},
    }
    for key in ("hbm", "mfma", "step_ms", "draft_tokens_per_s", "committed_tokens_per_s", "ctx_after",
                "roofline"):
        if key in main_r:
            result[key] = main_r[key]
    if repeats:
        allp = repeats + [ms]
        result["processes"] = {"ms_per_step": [round(x, 4) for x in allp],
                               "mean": round(float(np.mean(allp)), 4),
                               "ci95": round(1.96 * float(np.std(allp, ddof=1)) / len(allp) ** 0.5, 4)
                               if len(allp) > 1 else None,
                               "note": "the block step timed in separate fresh processes (this one last)"}
    if not args.no_kernel_timing:
        result["copy_probe_gbps"] = round(copy_probe(device), 1)
        rp = read_probe(device)
        result["read_probe_gbps"] = round(rp, 1)
        result["hbm"]["frac_of_read_probe"] = round(result["hbm"]["achieved_gbps"] / rp, 4)
    B, K, ctx = w["B"], w["K"], w["ctx"]
    if (not w12 and not args.no_w12 and B * K <= 64 and weights.rowmajor is not None):
        # the same step over the lossless 12-bit layout of the same weights (bit-identical to
        # the per-step bf16 plan), reported beside the bf16 line; `value` stays the bf16 one
        w["t_ctx"].copy_(w["ctx0"])
        result["w12"] = time_w12(weights, shape, w["kv"], w["t_tok"], w["t_par"], w["t_ctx"], w["ctx0"],
                                 B, K, ctx, w["acc"], w["bonus"], w["path"], w["ws"], stream,
                                 args.steps, args.warmup)
        log(f"W12: {result['w12']}")
    if not args.no_cpu_baseline:
        w["t_ctx"].copy_(w["ctx0"])
        result["cpu_baseline"] = cpu_baseline(weights, shape, w["kv"], w["tokens"], w["parent"], ctx,
                                              args.cpu_seconds)
        log(f"cpu baseline: {result['cpu_baseline']}")
        result["cpu_baseline_tiny"] = cpu_baseline_tiny()
        log(f"cpu baseline (tiny): {result['cpu_baseline_tiny']}")
    del w
    torch.cuda.empty_cache()
    if args.config == "block" and not args.no_sub and not w12:
        # the tree and batched workloads of the same stack, each with its dominant kernel
        for name in ("tree", "batched"):
            sub, ws_ = measure(name, shape, weights, device, stream, args, min(args.steps, 10),
                               min(args.warmup, 3), args.path,
                               kernel_timing=not args.no_kernel_timing)
            result[name] = sub
            del ws_
            torch.cuda.empty_cache()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
