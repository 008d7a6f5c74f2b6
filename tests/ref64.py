"""An independent float64 PyTorch evaluation of the target decoder, rounding to bf16 exactly
where the oracle stores tensors. It shares nothing with the oracle's C code: torch's own matmul,
scaled_dot_product_attention and SiLU, an explicit visibility mask built by following parents,
and the rotate-half RoPE written with torch ops. Its differences from the oracle are pure
arithmetic order and precision, which sizes what any correct fp32 implementation may differ by."""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

import oracle


def rb(t, dt=torch.float64):
    """Round to bf16 (through fp32) and return it in dtype dt."""
    return t.float().to(torch.bfloat16).to(dt)


def _t(x, dt=torch.float64):
    """bf16 bits (numpy uint16) or a torch tensor -> tensor of dtype dt."""
    if isinstance(x, np.ndarray):
        return torch.from_numpy(oracle.from_bf16(x)).to(dt)
    return x.to(dt)


def layer(shape, lw, k_ctx, v_ctx, parent, x, dt=torch.float64):
    """One decoder layer. lw: dict of bf16 tensors (or uint16 arrays); k_ctx/v_ctx: [ctx][nkv][d];
    x: [m][H]. Returns (x_out, k_new, v_new) as tensors of dtype dt holding bf16 values. With
    dt = float32 it is an fp32 evaluation in torch's own summation order: a correct implementation
    of the same storage points that differs from the oracle only in reduction order."""
    nq, nkv, d, Fd = shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.ffn
    eps = shape.rms_eps
    x = _t(x, dt)
    m = x.shape[0]
    kc, vc = _t(k_ctx, dt).reshape(-1, nkv, d), _t(v_ctx, dt).reshape(-1, nkv, d)
    ctx = kc.shape[0]
    depth = [0] * m
    vis = torch.zeros(m, ctx + m, dtype=torch.bool)
    vis[:, :ctx] = True
    for i in range(m):
        if i:
            depth[i] = depth[int(parent[i])] + 1
        j = i
        while j >= 0:
            vis[i, ctx + j] = True
            j = int(parent[j])
    pos = torch.tensor([ctx + dd for dd in depth], dtype=torch.float64)
    inv = shape.rope_theta ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
    ang = pos[:, None] * inv[None, :]
    cos = torch.cat([ang.cos(), ang.cos()], -1)[:, None, :].float().to(dt)
    sin = torch.cat([ang.sin(), ang.sin()], -1)[:, None, :].float().to(dt)

    def norm(v, g):
        return rb(v / torch.sqrt((v * v).mean(-1, keepdim=True) + eps) * g, dt)

    def rot(t):
        t1, t2 = t[..., : d // 2], t[..., d // 2:]
        return rb(t * cos + torch.cat([-t2, t1], -1) * sin, dt)

    W = {k: _t(v, dt) for k, v in lw.items()}
    u = norm(x, W["attn_norm"])
    qkv = u @ W["w_qkv"].T
    q = rot(rb(qkv[:, : nq * d], dt).view(m, nq, d))
    k = rot(rb(qkv[:, nq * d: (nq + nkv) * d], dt).view(m, nkv, d))
    v = rb(qkv[:, (nq + nkv) * d:], dt).view(m, nkv, d)
    K = torch.cat([kc, k], 0).permute(1, 0, 2).repeat_interleave(nq // nkv, 0)
    V = torch.cat([vc, v], 0).permute(1, 0, 2).repeat_interleave(nq // nkv, 0)
    o = F.scaled_dot_product_attention(q.permute(1, 0, 2), K, V, attn_mask=vis)
    o = rb(o.permute(1, 0, 2).reshape(m, nq * d), dt)
    x = rb(x + rb(o @ W["w_o"].T, dt), dt)
    u = norm(x, W["mlp_norm"])
    gu = u @ W["w_gate_up"].T
    h = rb(F.silu(rb(gu[:, :Fd], dt)) * rb(gu[:, Fd:], dt), dt)
    x = rb(x + rb(h @ W["w_down"].T, dt), dt)
    return x, k, v


def logits(shape, final_norm, lm_head, x):
    x = _t(x)
    g = _t(final_norm)
    u = rb(x / torch.sqrt((x * x).mean(-1, keepdim=True) + shape.rms_eps) * g)
    return (u @ _t(lm_head).T).numpy()


def decoder(w, shape, tokens, parent, k_ctx, v_ctx):
    """Whole pass: returns (logits [m][V], hidden list entering each layer and after the last)."""
    x = w["embed"].double()[torch.tensor(np.asarray(tokens), dtype=torch.long)]
    hidden = [x]
    for l, lw in enumerate(w["layers"]):
        x, _, _ = layer(shape, lw, k_ctx[l], v_ctx[l], parent, x)
        hidden.append(x)
    return logits(shape, w["final_norm"], w["lm_head"], x), hidden
