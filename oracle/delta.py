"""CPU oracle of gated delta-rule linear attention (Gated DeltaNet), fp64.

TEST INFRASTRUCTURE ONLY: imported by tests, never by the product path; it
shares no code with the HIP path.

The kernel benchmarks page (research.dws.rip/llm/kernels, section 03 "What
linear attention costs", Figs. 1 and 5) times Gated DeltaNet (Yang et al.)
from the flash-linear-attention library as the competing local layer and
says its kernels match a token-by-token 32-bit reference; the page does not
restate the method.  This oracle is that token-by-token reference, written
from the published recurrence of the gated delta rule.  Per head, with a
state S of d_v x d_k that starts at zero at every document start of
cu_seqlens:

    S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
        = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T
    o_t = scale * S_t q_t

with alpha_t = exp(g_t) (g_t <= 0, the log decay) and beta_t in (0, 1)
the write strength.  Readings where the pages are silent: q and k arrive as
given (the model normalises them before the layer), the scale multiplies
the read-out, and heads do not share state.  The backward is torch's
autograd of the same loop in float64 on the CPU (a library primitive as one
step); the tests pin it with central finite differences.
"""
from __future__ import annotations

import numpy as np


def _segments(cu_seqlens):
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return [(int(a), int(b)) for a, b in zip(cu[:-1], cu[1:]) if b > a]


def gated_delta_forward(q, k, v, g, beta, cu_seqlens, scale: float = 1.0):
    """o [T, H, d_v] (float64) of the gated delta rule, token by token.

    q, k: [T, H, d_k]; v: [T, H, d_v]; g, beta: [T, H].  Rows outside every
    segment are zero.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    t_, h_, dk = q.shape
    dv = v.shape[2]
    o = np.zeros((t_, h_, dv))
    for a, b in _segments(cu_seqlens):
        for h in range(h_):
            s = np.zeros((dv, dk))
            for t in range(a, b):
                alpha = np.exp(g[t, h])
                kt = k[t, h]
                s = alpha * s + beta[t, h] * np.outer(v[t, h] - alpha * (s @ kt), kt)
                o[t, h] = scale * (s @ q[t, h])
    return o


def gated_delta_backward(q, k, v, g, beta, dout, cu_seqlens, scale: float = 1.0):
    """Gradients of sum(dout * o): dq, dk, dv, dg, dbeta (float64), by torch
    autograd of the token loop on the CPU, plus o."""
    import torch

    def t64(x):
        return torch.tensor(np.asarray(x, dtype=np.float64), dtype=torch.float64, requires_grad=True)

    tq, tk, tv, tg, tb = (t64(x) for x in (q, k, v, g, beta))
    tdo = torch.tensor(np.asarray(dout, dtype=np.float64), dtype=torch.float64)
    t_, h_, dk = tq.shape
    dv = tv.shape[2]
    rows = [None] * t_
    for a, b in _segments(cu_seqlens):
        per_head = []
        for h in range(h_):
            s = torch.zeros((dv, dk), dtype=torch.float64)
            outs = []
            for t in range(a, b):
                alpha = torch.exp(tg[t, h])
                kt = tk[t, h]
                s = alpha * s + tb[t, h] * torch.outer(tv[t, h] - alpha * (s @ kt), kt)
                outs.append(scale * (s @ tq[t, h]))
            per_head.append(torch.stack(outs))                    # [L, d_v]
        seg_o = torch.stack(per_head, dim=1)                      # [L, H, d_v]
        for i, t in enumerate(range(a, b)):
            rows[t] = seg_o[i]
    zero = torch.zeros((h_, dv), dtype=torch.float64)
    o = torch.stack([r if r is not None else zero for r in rows])
    loss = (o * tdo).sum()
    grads = torch.autograd.grad(loss, (tq, tk, tv, tg, tb), allow_unused=True)
    out = [np.zeros_like(np.asarray(x, dtype=np.float64)) if gr is None else gr.numpy()
           for x, gr in zip((q, k, v, g, beta), grads)]
    return (*out, o.detach().numpy())
