"""CPU oracle of Kimi Delta Attention (gated delta rule with a per-channel
gate), fp64.

TEST INFRASTRUCTURE ONLY: imported by tests, never by the product path; it
shares no code with the HIP path.

The kernel benchmarks page (research.dws.rip/llm/kernels, section 03 "What
linear attention costs", Figs. 1 and 5) times Kimi Delta Attention from the
flash-linear-attention library beside Gated DeltaNet and does not define
either.  This is the published recurrence written token by token.  Per head,
a state S of d_v x d_k starts at zero at every document start of
cu_seqlens; the decay alpha_t = exp(g_t) is a d_k vector, one factor per key
channel:

    S'_t = S_{t-1} Diag(alpha_t)
    S_t  = S'_t + beta_t (v_t - S'_t k_t) k_t^T
    o_t  = scale * S_t q_t

The authors keep the state as d_k x d_v and write the transition as
(I - beta k k^T) Diag(alpha) S + beta k v^T; the form above is its
transpose.  Readings where the pages are silent: as for Gated DeltaNet (q
and k arrive normalised by the layer, the scale multiplies the read-out,
heads do not share state).  A gate equal on every channel gives Gated
DeltaNet (oracle/delta.py); the tests pin the two against each other.  The
backward is torch's autograd of the same loop in float64 on the CPU.
"""
from __future__ import annotations

import numpy as np


def _segments(cu_seqlens):
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return [(int(a), int(b)) for a, b in zip(cu[:-1], cu[1:]) if b > a]


def kimi_delta_forward(q, k, v, g, beta, cu_seqlens, scale: float = 1.0):
    """o [T, H, d_v] (float64), token by token.

    q, k: [T, H, d_k]; v: [T, H, d_v]; g: [T, H, d_k] (per-channel log
    decay); beta: [T, H].  Rows outside every segment are zero.
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
                sp = s * np.exp(g[t, h])[None, :]
                kt = k[t, h]
                s = sp + beta[t, h] * np.outer(v[t, h] - sp @ kt, kt)
                o[t, h] = scale * (s @ q[t, h])
    return o


def kimi_delta_backward(q, k, v, g, beta, dout, cu_seqlens, scale: float = 1.0):
    """Gradients of sum(dout * o): dq, dk, dv, dg ([T, H, d_k]), dbeta
    (float64), by torch autograd of the token loop on the CPU, plus o."""
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
            st = torch.zeros((dv, dk), dtype=torch.float64)
            outs = []
            for t in range(a, b):
                sd = st * torch.exp(tg[t, h])[None, :]
                kt = tk[t, h]
                st = sd + tb[t, h] * torch.outer(tv[t, h] - sd @ kt, kt)
                outs.append(scale * (st @ tq[t, h]))
            per_head.append(torch.stack(outs))
        seg_o = torch.stack(per_head, dim=1)
        for i, t in enumerate(range(a, b)):
            rows[t] = seg_o[i]
    zero = torch.zeros((h_, dv), dtype=torch.float64)
    o = torch.stack([r if r is not None else zero for r in rows])
    loss = (o * tdo).sum()
    grads = torch.autograd.grad(loss, (tq, tk, tv, tg, tb), allow_unused=True)
    out = [np.zeros_like(np.asarray(x, dtype=np.float64)) if gr is None else gr.numpy()
           for x, gr in zip((q, k, v, g, beta), grads)]
    return (*out, o.detach().numpy())
