"""CPU oracle: document-masked causal grouped-query attention, fp64.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links this module; only the tests, the smoke check and the bench's CPU
baseline do.  It shares no code with the HIP path.

What is computed
----------------
The kernel benchmarks page (research.dws.rip/llm/kernels) fixes the
workload: section 01 "How it was measured" describes packed rows, ended at
the context length, in which attention stays inside each document, so it is
causal inside each segment of a packed microbatch; Fig. 2 "Benchmark setup"
gives 8 query and 2 key-value heads of width 128 and a 512-token window for
the local layers; section 02 says the kernel is FlashAttention-2's varlen
call with sliding windows and grouped-query attention.  The arithmetic is
textbook scaled-dot-product softmax attention and its analytic gradient.
Written out, for segment [a, b), query head h, its key-value head
g = floor(h / G) with G = Hq / Hkv, and query i in [a, b):

    V(i)   = { j : max(a, i - W + 1) <= j <= i }     (W <= 0: { j : a <= j <= i })
    S_ij   = scale * q_{i,h} . k_{j,g}               for j in V(i)
    LSE_hi = log sum_{j in V(i)} exp(S_ij)            (natural log)
    P_ij   = exp(S_ij - LSE_hi)
    O_ih   = sum_j P_ij v_{j,g}
    dP_ij  = dO_ih . v_{j,g}
    D_hi   = sum_j P_ij dP_ij
    dS_ij  = P_ij (dP_ij - D_hi)
    dq_ih  = scale sum_j dS_ij k_{j,g}
    dk_jg  = scale sum_{h in g} sum_i dS_ij q_{i,h}
    dv_jg  =       sum_{h in g} sum_i P_ij dO_ih

Readings where the pages are silent: the window holds W keys counting the
query itself (i - W < j <= i); window <= 0 means full causal context; query
head h reads key-value head floor(h / G); the scale multiplies q.k before
the softmax; LSE is the natural log, laid out [Hq, T].

Logit soft-cap (optional, softcap = c > 0).  The performance reference page
(dewml.dev/reference/performance, section "Head dimension 256 through
tokamax's Triton flash attention") lists Gemma 2's attention-logit soft-cap
as a feature a training kernel needs in its forward and its backward.  The
cap bounds each scaled logit smoothly to (-c, c) before the softmax:

    S'_ij  = c * tanh(S_ij / c)        (replaces S_ij above; no bias term)
    dS_ij  = P_ij (dP_ij - D_hi) * (1 - tanh(S_ij / c)^2)

i.e. the softmax gradient taken with respect to S' and carried back through
the cap by the chain rule.  The page gives no value for c; softcap <= 0
means no cap.

Implementation: one dense [L, L] block per (segment, query head) with a
boolean mask, all in float64.  Inputs are taken as float arrays (the exact
bf16 values the GPU reads, widened); nothing is rounded on the way.
"""
from __future__ import annotations

import numpy as np


def segments(cu_seqlens):
    """Non-empty segments [a, b) of a packed microbatch, in order."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return [(int(a), int(b)) for a, b in zip(cu[:-1], cu[1:]) if b > a]


def visible_mask(length: int, window: int) -> np.ndarray:
    """mask[i, j] is True when local query i sees local key j in one segment.

    Causal (j <= i) and, for window W > 0, j > i - W, i.e. W keys counting
    the query itself.  Indices are local to the segment, so keys of other
    documents never appear.
    """
    i = np.arange(length)[:, None]
    j = np.arange(length)[None, :]
    m = j <= i
    if window > 0:
        m &= j > i - window
    return m


def _check(q, k, v):
    if q.ndim != 3 or k.ndim != 3 or v.ndim != 3:
        raise ValueError("q, k, v must be [T, H, d]")
    hq, hkv = q.shape[1], k.shape[1]
    if hq % hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    return hq // hkv


def _capped_logits(qs, ks, scale, softcap):
    """Scaled logits of one segment and head, soft-capped when softcap > 0.

    Also returns d S' / d S (all ones without a cap)."""
    s = scale * (qs @ ks.T)
    if softcap > 0:
        t = np.tanh(s / softcap)
        return softcap * t, 1.0 - t * t
    return s, np.ones_like(s)


def _segment_head_forward(qs, ks, vs, mask, scale, softcap=0.0):
    """Softmax attention of one segment and one query head (fp64)."""
    s, dcap = _capped_logits(qs, ks, scale, softcap)
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)          # every row sees at least itself
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    lse = (m + np.log(z))[:, 0]
    p = e / z
    return p @ vs, lse, p, dcap


def attention_forward(q, k, v, cu_seqlens, window: int, scale: float, softcap: float = 0.0):
    """out [T, Hq, d] and lse [Hq, T], float64.  Rows outside every segment are 0 / -inf."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    group = _check(q, k, v)
    t, hq, d = q.shape
    out = np.zeros((t, hq, d))
    lse = np.full((hq, t), -np.inf)
    for a, b in segments(cu_seqlens):
        mask = visible_mask(b - a, window)
        for h in range(hq):
            g = h // group
            o, l, _, _ = _segment_head_forward(q[a:b, h], k[a:b, g], v[a:b, g], mask, scale,
                                               softcap)
            out[a:b, h] = o
            lse[h, a:b] = l
    return out, lse


def attention_backward(q, k, v, dout, cu_seqlens, window: int, scale: float,
                       softcap: float = 0.0):
    """Analytic gradients of sum(dout * out): dq, dk, dv (float64), plus out, lse, D."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(dout, dtype=np.float64)
    group = _check(q, k, v)
    t, hq, d = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    out = np.zeros_like(q)
    lse = np.full((hq, t), -np.inf)
    dsum = np.zeros((hq, t))
    for a, b in segments(cu_seqlens):
        mask = visible_mask(b - a, window)
        for h in range(hq):
            g = h // group
            qs, ks, vs, dos = q[a:b, h], k[a:b, g], v[a:b, g], do[a:b, h]
            o, l, p, dcap = _segment_head_forward(qs, ks, vs, mask, scale, softcap)
            out[a:b, h] = o
            lse[h, a:b] = l
            dp = dos @ vs.T
            dd = (p * dp).sum(axis=1, keepdims=True)
            ds = p * (dp - dd) * dcap
            dsum[h, a:b] = dd[:, 0]
            dq[a:b, h] = scale * (ds @ ks)
            dk[a:b, g] += scale * (ds.T @ qs)
            dv[a:b, g] += p.T @ dos
    return dq, dk, dv, out, lse, dsum


def attention_row(q, k, v, dout, cu_seqlens, window: int, scale: float, h: int, i: int,
                  softcap: float = 0.0):
    """One query row, computed alone: (out_ih [d], lse_hi, dq_ih [d]).

    Used to check single sampled outputs of large problems without running
    the whole oracle.  Same definitions as above, restricted to row i.
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    s_idx = int(np.searchsorted(cu, i, side="right")) - 1
    a = int(cu[s_idx])
    lo = max(a, i - window + 1) if window > 0 else a
    group = q.shape[1] // k.shape[1]
    g = h // group
    ks = np.asarray(k[lo:i + 1, g], dtype=np.float64)
    vs = np.asarray(v[lo:i + 1, g], dtype=np.float64)
    qi = np.asarray(q[i, h], dtype=np.float64)
    doi = np.asarray(dout[i, h], dtype=np.float64)
    s = scale * (ks @ qi)
    dcap = np.ones_like(s)
    if softcap > 0:
        t = np.tanh(s / softcap)
        s = softcap * t
        dcap = 1.0 - t * t
    m = s.max()
    e = np.exp(s - m)
    z = e.sum()
    p = e / z
    o = p @ vs
    dp = vs @ doi
    ds = p * (dp - p @ dp) * dcap
    return o, m + np.log(z), scale * (ds @ ks)


def attention_key(q, k, v, dout, cu_seqlens, window: int, scale: float, g: int, j: int,
                  softcap: float = 0.0):
    """One key's gradients, computed alone: (dk_jg [d], dv_jg [d]).

    The column counterpart of attention_row: the same definitions restricted
    to the queries i that see key j (j in V(i)), each with its whole row
    softmax, summed over the query heads of key-value head g.  Used to check
    sampled dK/dV entries of problems too large for the whole oracle.
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    s_idx = int(np.searchsorted(cu, j, side="right")) - 1
    a, b = int(cu[s_idx]), int(cu[s_idx + 1])
    hi = min(b - 1, j + window - 1) if window > 0 else b - 1
    rows = np.arange(j, hi + 1)                     # queries that see key j
    lo = np.maximum(a, rows - window + 1) if window > 0 else np.full_like(rows, a)
    keys = np.arange(int(lo.min()), hi + 1)
    mask = (keys[None, :] >= lo[:, None]) & (keys[None, :] <= rows[:, None])
    group = q.shape[1] // k.shape[1]
    kk = np.asarray(k[keys, g], dtype=np.float64)
    vv = np.asarray(v[keys, g], dtype=np.float64)
    col = j - int(keys[0])
    dk = np.zeros(k.shape[2])
    dv = np.zeros(k.shape[2])
    for h in range(g * group, (g + 1) * group):
        qs = np.asarray(q[rows, h], dtype=np.float64)
        dos = np.asarray(dout[rows, h], dtype=np.float64)
        s = scale * (qs @ kk.T)
        dcap = np.ones_like(s)
        if softcap > 0:
            t = np.tanh(s / softcap)
            s = softcap * t
            dcap = 1.0 - t * t
        s = np.where(mask, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        p = e / e.sum(axis=1, keepdims=True)
        dp = dos @ vv.T
        dd = (p * dp).sum(axis=1, keepdims=True)
        ds = p * (dp - dd) * dcap
        dk += scale * (ds[:, col] @ qs)
        dv += p[:, col] @ dos
    return dk, dv
