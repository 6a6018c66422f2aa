"""CPU oracle of the band-block formulation of packed local attention (fp64).

TEST INFRASTRUCTURE ONLY: imported by tests, never by the product path; it
shares no code with the HIP path.

The performance reference page (dewml.dev/reference/performance, section
"Packed sliding-window attention on GPU: local_attention") computes a
packed batch with a sliding window of W keys by cutting the queries into
blocks of W and giving each block a [W, 2W] additive bias over the keys of
its own block and the block before it: 0 where the key is visible, -inf
elsewhere.  The page fixes neither the block alignment nor the bias
contents beyond that; the readings taken here are
  * blocks are aligned to the start of the packed microbatch (token 0), so
    query block b is tokens [b W, (b + 1) W) and its band keys
    [(b - 1) W, (b + 1) W), cut to [0, T);
  * the bias makes key j visible to query i when both lie in the same
    segment of cu_seqlens, j <= i and j > i - W (the window of the kernel
    benchmarks page, W keys counting the query itself);
  * the band's softmax runs over its 2W columns with that bias, so every
    key outside it counts as -inf.
Since a query's W visible keys all lie in its own block or the one before,
the result equals the dense definition in oracle/attention.py; the tests
pin the two against each other.
"""
from __future__ import annotations

import numpy as np


def _segment_ids(cu_seqlens, total: int) -> np.ndarray:
    """Segment index of every token (-1 outside every segment)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    ids = np.full(total, -1, dtype=np.int64)
    for s, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        ids[int(a):int(b)] = s
    return ids


def band_bias(cu_seqlens, total: int, window: int, b: int):
    """Key range [lo, hi) of query block b and its [rows, hi - lo] bias (0 / -inf)."""
    if window <= 0:
        raise ValueError("the band formulation needs a window W >= 1")
    q0, q1 = b * window, min(total, (b + 1) * window)
    lo, hi = max(0, (b - 1) * window), q1
    seg = _segment_ids(cu_seqlens, total)
    i = np.arange(q0, q1)[:, None]
    j = np.arange(lo, hi)[None, :]
    vis = (seg[i] == seg[j]) & (seg[i] >= 0) & (j <= i) & (j > i - window)
    return q0, q1, lo, hi, np.where(vis, 0.0, -np.inf)


def band_attention(q, k, v, dout, cu_seqlens, window: int, scale: float):
    """out, lse [Hq, T], dq, dk, dv of the band formulation (float64).

    Rows outside every segment get out 0, lse -inf and zero gradients, as in
    the dense oracle.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(dout, dtype=np.float64)
    t, hq, d = q.shape
    group = hq // k.shape[1]
    out = np.zeros_like(q)
    lse = np.full((hq, t), -np.inf)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range((t + window - 1) // window):
        q0, q1, lo, hi, bias = band_bias(cu_seqlens, t, window, b)
        live = np.isfinite(bias).any(axis=1)          # rows with a visible key
        if not live.any():
            continue
        rows = np.arange(q0, q1)[live]
        bias = bias[live]
        for h in range(hq):
            g = h // group
            kb, vb = k[lo:hi, g], v[lo:hi, g]
            s = scale * (q[rows, h] @ kb.T) + bias
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            z = e.sum(axis=1, keepdims=True)
            p = e / z
            out[rows, h] = p @ vb
            lse[h, rows] = (m + np.log(z))[:, 0]
            dp = do[rows, h] @ vb.T
            dd = (p * dp).sum(axis=1, keepdims=True)
            ds = p * (dp - dd)
            dq[rows, h] = scale * (ds @ kb)
            dk[lo:hi, g] += scale * (ds.T @ q[rows, h])
            dv[lo:hi, g] += p.T @ do[rows, h]
    return out, lse, dq, dk, dv
