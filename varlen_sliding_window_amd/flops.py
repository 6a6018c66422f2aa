"""Exact work counts for document-masked causal attention (host-side measurement).

Throughput is counted the way the kernel benchmarks page's workload implies
(research.dws.rip/llm/kernels, Fig. 2 "Benchmark setup": forward plus
backward per layer): 4*d flops per unmasked (query, key) pair per query head
in the forward pass (two d-long dot products: q.k and p*v), and 2.5 times
that, 10*d, in the backward pass (q.k recomputed is not counted; dP, dV, dK,
dQ are).  Pairs are counted exactly from the segment lengths and the window.
"""
from __future__ import annotations

from typing import Iterable


def pairs_in_segment(length: int, window: int) -> int:
    """Unmasked (query, key) pairs of one causal segment of ``length`` tokens.

    Query i (local index) sees min(i + 1, W) keys when W > 0, else i + 1.
    Summing: L(L+1)/2 if W <= 0 or W >= L, else W(W+1)/2 + (L - W) W.
    """
    n = int(length)
    if n <= 0:
        return 0
    w = int(window)
    if w <= 0 or w >= n:
        return n * (n + 1) // 2
    return w * (w + 1) // 2 + (n - w) * w


def count_pairs(cu_seqlens: Iterable[int], window: int) -> int:
    cu = [int(x) for x in cu_seqlens]
    return sum(pairs_in_segment(b - a, window) for a, b in zip(cu[:-1], cu[1:]))


def attention_flops(cu_seqlens, window: int, num_q_heads: int, head_dim: int) -> dict:
    """Counted flops: {'pairs', 'fwd', 'bwd', 'fwd_bwd'} for one layer."""
    p = count_pairs(cu_seqlens, window)
    fwd = 4 * head_dim * p * num_q_heads
    bwd = 10 * head_dim * p * num_q_heads
    return {"pairs": p, "fwd": fwd, "bwd": bwd, "fwd_bwd": fwd + bwd}


def algorithmic_bytes(total_tokens: int, num_q_heads: int, num_kv_heads: int,
                      head_dim: int) -> dict:
    """Bytes each pass must move at least once (bf16 tensors, fp32 LSE and D).

    Forward: read q, k, v; write out, lse.  Backward: read q, k, v, out,
    dout, lse; write and read back D; write dq, dk, dv.
    """
    t, hq, hkv, d = total_tokens, num_q_heads, num_kv_heads, head_dim
    qb = t * hq * d * 2
    kb = t * hkv * d * 2
    row = t * hq * 4
    fwd = qb + 2 * kb + qb + row
    bwd = (qb + 2 * kb + qb + qb + row) + 2 * row + (qb + 2 * kb)
    return {"fwd": fwd, "bwd": bwd, "fwd_bwd": fwd + bwd}
