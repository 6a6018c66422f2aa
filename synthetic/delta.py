"""Seeded inputs for gated delta-rule linear attention (input drawing only).

Stands in for the projections a Gated DeltaNet layer feeds its kernel (the
kernel benchmarks page, research.dws.rip/llm/kernels, section 03, times the
layer on the same 16,384-token microbatches as attention and does not give
the projections): with the microbatch's cu_seqlens and one
``numpy.random.default_rng(seed)``, in this order
  q, k  standard_normal [T, H, D], each token-head vector scaled to unit
        length (the layer normalises q and k), then rounded to bf16;
  v     standard_normal [T, H, D] rounded to bf16;
  g     log of uniform(0.85, 0.999) [T, H] (per-token decay), fp32;
  beta  uniform(0.05, 0.95) [T, H] (write strength), fp32.
Kimi Delta inputs (``make_kda_inputs``) draw the same way, except that g is
log of uniform(0.85, 0.999) per key channel, [T, H, D].
The output gradient of the backward (``make_delta_dout``) is standard_normal
[T, H, D] from its own ``default_rng(seed)``, rounded to bf16.
The bf16 values come back as raw bit patterns (what the GPU reads) and as the
equal float32 arrays (what the oracle reads).
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .microbatch import bf16_bits_to_f32, f32_to_bf16_bits


@dataclasses.dataclass
class DeltaInputs:
    cu_seqlens: np.ndarray
    q_bits: np.ndarray
    k_bits: np.ndarray
    v_bits: np.ndarray
    g: np.ndarray
    beta: np.ndarray

    def f32(self, name: str) -> np.ndarray:
        return bf16_bits_to_f32(getattr(self, name + "_bits"))


def make_delta_inputs(cu_seqlens, num_heads: int, head_dim: int, seed: int) -> DeltaInputs:
    cu = np.asarray(cu_seqlens, dtype=np.int32)
    t = int(cu[-1])
    rng = np.random.default_rng(seed)

    def unit(x):
        n = np.linalg.norm(x, axis=-1, keepdims=True)
        return x / np.where(n > 0, n, 1.0)

    q = unit(rng.standard_normal((t, num_heads, head_dim), dtype=np.float32))
    k = unit(rng.standard_normal((t, num_heads, head_dim), dtype=np.float32))
    v = rng.standard_normal((t, num_heads, head_dim), dtype=np.float32)
    g = np.log(rng.uniform(0.85, 0.999, size=(t, num_heads))).astype(np.float32)
    beta = rng.uniform(0.05, 0.95, size=(t, num_heads)).astype(np.float32)
    return DeltaInputs(cu, f32_to_bf16_bits(q.astype(np.float32)), f32_to_bf16_bits(k.astype(np.float32)),
                       f32_to_bf16_bits(v), g, beta)


def make_kda_inputs(cu_seqlens, num_heads: int, head_dim: int, seed: int) -> DeltaInputs:
    """As make_delta_inputs, with a per-channel gate g [T, H, D]."""
    cu = np.asarray(cu_seqlens, dtype=np.int32)
    t = int(cu[-1])
    rng = np.random.default_rng(seed)

    def unit(x):
        n = np.linalg.norm(x, axis=-1, keepdims=True)
        return x / np.where(n > 0, n, 1.0)

    q = unit(rng.standard_normal((t, num_heads, head_dim), dtype=np.float32))
    k = unit(rng.standard_normal((t, num_heads, head_dim), dtype=np.float32))
    v = rng.standard_normal((t, num_heads, head_dim), dtype=np.float32)
    g = np.log(rng.uniform(0.85, 0.999, size=(t, num_heads, head_dim))).astype(np.float32)
    beta = rng.uniform(0.05, 0.95, size=(t, num_heads)).astype(np.float32)
    return DeltaInputs(cu, f32_to_bf16_bits(q.astype(np.float32)), f32_to_bf16_bits(k.astype(np.float32)),
                       f32_to_bf16_bits(v), g, beta)


def make_delta_dout(num_tokens: int, num_heads: int, head_dim: int, seed: int) -> np.ndarray:
    """bf16 bit pattern [T, H, D] of a standard-normal output gradient."""
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.standard_normal((num_tokens, num_heads, head_dim),
                                                dtype=np.float32))
