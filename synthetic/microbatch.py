"""Seeded synthetic microbatches for packed, document-masked attention.

This module only draws inputs. It holds none of the attention arithmetic, so
both the CPU oracle (``oracle/``) and the GPU path's tests and bench can use
it without sharing any of the method's code.

What it stands in for
---------------------
The kernel benchmarks page (research.dws.rip/llm/kernels, section 01 "How it
was measured", and Fig. 2 "Benchmark setup") times attention on 16,384-token
microbatches cut from real token shards: attention is confined to each
document, rows end every 512 to 4,096 tokens (the context length), the
median document is 457 tokens and almost half of the tokens sit in long
documents. Those shards are not available, so this generator draws document
lengths from a lognormal with median 457 and sigma 1.6 instead, lays the
documents end to end in one stream, and cuts a microbatch out of it.

Recipe (all draws from one ``numpy.random.default_rng(seed)``, PCG64):

1. Document lengths: ``rint(lognormal(mean=ln 457, sigma=1.6))`` clipped to
   [8, 65,536], drawn in chunks of 4,096 until the stream is at least
   ``BURN_IN + T`` tokens long.
2. The microbatch is stream tokens ``[BURN_IN, BURN_IN + T)`` with
   ``BURN_IN = 65,536`` (the clip maximum, so the slice start is stationary).
   Segments are cut at every row end (multiples of ``ctx`` inside the
   microbatch) and at every document end.  The result is ``cu_seqlens``
   (int32, non-decreasing, first 0, last T).
3. Then, in this order, ``standard_normal`` float32 draws for q [T, Hq, d],
   k [T, Hkv, d], v [T, Hkv, d] and dout [T, Hq, d], each rounded to bf16
   with round-to-nearest-even.  The bf16 values are returned both as raw
   16-bit patterns (what the GPU reads) and as exactly equal float32 arrays
   (what the oracle reads).

For a layer stack, layer ``l`` of seed ``s`` draws its tensors from seed
``1000*s + l`` while keeping the ``cu_seqlens`` of seed ``s``.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

BURN_IN = 65536
DOC_MEDIAN = 457
DOC_SIGMA = 1.6
DOC_MIN = 8
DOC_MAX = 65536
HEAD_DIM = 128


@dataclasses.dataclass(frozen=True)
class Config:
    """One workload shape: packing context, window and head layout."""

    name: str
    total_tokens: int
    ctx: int
    window: int          # <= 0 means full causal context inside each document
    num_q_heads: int = 8
    num_kv_heads: int = 2
    head_dim: int = HEAD_DIM

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


# The workloads of the kernel benchmarks page (Fig. 2 setup, Figs. 3 and 4
# timings): 16,384-token microbatches, 8 query / 2 key-value heads of 128,
# a 512-token window on local layers, full causal context on global layers.
CONFIGS = {
    "tiny_ctx512_w512": Config("tiny_ctx512_w512", 1024, 512, 512),
    "ctx512_w512": Config("ctx512_w512", 16384, 512, 512),
    "ctx4096_w512": Config("ctx4096_w512", 16384, 4096, 512),
    "ctx4096_global": Config("ctx4096_global", 16384, 4096, 0),
    "ctx1024_global": Config("ctx1024_global", 16384, 1024, 0),
    "ctx2048_global": Config("ctx2048_global", 16384, 2048, 0),
    "ctx1024_w512": Config("ctx1024_w512", 16384, 1024, 512),
    "ctx2048_w512": Config("ctx2048_w512", 16384, 2048, 512),
    "ctx4096_w512_h16": Config("ctx4096_w512_h16", 16384, 4096, 512, 16, 4),
    "ctx4096_global_h16": Config("ctx4096_global_h16", 16384, 4096, 0, 16, 4),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return bits.

    Inputs here are finite normal draws, so NaN handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding_bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding_bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw_document_lengths(rng: np.random.Generator, need: int) -> np.ndarray:
    """Draw lognormal document lengths until their sum reaches ``need``."""
    chunks = []
    total = 0
    while total < need:
        raw = rng.lognormal(mean=math.log(DOC_MEDIAN), sigma=DOC_SIGMA, size=4096)
        lens = np.clip(np.rint(raw), DOC_MIN, DOC_MAX).astype(np.int64)
        chunks.append(lens)
        total += int(lens.sum())
    return np.concatenate(chunks)


def pack_cu_seqlens(doc_lengths: np.ndarray, total_tokens: int, ctx: int,
                    burn_in: int = BURN_IN) -> np.ndarray:
    """Cut stream tokens [burn_in, burn_in+T) at row ends and document ends."""
    ends = np.cumsum(doc_lengths)  # stream positions where documents end
    lo, hi = burn_in, burn_in + total_tokens
    cuts = set(range(0, total_tokens + 1, ctx))
    cuts.add(total_tokens)
    inside = ends[(ends > lo) & (ends < hi)] - lo
    cuts.update(int(c) for c in inside)
    return np.array(sorted(cuts), dtype=np.int32)


def round_bf16(rng: np.random.Generator, shape) -> tuple[np.ndarray, np.ndarray]:
    bits = f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
    return bits, bf16_bits_to_f32(bits)


@dataclasses.dataclass
class Microbatch:
    cfg: Config
    seed: int
    cu_seqlens: np.ndarray          # int32 [num_seqs + 1]
    q_bits: np.ndarray              # uint16 [T, Hq, d]   (bf16 patterns)
    k_bits: np.ndarray              # uint16 [T, Hkv, d]
    v_bits: np.ndarray
    dout_bits: np.ndarray           # uint16 [T, Hq, d]

    @property
    def max_seqlen(self) -> int:
        return int(np.diff(self.cu_seqlens).max()) if len(self.cu_seqlens) > 1 else 0

    @property
    def num_seqs(self) -> int:
        return len(self.cu_seqlens) - 1

    def f32(self, name: str) -> np.ndarray:
        return bf16_bits_to_f32(getattr(self, name + "_bits"))


def make_cu_seqlens(cfg: Config, seed: int) -> tuple[np.ndarray, np.random.Generator]:
    rng = np.random.default_rng(seed)
    lens = draw_document_lengths(rng, BURN_IN + cfg.total_tokens)
    return pack_cu_seqlens(lens, cfg.total_tokens, cfg.ctx), rng


def make_tensors(cfg: Config, rng: np.random.Generator, total_tokens: int | None = None):
    t = cfg.total_tokens if total_tokens is None else total_tokens
    d = cfg.head_dim
    q, _ = round_bf16(rng, (t, cfg.num_q_heads, d))
    k, _ = round_bf16(rng, (t, cfg.num_kv_heads, d))
    v, _ = round_bf16(rng, (t, cfg.num_kv_heads, d))
    do, _ = round_bf16(rng, (t, cfg.num_q_heads, d))
    return q, k, v, do


def make_microbatch(cfg: Config | str, seed: int) -> Microbatch:
    """The seeded microbatch of ``cfg`` (a Config or a CONFIGS key)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    cu, rng = make_cu_seqlens(cfg, seed)
    q, k, v, do = make_tensors(cfg, rng)
    return Microbatch(cfg, seed, cu, q, k, v, do)


def make_layer(cfg: Config, seed: int, layer: int, cu_seqlens: np.ndarray) -> Microbatch:
    """Layer ``layer`` of a stack: tensors from seed 1000*seed+layer, fixed boundaries."""
    rng = np.random.default_rng(1000 * seed + layer)
    q, k, v, do = make_tensors(cfg, rng)
    return Microbatch(cfg, seed, np.asarray(cu_seqlens, dtype=np.int32), q, k, v, do)


def make_custom(cu_seqlens, num_q_heads: int, num_kv_heads: int, seed: int,
                head_dim: int = HEAD_DIM, window: int = 0, name: str = "custom") -> Microbatch:
    """Hand-built boundaries (edge cases) with seeded N(0,1) bf16 tensors."""
    cu = np.asarray(cu_seqlens, dtype=np.int32)
    t = int(cu[-1])
    cfg = Config(name, t, max(t, 1), window, num_q_heads, num_kv_heads, head_dim)
    rng = np.random.default_rng(seed)
    q, k, v, do = make_tensors(cfg, rng)
    return Microbatch(cfg, seed, cu, q, k, v, do)
