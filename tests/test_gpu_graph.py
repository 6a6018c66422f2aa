"""Graph capture and replay of forward + backward with fixed-capacity
cu_seqlens (the deployment mode of the kernel benchmarks page,
research.dws.rip/llm/kernels, section 06 and Fig. 8: boundaries padded with
empty documents to a fixed count, so that one recorded graph serves every
microbatch).

The library allocates nothing and never synchronises with the host, so a
whole fwd + bwd call sequence can be captured once and replayed while the
caller rewrites the boundary list in place between replays.  Each replay
must equal an eager run on the same boundaries bit for bit.  Replays are
interleaved with eager work and host synchronisations, and every replay is
checked, as graphs of this kind are known to go wrong only on later replays;
one later replay is also held to the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import varlen_sliding_window_amd as attn
from synthetic import CONFIGS, make_cu_seqlens, make_custom

from gpu_common import assert_parity, bits_to_torch
from oracle import attention_backward

pytestmark = pytest.mark.gpu

CAPACITY = 80   # documents per microbatch after padding (sample sizes: 4 to 67)


def padded_boundaries(cfg_name: str, seed: int, capacity: int = CAPACITY) -> np.ndarray:
    cu, _ = make_cu_seqlens(CONFIGS[cfg_name], seed)
    n = len(cu) - 1
    assert n <= capacity
    out = np.full(capacity + 1, cu[-1], dtype=np.int32)
    out[: n + 1] = cu
    return out


@pytest.mark.parametrize("window,reuse", [(512, False), (0, False), (512, True)])
def test_graph_replay_matches_eager(window, reuse):
    cfg = CONFIGS["ctx4096_w512"]
    T, hq, hkv, d = cfg.total_tokens, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    # tensors from one seed; boundaries from several (all pad to CAPACITY)
    mb = make_custom(np.array([0, T], dtype=np.int32), hq, hkv, seed=11)
    dev = "cuda"
    q, k, v, do = (bits_to_torch(b, dev) for b in (mb.q_bits, mb.k_bits, mb.v_bits, mb.dout_bits))
    cu = torch.empty(CAPACITY + 1, dtype=torch.int32, device=dev)
    scale = cfg.scale
    out = torch.empty_like(q)
    lse = torch.empty((hq, T), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = attn.new_workspace(T, CAPACITY, hq, hkv, d, T, window, dev)
    outs = (out, lse, dq, dk, dv)

    def step():
        attn.fwd(q, k, v, cu, T, window, scale, out=out, lse=lse, workspace=ws)
        attn.bwd(q, k, v, out, lse, do, cu, T, window, scale, dq=dq, dk=dk, dv=dv, workspace=ws,
                 reuse_schedule=reuse)

    def set_boundaries(b: np.ndarray):
        cu.copy_(torch.from_numpy(b))

    bounds = [padded_boundaries("ctx4096_w512", s) for s in (0, 1, 2)]
    bounds.append(padded_boundaries("ctx512_w512", 0))

    # eager references for each boundary set
    refs = []
    for b in bounds:
        set_boundaries(b)
        step()
        torch.cuda.synchronize()
        refs.append([t.clone() for t in outs])

    # capture once (warm-up on a side stream first, as graph capture asks)
    set_boundaries(bounds[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    order = [0, 1, 2, 3, 0, 2, 1, 3]
    for rep, i in enumerate(order):
        set_boundaries(bounds[i])
        for t in outs:
            t.fill_(float("nan"))          # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("out", "lse", "dq", "dk", "dv"), outs, refs[i]):
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                               want.view(torch.int16) if want.dtype == torch.bfloat16 else want), \
                f"replay {rep} (boundaries {i}, window {window}): {name} differs from eager"
        if rep == 4:
            # a later replay (boundary set 0, the workload's ctx-4,096 packing)
            # against the oracle, whole arrays
            got = {n: t.float().cpu().numpy().astype(np.float64)
                   for n, t in zip(("out", "lse", "dq", "dk", "dv"), outs)}
            dq_r, dk_r, dv_r, out_r, lse_r, _ = attention_backward(
                mb.f32("q"), mb.f32("k"), mb.f32("v"), mb.f32("dout"), bounds[i], window, scale)
            assert_parity(got, {"dq": dq_r, "dk": dk_r, "dv": dv_r, "out": out_r, "lse": lse_r},
                          f"graph replay {rep}, window {window}")
