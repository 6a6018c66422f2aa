"""Gated DeltaNet and Kimi Delta layers in the deployment mode of the kernel
benchmarks page (research.dws.rip/llm/kernels, section 06 "CUDA graphs work,
with padding", Fig. 8), which reports that both linear layers matched an
unrecorded run exactly: boundaries padded with empty documents to a fixed
count, one captured forward (saving) + backward (reusing) step replayed while
the boundaries change in place.

Checked here, through the C ABI: repeat runs and padding with empty documents
are bitwise neutral; every graph replay equals the eager step bit for bit;
one replay per gate is also held to the oracle on a sampled document.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle.delta import gated_delta_backward  # noqa: E402
from oracle.kimi_delta import kimi_delta_backward  # noqa: E402
from synthetic import (CONFIGS, bf16_bits_to_f32, make_cu_seqlens, make_delta_dout,  # noqa: E402
                       make_delta_inputs, make_kda_inputs)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import varlen_sliding_window_amd as attn  # noqa: E402
    from gpu_common import FRO_REL, MAX_REL, bits_to_torch, rel_errors  # noqa: E402

T, H, D = 4096, 4, 128
CAPACITY = 24          # documents per microbatch after padding
SCALE = D ** -0.5


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


GATES = {
    "delta": dict(make=make_delta_inputs, fwd="delta_fwd", bwd="delta_bwd",
                  ws="delta_bwd_workspace_size", obwd=gated_delta_backward),
    "kda": dict(make=make_kda_inputs, fwd="kda_fwd", bwd="kda_bwd",
                ws="kda_bwd_workspace_size", obwd=kimi_delta_backward),
}


def boundaries(seed: int) -> np.ndarray:
    """cu_seqlens of the workload's packing at context 1,024 over T tokens,
    padded with empty documents to CAPACITY."""
    cfg = CONFIGS["ctx1024_global"]
    cu, _ = make_cu_seqlens(cfg, seed)
    cu = cu[cu <= T]
    if cu[-1] != T:
        cu = np.append(cu, T)
    n = len(cu) - 1
    assert n <= CAPACITY, n
    out = np.full(CAPACITY + 1, T, dtype=np.int32)
    out[: n + 1] = cu
    return out


class Layer:
    def __init__(self, gate: str, seed: int):
        spec = GATES[gate]
        self.gate, self.spec = gate, spec
        self.inp = spec["make"](np.array([0, T], dtype=np.int32), H, D, seed)
        self.dout_bits = make_delta_dout(T, H, D, seed + 1)
        self.q, self.k, self.v = (bits_to_torch(getattr(self.inp, n + "_bits"))
                                  for n in ("q", "k", "v"))
        self.g = torch.from_numpy(self.inp.g).cuda()
        self.beta = torch.from_numpy(self.inp.beta).cuda()
        self.do = bits_to_torch(self.dout_bits)
        self.cu = torch.empty(CAPACITY + 1, dtype=torch.int32, device="cuda")
        self.ws = torch.empty(getattr(attn, spec["ws"])(T, CAPACITY, H, D), dtype=torch.uint8,
                              device="cuda")
        self.out = torch.empty_like(self.q)
        self.grads = (torch.empty_like(self.q), torch.empty_like(self.k), torch.empty_like(self.v),
                      torch.empty_like(self.g), torch.empty_like(self.beta))

    def buffers(self):
        return (self.out,) + self.grads

    def step(self):
        getattr(attn, self.spec["fwd"])(self.q, self.k, self.v, self.g, self.beta, self.cu, SCALE,
                                        out=self.out, workspace=self.ws, save=True)
        getattr(attn, self.spec["bwd"])(self.q, self.k, self.v, self.g, self.beta, self.do,
                                        self.cu, SCALE, workspace=self.ws, reuse=True,
                                        check_reuse=False, grads=self.grads)

    def oracle_document(self, cu: np.ndarray, s: int):
        lo, hi = int(cu[s]), int(cu[s + 1])
        sl = slice(lo, hi)
        one = np.array([0, hi - lo])
        args = (self.inp.f32("q")[sl], self.inp.f32("k")[sl], self.inp.f32("v")[sl],
                self.inp.g[sl], self.inp.beta[sl])
        res = self.spec["obwd"](*args, bf16_bits_to_f32(self.dout_bits)[sl], one, SCALE)
        return lo, hi, [res[5]] + list(res[:5])   # out, then dq, dk, dv, dg, dbeta


def _equal(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


@pytest.mark.parametrize("gate", sorted(GATES))
def test_repeat_and_padding_are_bitwise_neutral(gate):
    lay = Layer(gate, seed=61)
    cu = boundaries(0)
    n = int(np.searchsorted(cu, T)) + 1      # real entries (through the first T)
    lay.cu.copy_(torch.from_numpy(cu))
    lay.step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in lay.buffers()]
    lay.step()
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(lay.buffers(), ref)):
        assert _equal(a, b), f"{gate}: output {i} differs on a repeat"
    # the same documents with the empty padding moved to the front and middle
    real = cu[:n]
    pad = CAPACITY + 1 - n
    moved = np.concatenate([[0] * (pad // 2), real[:3], [real[2]] * (pad - pad // 2), real[3:]])
    assert len(moved) == CAPACITY + 1
    lay.cu.copy_(torch.from_numpy(moved.astype(np.int32)))
    lay.step()
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(lay.buffers(), ref)):
        assert _equal(a, b), f"{gate}: output {i} changes with empty documents elsewhere"


@pytest.mark.parametrize("gate", sorted(GATES))
def test_graph_replay_matches_eager_and_oracle(gate):
    lay = Layer(gate, seed=71)
    bounds = [boundaries(s) for s in (0, 1, 2)]
    refs = []
    for b in bounds:
        lay.cu.copy_(torch.from_numpy(b))
        lay.step()
        torch.cuda.synchronize()
        refs.append([t.clone() for t in lay.buffers()])

    lay.cu.copy_(torch.from_numpy(bounds[0]))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lay.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lay.step()
    torch.cuda.synchronize()

    for rep, i in enumerate([0, 1, 2, 0, 2, 1]):
        lay.cu.copy_(torch.from_numpy(bounds[i]))
        for t in lay.buffers():
            t.fill_(float("nan"))                # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for j, (got, want) in enumerate(zip(lay.buffers(), refs[i])):
            assert _equal(got, want), f"{gate} replay {rep} (boundaries {i}): output {j} differs"
        if rep == 1:
            # this replay's longest document against the oracle
            cu = bounds[i]
            s = int(np.argmax(np.diff(cu)))
            lo, hi, want = lay.oracle_document(cu, s)
            names = ("out", "dq", "dk", "dv", "dg", "dbeta")
            for name, x, y in zip(names, lay.buffers(), want):
                xv = x[lo:hi].float().cpu().numpy().astype(np.float64)
                mr, fr = rel_errors(xv, np.asarray(y, dtype=np.float64))
                print(f"[parity] {gate} replay, document {s} ({hi - lo} tokens) {name}: "
                      f"max-rel {mr:.2e} fro-rel {fr:.2e}", flush=True)
                assert mr <= MAX_REL and fr <= FRO_REL, name
    del graph
