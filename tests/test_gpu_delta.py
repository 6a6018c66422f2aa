"""Gated delta-rule forward (attn_delta_fwd) against the token-by-token fp64
oracle (oracle/delta.py) on seeded inputs: documents of one token, of chunk
edges (63, 64, 65, 128 tokens) and long ones, empty documents, several heads,
and the full 16,384-token microbatch of the attention workload."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle.delta import gated_delta_forward  # noqa: E402
from synthetic import CONFIGS, make_cu_seqlens, make_delta_inputs  # noqa: E402

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import varlen_sliding_window_amd as attn  # noqa: E402
    from gpu_common import FRO_REL, MAX_REL, bits_to_torch, rel_errors  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run(inp, heads, scale):
    q, k, v = (bits_to_torch(getattr(inp, n + "_bits")) for n in ("q", "k", "v"))
    g = torch.from_numpy(inp.g).cuda()
    beta = torch.from_numpy(inp.beta).cuda()
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).cuda()
    out = attn.delta_fwd(q, k, v, g, beta, cu, scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def check(inp, heads, label, scale=128 ** -0.5):
    got = run(inp, heads, scale)
    ref = gated_delta_forward(inp.f32("q"), inp.f32("k"), inp.f32("v"), inp.g, inp.beta,
                              inp.cu_seqlens, scale)
    mr, fr = rel_errors(got, ref)
    print(f"[parity] delta {label}: max-rel {mr:.2e} fro-rel {fr:.2e}", flush=True)
    assert np.all(np.isfinite(got)), label
    assert mr <= MAX_REL and fr <= FRO_REL, f"{label}: max-rel {mr:.3e} fro-rel {fr:.3e}"


EDGE = [1, 63, 64, 65, 2, 128, 129, 7, 300, 1, 33]


def test_delta_edge_documents():
    cu = np.concatenate([[0, 0], np.cumsum(EDGE)[:4], [np.cumsum(EDGE)[3]], np.cumsum(EDGE)[4:]])
    inp = make_delta_inputs(np.concatenate([[0], cu[1:]]).astype(np.int32), 2, 128, seed=11)
    check(inp, 2, f"edge T={int(cu[-1])}")


@pytest.mark.parametrize("heads", [1, 4])
def test_delta_one_long_document(heads):
    inp = make_delta_inputs(np.array([0, 1000], dtype=np.int32), heads, 128, seed=12 + heads)
    check(inp, heads, f"one 1000-token document, H={heads}")


def test_delta_workload_microbatch():
    cu, _ = make_cu_seqlens(CONFIGS["ctx4096_w512"], 0)
    inp = make_delta_inputs(cu, 8, 128, seed=0)
    check(inp, 8, "ctx 4,096 microbatch, T=16,384, H=8")


def test_delta_deterministic_and_scale():
    inp = make_delta_inputs(np.array([0, 70, 200], dtype=np.int32), 2, 128, seed=14)
    a = run(inp, 2, 0.3)
    b = run(inp, 2, 0.3)
    assert np.array_equal(a, b)
    check(inp, 2, "scale 0.3", scale=0.3)
