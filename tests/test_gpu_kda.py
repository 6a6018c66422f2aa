"""Kimi Delta Attention forward (attn_kda_fwd) against the token-by-token
fp64 oracle (oracle/kimi_delta.py) on seeded inputs: chunk-edge and empty
documents, a long document, several heads, the full 16,384-token
microbatch, a gate equal on every channel (which must give the Gated
DeltaNet kernel's result) and strong decays."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle.kimi_delta import kimi_delta_forward  # noqa: E402
from synthetic import CONFIGS, make_cu_seqlens, make_kda_inputs  # noqa: E402

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import varlen_sliding_window_amd as attn  # noqa: E402
    from gpu_common import FRO_REL, MAX_REL, bits_to_torch, rel_errors  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run(inp, scale, g=None):
    q, k, v = (bits_to_torch(getattr(inp, n + "_bits")) for n in ("q", "k", "v"))
    gt = torch.from_numpy(inp.g if g is None else g).cuda()
    beta = torch.from_numpy(inp.beta).cuda()
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).cuda()
    out = attn.kda_fwd(q, k, v, gt, beta, cu, scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def check(inp, label, scale=128 ** -0.5, g=None):
    got = run(inp, scale, g)
    gg = inp.g if g is None else g
    ref = kimi_delta_forward(inp.f32("q"), inp.f32("k"), inp.f32("v"), gg, inp.beta,
                             inp.cu_seqlens, scale)
    mr, fr = rel_errors(got, ref)
    print(f"[parity] kda {label}: max-rel {mr:.2e} fro-rel {fr:.2e}", flush=True)
    assert np.all(np.isfinite(got)), label
    assert mr <= MAX_REL and fr <= FRO_REL, f"{label}: max-rel {mr:.3e} fro-rel {fr:.3e}"


EDGE = [1, 63, 64, 65, 2, 128, 129, 7, 300, 1, 33]


def test_kda_edge_documents():
    c = np.cumsum(EDGE)
    cu = np.concatenate([[0, 0], c[:4], [c[3]], c[4:]]).astype(np.int32)
    check(make_kda_inputs(cu, 2, 128, seed=31), f"edge T={int(cu[-1])}")


@pytest.mark.parametrize("heads", [1, 4])
def test_kda_one_long_document(heads):
    check(make_kda_inputs(np.array([0, 1000], dtype=np.int32), heads, 128, seed=32 + heads),
          f"one 1000-token document, H={heads}")


def test_kda_workload_microbatch():
    cu, _ = make_cu_seqlens(CONFIGS["ctx4096_w512"], 0)
    check(make_kda_inputs(cu, 8, 128, seed=0), "ctx 4,096 microbatch, T=16,384, H=8")


def test_kda_strong_decay():
    # per-token decays down to 0.05 on some channels: the chunk's cumulative
    # decay underflows to zero there, which the factored products must survive
    inp = make_kda_inputs(np.array([0, 150, 300], dtype=np.int32), 2, 128, seed=35)
    rng = np.random.default_rng(36)
    g = np.log(rng.uniform(0.05, 1.0, size=inp.g.shape)).astype(np.float32)
    check(inp, "strong decay", g=g)


def test_kda_equal_channels_match_the_scalar_gate_kernel():
    inp = make_kda_inputs(np.array([0, 90, 300], dtype=np.int32), 2, 128, seed=37)
    gs = inp.g[..., 0].copy()
    g = np.repeat(gs[..., None], 128, axis=-1)
    got = run(inp, 0.1, g)
    q, k, v = (bits_to_torch(getattr(inp, n + "_bits")) for n in ("q", "k", "v"))
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).cuda()
    ref = attn.delta_fwd(q, k, v, torch.from_numpy(gs).cuda(), torch.from_numpy(inp.beta).cuda(),
                         cu, 0.1).float().cpu().numpy()
    mr, fr = rel_errors(got, ref.astype(np.float64))
    print(f"[parity] kda equal channels vs delta_fwd: max-rel {mr:.2e} fro-rel {fr:.2e}", flush=True)
    assert mr <= MAX_REL and fr <= FRO_REL
