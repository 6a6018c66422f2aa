"""Band-block calls (attn_varlen_band_fwd / attn_varlen_band_bwd): bit for bit
the plain calls' results, and the band-block oracle's within the parity bar.

The band formulation (dewml.dev/reference/performance, section "Packed
sliding-window attention on GPU: local_attention") gives every W-token query
block the keys of its own block and the one before; the kernels then loop
over more key blocks (or query blocks) than the rows can see, all masked, so
equality with the plain calls checks that the plain ranges leave out no
visible key."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle.band import band_attention  # noqa: E402
from synthetic import CONFIGS, make_custom, make_microbatch  # noqa: E402

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import varlen_sliding_window_amd as attn  # noqa: E402
    from gpu_common import assert_parity, device_inputs  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run(mb, window, band):
    q, k, v, do, cu = device_inputs(mb)
    ms, sc = mb.max_seqlen, mb.cfg.scale
    out, lse = attn.fwd(q, k, v, cu, ms, window, sc, band=band)
    dq, dk, dv = attn.bwd(q, k, v, out, lse, do, cu, ms, window, sc, band=band)
    torch.cuda.synchronize()
    return {"out": out, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def assert_bitwise(a, b, label):
    for name in ("out", "lse", "dq", "dk", "dv"):
        assert torch.equal(a[name], b[name]), f"{label}: band {name} differs from the plain call"


EDGE_LENGTHS = [1, 7, 8, 9, 63, 64, 65, 127, 128, 129, 333, 1, 511, 512, 513, 2, 31, 32, 33]


def edge_mb(head_dim=128, seed=200):
    cu = np.concatenate([[0], np.cumsum(EDGE_LENGTHS)])
    cu = np.concatenate([[0, 0], cu[1:6], [cu[5]], cu[6:], [cu[-1]]]).astype(np.int32)
    return make_custom(cu, 8, 2, seed=seed, head_dim=head_dim)


@pytest.mark.parametrize("name", ["ctx4096_w512", "ctx512_w512", "tiny_ctx512_w512",
                                  "ctx4096_w512_h16"])
def test_band_equals_plain_config(name):
    cfg = CONFIGS[name]
    mb = make_microbatch(cfg, 0)
    print(f"[case] band {name} W={cfg.window}", flush=True)
    assert_bitwise(run(mb, cfg.window, True), run(mb, cfg.window, False), name)


@pytest.mark.parametrize("window", [1, 3, 33, 64, 100, 512, 5000])
def test_band_equals_plain_edge(window):
    mb = edge_mb()
    print(f"[case] band edge W={window} T={mb.cfg.total_tokens}", flush=True)
    assert_bitwise(run(mb, window, True), run(mb, window, False), f"edge/W{window}")


@pytest.mark.parametrize("head_dim", [64, 256])
def test_band_equals_plain_head_dims(head_dim):
    mb = edge_mb(head_dim, seed=201)
    print(f"[case] band edge D={head_dim} W=64", flush=True)
    assert_bitwise(run(mb, 64, True), run(mb, 64, False), f"edge/D{head_dim}")


@pytest.mark.parametrize("window", [37, 512])
def test_band_parity_tiny(window):
    mb = make_microbatch("tiny_ctx512_w512", 2)
    got = {k_: v_.float().cpu().numpy().astype(np.float64) for k_, v_ in run(mb, window, True).items()}
    out, lse, dq, dk, dv = band_attention(mb.f32("q"), mb.f32("k"), mb.f32("v"), mb.f32("dout"),
                                          mb.cu_seqlens, window, mb.cfg.scale)
    assert_parity(got, {"out": out, "lse": lse, "dq": dq, "dk": dk, "dv": dv},
                  f"band tiny/W{window}")


def test_band_parity_edge():
    mb = edge_mb(seed=202)
    got = {k_: v_.float().cpu().numpy().astype(np.float64) for k_, v_ in run(mb, 33, True).items()}
    out, lse, dq, dk, dv = band_attention(mb.f32("q"), mb.f32("k"), mb.f32("v"), mb.f32("dout"),
                                          mb.cu_seqlens, 33, mb.cfg.scale)
    assert_parity(got, {"out": out, "lse": lse, "dq": dq, "dk": dk, "dv": dv}, "band edge/W33")
