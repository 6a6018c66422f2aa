"""Logit soft-cap (attn_varlen_fwd_ex / attn_varlen_bwd_ex, softcap > 0)
against the fp64 oracle: every logit S becomes c tanh(S / c) before the
softmax and the backward carries 1 - tanh^2 (the Gemma 2 attention cap that
the performance reference page, dewml.dev/reference/performance, lists in
its section on head dimension 256 through tokamax's Triton flash attention).

Caps range from strongly nonlinear (c below the logits' spread) to far
above every logit; some cases raise the scale so that tanh saturates."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import attention_backward  # noqa: E402
from synthetic import CONFIGS, make_custom, make_microbatch  # noqa: E402

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_common import assert_parity, raw_outputs, run_hip  # noqa: E402


def oracle(mb, window, scale, softcap, cu=None):
    cu = mb.cu_seqlens if cu is None else cu
    dq, dk, dv, out, lse, _ = attention_backward(mb.f32("q"), mb.f32("k"), mb.f32("v"),
                                                 mb.f32("dout"), cu, window, scale, softcap)
    return {"dq": dq, "dk": dk, "dv": dv, "out": out, "lse": lse}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("name,cap,scale_mul", [
    ("tiny_ctx512_w512", 1.5, 1.0),
    ("tiny_ctx512_w512", 5.0, 8.0),
    ("ctx512_w512", 0.75, 1.0),
    ("ctx4096_w512", 2.0, 1.0),
    ("ctx4096_global", 30.0, 8.0),
    ("ctx4096_w512_h16", 50.0, 4.0),
    ("ctx4096_global_h16", 20.0, 4.0),
])
def test_softcap_parity_config(name, cap, scale_mul):
    cfg = CONFIGS[name]
    mb = make_microbatch(cfg, 0)
    scale = cfg.scale * scale_mul
    print(f"[case] softcap {name} seed 0 cap={cap} scale={scale:.4f}", flush=True)
    got = run_hip(mb, cfg.window, softcap=cap, scale=scale)
    assert_parity(got, oracle(mb, cfg.window, scale, cap), f"{name}/cap{cap}")


EDGE_LENGTHS = [1, 7, 8, 9, 63, 64, 65, 127, 128, 129, 333, 1, 511, 512, 513, 2, 31, 32, 33]


@pytest.mark.parametrize("window", [0, 3, 64, 512])
def test_softcap_edge_segments(window):
    cu = np.concatenate([[0], np.cumsum(EDGE_LENGTHS)])
    cu = np.concatenate([[0, 0], cu[1:6], [cu[5]], cu[6:], [cu[-1]]]).astype(np.int32)
    mb = make_custom(cu, 8, 2, seed=200 + window)
    print(f"[case] softcap edge window={window} T={int(cu[-1])}", flush=True)
    got = run_hip(mb, window, softcap=1.0)
    assert_parity(got, oracle(mb, window, mb.cfg.scale, 1.0), f"cap edge/W{window}")


def test_softcap_far_above_logits_is_uncapped():
    """c tanh(S / c) -> S as c grows: a cap of 1e6 meets the uncapped oracle."""
    mb = make_microbatch("tiny_ctx512_w512", 3)
    got = run_hip(mb, 512, softcap=1e6)
    assert_parity(got, oracle(mb, 512, mb.cfg.scale, 0.0), "cap 1e6 vs uncapped")


def test_softcap_changes_the_result():
    """A cap inside the logits' range must move the outputs (the cap is applied)."""
    mb = make_microbatch("tiny_ctx512_w512", 4)
    capped = run_hip(mb, 512, softcap=0.5, scale=1.0)
    plain = run_hip(mb, 512, scale=1.0)
    assert np.max(np.abs(capped["out"] - plain["out"])) > 0.1
    assert_parity(capped, oracle(mb, 512, 1.0, 0.5), "cap 0.5 scale 1")


def test_softcap_padding_is_bitwise_neutral_and_deterministic():
    mb = make_microbatch("ctx512_w512", 5)
    cu = mb.cu_seqlens
    a = raw_outputs(mb, 512, softcap=3.0)
    b = raw_outputs(mb, 512, softcap=3.0)
    padded = np.concatenate([cu, np.full(20, cu[-1], dtype=np.int32)])
    c = raw_outputs(mb, 512, cu=padded, softcap=3.0)
    for other, label in ((b, "repeat"), (c, "padded")):
        for name in ("out", "lse", "dq", "dk", "dv"):
            x, y = a[name], other[name]
            view = torch.int16 if x.dtype == torch.bfloat16 else torch.int32
            assert torch.equal(x.view(view), y.view(view)), f"cap {label}: {name} differs"
