"""Head dims other than 128 against the fp64 oracle.

The performance reference page (dewml.dev/reference/performance, section
"Head dimension 256 through tokamax's Triton flash attention") expects a
training attention kernel to take any power-of-two head dimension with
grouped query heads, causal masks and windows; these cases run the kernels'
head-dim instantiations on the workload's packed boundaries and on the edge
cases, with the default scale 1 / sqrt(D)."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import attention_backward  # noqa: E402
from synthetic import CONFIGS, make_cu_seqlens, make_custom  # noqa: E402

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_common import assert_parity, run_hip  # noqa: E402

HEAD_DIMS = [64, 256]


def oracle(mb, window, softcap=0.0):
    dq, dk, dv, out, lse, _ = attention_backward(mb.f32("q"), mb.f32("k"), mb.f32("v"),
                                                 mb.f32("dout"), mb.cu_seqlens, window,
                                                 mb.cfg.scale, softcap)
    return {"dq": dq, "dk": dk, "dv": dv, "out": out, "lse": lse}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("d", HEAD_DIMS)
@pytest.mark.parametrize("name,hq,hkv", [
    ("tiny_ctx512_w512", 8, 2),
    ("ctx512_w512", 8, 2),
    ("ctx4096_w512", 8, 2),
    ("ctx4096_global", 8, 2),
    ("ctx4096_w512", 16, 4),
])
def test_headdim_parity_config(d, name, hq, hkv):
    cfg = CONFIGS[name]
    cu, _ = make_cu_seqlens(cfg, 0)
    mb = make_custom(cu, hq, hkv, seed=300 + d, head_dim=d, window=cfg.window)
    print(f"[case] D={d} {name} {hq}q/{hkv}kv W={cfg.window} segs={len(cu) - 1}", flush=True)
    got = run_hip(mb, cfg.window)
    assert_parity(got, oracle(mb, cfg.window), f"D{d}/{name}/{hq}q{hkv}kv")


EDGE_LENGTHS = [1, 7, 8, 9, 63, 64, 65, 127, 128, 129, 333, 1, 511, 512, 513, 2, 31, 32, 33]


@pytest.mark.parametrize("d", HEAD_DIMS)
@pytest.mark.parametrize("window", [0, 1, 3, 64, 512])
def test_headdim_edge_segments(d, window):
    cu = np.concatenate([[0], np.cumsum(EDGE_LENGTHS)])
    cu = np.concatenate([[0, 0], cu[1:6], [cu[5]], cu[6:], [cu[-1]]]).astype(np.int32)
    mb = make_custom(cu, 8, 2, seed=400 + window, head_dim=d)
    print(f"[case] D={d} edge window={window} T={int(cu[-1])}", flush=True)
    got = run_hip(mb, window)
    assert_parity(got, oracle(mb, window), f"D{d} edge/W{window}")


@pytest.mark.parametrize("d", HEAD_DIMS)
def test_headdim_softcap(d):
    cu, _ = make_cu_seqlens(CONFIGS["ctx512_w512"], 1)
    mb = make_custom(cu, 8, 2, seed=500 + d, head_dim=d)
    print(f"[case] D={d} softcap 1.5 W=512", flush=True)
    got = run_hip(mb, 512, softcap=1.5)
    assert_parity(got, oracle(mb, 512, 1.5), f"D{d} cap 1.5")


@pytest.mark.parametrize("d", HEAD_DIMS)
def test_headdim_single_token(d):
    mb = make_custom([0, 1], 4, 1, seed=6, head_dim=d)
    got = run_hip(mb, 0)
    np.testing.assert_array_equal(got["out"], oracle(mb, 0)["out"])   # out = v exactly
