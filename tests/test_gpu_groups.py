"""Any query/key-value head grouping (Hq % Hkv = 0): the performance reference
page runs 8 query over 4 key-value heads (dewml.dev/reference/performance,
"Attention metadata and the masked conv"), and multi-head (G = 1) and odd
groups are legal shapes of the same call.  The kernels give each 4 query
heads of a group a work-group (waves past the group's last head only stage
key/value blocks) and sum dK/dV over however many heads a group has.

HIP path through the C ABI against the fp64 oracle, whole arrays."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import attention_backward  # noqa: E402
from synthetic import CONFIGS, make_cu_seqlens, make_custom  # noqa: E402

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_common import assert_parity, run_hip  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def oracle(mb, window, softcap=0.0):
    dq, dk, dv, out, lse, _ = attention_backward(mb.f32("q"), mb.f32("k"), mb.f32("v"),
                                                 mb.f32("dout"), mb.cu_seqlens, window,
                                                 mb.cfg.scale, softcap)
    return {"dq": dq, "dk": dk, "dv": dv, "out": out, "lse": lse}


EDGE_LENGTHS = [1, 7, 8, 9, 63, 64, 65, 127, 128, 129, 333, 1, 511, 512, 513, 2, 31, 32, 33]
EDGE_CU = np.concatenate([[0, 0], np.cumsum(EDGE_LENGTHS)]).astype(np.int32)


@pytest.mark.parametrize("hq,hkv", [(8, 4), (8, 8), (6, 2), (12, 2), (5, 1), (3, 3)])
@pytest.mark.parametrize("window", [0, 33])
def test_groups_edge_segments(hq, hkv, window):
    mb = make_custom(EDGE_CU, hq, hkv, seed=200 + hq + 10 * hkv + window)
    print(f"[case] groups {hq}q/{hkv}kv edge window={window}", flush=True)
    got = run_hip(mb, window)
    assert_parity(got, oracle(mb, window), f"{hq}q/{hkv}kv edge/W{window}")


@pytest.mark.parametrize("hq,hkv", [(8, 4), (8, 8)])
@pytest.mark.parametrize("window", [512, 0])
def test_groups_workload(hq, hkv, window):
    """The ctx-4,096 packing of the workload (seed 0) at 8q/4kv and 8q/8kv."""
    cu, _ = make_cu_seqlens(CONFIGS["ctx4096_w512"], 0)
    mb = make_custom(cu, hq, hkv, seed=300 + hkv)
    print(f"[case] groups {hq}q/{hkv}kv ctx4096 window={window}", flush=True)
    got = run_hip(mb, window)
    assert_parity(got, oracle(mb, window), f"{hq}q/{hkv}kv ctx4096/W{window}")


@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("hq,hkv", [(8, 4), (6, 2), (3, 1)])
def test_groups_head_dims(d, hq, hkv):
    """The other head dims' dK/dV kernels (the pipelined one at 64, the wave
    pairs that split the head dim at 256, which must keep their shared
    barriers in step when a pair has fewer heads)."""
    mb = make_custom(EDGE_CU, hq, hkv, seed=400 + d + hq, head_dim=d)
    print(f"[case] groups {hq}q/{hkv}kv d={d} edge window=64", flush=True)
    got = run_hip(mb, 64)
    assert_parity(got, oracle(mb, 64), f"{hq}q/{hkv}kv d{d}")


def test_groups_softcap():
    mb = make_custom(EDGE_CU, 6, 2, seed=501)
    got = run_hip(mb, 0, softcap=3.0)
    assert_parity(got, oracle(mb, 0, 3.0), "6q/2kv cap 3")
