"""A backward call that reuses the forward call's tile schedule
(ATTN_BWD_REUSE_SCHEDULE) gives the same results, bit for bit, as one that
rebuilds it; with a schedule built for another window the kernels leave the
outputs untouched (the device-side check of the workspace header)."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import varlen_sliding_window_amd as attn  # noqa: E402
from synthetic import make_microbatch  # noqa: E402

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_common import device_inputs  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _views(x):
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)


@pytest.mark.parametrize("name,softcap", [("ctx4096_w512", 0.0), ("ctx4096_global", 0.0),
                                          ("ctx512_w512", 3.0)])
def test_reused_schedule_is_bitwise_equal(name, softcap):
    mb = make_microbatch(name, 2)
    q, k, v, do, cu = device_inputs(mb)
    t, hq, d = q.shape
    w, sc, ms = mb.cfg.window, mb.cfg.scale, mb.max_seqlen
    print(f"[case] reuse {name} cap={softcap}", flush=True)
    ws = attn.new_workspace(t, mb.num_seqs, hq, k.shape[1], d, ms, w, q.device)
    out, lse = attn.fwd(q, k, v, cu, ms, w, sc, workspace=ws, softcap=softcap)
    got = attn.bwd(q, k, v, out, lse, do, cu, ms, w, sc, workspace=ws, softcap=softcap,
                   reuse_schedule=True)
    ref = attn.bwd(q, k, v, out, lse, do, cu, ms, w, sc, softcap=softcap)
    torch.cuda.synchronize()
    for name_, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(_views(a), _views(b)), f"{name_} differs with a reused schedule"


def test_schedule_for_another_window_is_refused_on_device():
    mb = make_microbatch("tiny_ctx512_w512", 3)
    q, k, v, do, cu = device_inputs(mb)
    t, hq, d = q.shape
    sc, ms = mb.cfg.scale, mb.max_seqlen
    ws = attn.new_workspace(t, mb.num_seqs, hq, k.shape[1], d, ms, 512, q.device)
    out, lse = attn.fwd(q, k, v, cu, ms, 0, sc)              # outputs for window 0
    attn.fwd(q, k, v, cu, ms, 64, sc, workspace=ws)          # schedule for window 64
    dq, dk, dv = (torch.full_like(x, float("nan")) for x in (q, k, v))
    attn.bwd(q, k, v, out, lse, do, cu, ms, 0, sc, dq=dq, dk=dk, dv=dv, workspace=ws,
             reuse_schedule=True)
    torch.cuda.synchronize()
    for x in (dq, dk, dv):
        assert torch.isnan(x.float()).all(), "kernels ran on a schedule built for another window"
    # the same call without the flag rebuilds the schedule and fills them
    attn.bwd(q, k, v, out, lse, do, cu, ms, 0, sc, dq=dq, dk=dk, dv=dv, workspace=ws)
    torch.cuda.synchronize()
    for x in (dq, dk, dv):
        assert torch.isfinite(x.float()).all()
