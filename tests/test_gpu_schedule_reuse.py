"""Schedule reuse and boundary checks: a backward call that reuses the
forward call's tile schedule (ATTN_BWD_REUSE_SCHEDULE), and the layers of a
stack that share one schedule (ATTN_FWD_REUSE_SCHEDULE), give the same
results, bit for bit, as calls that rebuild it; a schedule built for another
window is refused by the binding and, on the device, turns every output into
NaN; malformed boundaries do the same."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import varlen_sliding_window_amd as attn  # noqa: E402
from synthetic import CONFIGS, make_cu_seqlens, make_layer, make_microbatch  # noqa: E402

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


def test_schedule_for_another_window_is_refused():
    mb = make_microbatch("tiny_ctx512_w512", 3)
    q, k, v, do, cu = device_inputs(mb)
    t, hq, d = q.shape
    sc, ms = mb.cfg.scale, mb.max_seqlen
    ws = attn.new_workspace(t, mb.num_seqs, hq, k.shape[1], d, ms, 512, q.device)
    out, lse = attn.fwd(q, k, v, cu, ms, 0, sc)              # outputs for window 0
    attn.fwd(q, k, v, cu, ms, 64, sc, workspace=ws)          # schedule for window 64
    # the binding's record of the workspace refuses the call on the host
    with pytest.raises(ValueError):
        attn.bwd(q, k, v, out, lse, do, cu, ms, 0, sc, workspace=ws, reuse_schedule=True)
    with pytest.raises(ValueError):
        attn.fwd(q, k, v, cu, ms, 0, sc, workspace=ws, reuse_schedule=True)
    # the device-side check: every output of the call becomes NaN
    dq, dk, dv = (torch.zeros_like(x) for x in (q, k, v))
    attn.bwd(q, k, v, out, lse, do, cu, ms, 0, sc, dq=dq, dk=dk, dv=dv, workspace=ws,
             reuse_schedule=True, check_reuse=False)
    o2, l2 = torch.zeros_like(out), torch.zeros_like(lse)
    attn.fwd(q, k, v, cu, ms, 0, sc, out=o2, lse=l2, workspace=ws, reuse_schedule=True,
             check_reuse=False)
    torch.cuda.synchronize()
    for x in (dq, dk, dv, o2, l2):
        assert torch.isnan(x.float()).all(), "kernels ran on a schedule built for another window"
    # the same calls without the flag rebuild the schedule and fill them
    attn.bwd(q, k, v, out, lse, do, cu, ms, 0, sc, dq=dq, dk=dk, dv=dv, workspace=ws)
    attn.fwd(q, k, v, cu, ms, 0, sc, out=o2, lse=l2, workspace=ws)
    torch.cuda.synchronize()
    for x in (dq, dk, dv, o2, l2):
        assert torch.isfinite(x.float()).all()


@pytest.mark.parametrize("window", [512, 0])
def test_one_schedule_serves_a_stack_of_layers(window):
    """Layers that share cu_seqlens and the window (the per-microbatch stack of
    15 local + 5 global layers) may build the schedule once: every later
    forward and backward reuses it, with results equal bit for bit to calls
    that rebuild it."""
    name = "ctx4096_w512" if window else "ctx4096_global"
    cfg = CONFIGS[name]
    cu_np, _ = make_cu_seqlens(cfg, 4)
    ws = None
    for layer in range(3):
        mb = make_layer(cfg, 4, layer, cu_np)
        q, k, v, do, cu = device_inputs(mb)
        t, hq, d = q.shape
        sc, ms = cfg.scale, mb.max_seqlen
        if ws is None:
            ws = attn.new_workspace(t, mb.num_seqs, hq, k.shape[1], d, ms, window, q.device)
        out, lse = attn.fwd(q, k, v, cu, ms, window, sc, workspace=ws,
                            reuse_schedule=layer > 0)
        got = attn.bwd(q, k, v, out, lse, do, cu, ms, window, sc, workspace=ws,
                       reuse_schedule=True)
        ref_out, ref_lse = attn.fwd(q, k, v, cu, ms, window, sc)
        ref = attn.bwd(q, k, v, ref_out, ref_lse, do, cu, ms, window, sc)
        torch.cuda.synchronize()
        for name_, a, b in zip(("out", "lse", "dq", "dk", "dv"), (out, lse) + got,
                               (ref_out, ref_lse) + ref):
            assert torch.equal(_views(a), _views(b)), f"layer {layer}: {name_} differs"


@pytest.mark.parametrize("case", ["first_not_zero", "decreasing", "last_not_T"])
def test_malformed_boundaries_give_nan_outputs(case):
    """Boundaries that break cu[0] = 0, non-decreasing or cu[n] = T are caught
    by the schedule kernel on the device: every output of the call is NaN (the
    kernels stay inside their buffers, and nothing waits for the host)."""
    mb = make_microbatch("tiny_ctx512_w512", 9)
    q, k, v, do, cu = device_inputs(mb)
    t = q.shape[0]
    bad = {"first_not_zero": [5, 300, 700, t], "decreasing": [0, 300, 200, t],
           "last_not_T": [0, 300, 700, t - 3]}[case]
    bad = np.asarray(bad, dtype=np.int32)
    cu_bad = torch.from_numpy(bad).cuda()
    print(f"[case] malformed cu_seqlens ({case}): {bad.tolist()}", flush=True)
    out, lse = attn.fwd(q, k, v, cu_bad, t, 512, mb.cfg.scale)
    good_out, good_lse = attn.fwd(q, k, v, cu, mb.max_seqlen, 512, mb.cfg.scale)
    dq, dk, dv = attn.bwd(q, k, v, good_out, good_lse, do, cu_bad, t, 512, mb.cfg.scale)
    torch.cuda.synchronize()
    for name_, x in (("out", out), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.isnan(x.float()).all(), f"{case}: {name_} not NaN"


@pytest.mark.parametrize("name", ["ctx4096_w512", "ctx4096_global"])
def test_schedule_built_ahead_on_another_stream(name):
    """attn_varlen_schedule on a second stream, ordered by an event before a
    forward and backward that reuse it: bit for bit the calls that build
    their own; rebuilt while the first stream still runs an earlier pair of
    calls on another workspace."""
    mb = make_microbatch(name, 4)
    q, k, v, do, cu = device_inputs(mb)
    t, hq, d = q.shape
    w, sc, ms = mb.cfg.window, mb.cfg.scale, mb.max_seqlen
    print(f"[case] schedule ahead {name}", flush=True)
    out0, lse0 = attn.fwd(q, k, v, cu, ms, w, sc)
    ref = attn.bwd(q, k, v, out0, lse0, do, cu, ms, w, sc)
    ws = attn.new_workspace(t, mb.num_seqs, hq, k.shape[1], d, ms, w, q.device)
    ws.fill_(0x5A)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(main)
    for rep in range(2):
        other = attn.fwd(q, k, v, cu, ms, w, sc)             # busy work on the first stream
        with torch.cuda.stream(side):
            attn.schedule(cu, t, ms, w, ws, hq, k.shape[1], d)
            ready = torch.cuda.Event()
            ready.record(side)
        main.wait_event(ready)
        out, lse = attn.fwd(q, k, v, cu, ms, w, sc, workspace=ws, reuse_schedule=True)
        got = attn.bwd(q, k, v, out, lse, do, cu, ms, w, sc, workspace=ws, reuse_schedule=True)
        done = torch.cuda.Event()
        done.record(main)
        side.wait_event(done)                                # before the next rebuild
        torch.cuda.synchronize()
        assert torch.equal(_views(out), _views(out0)), f"out differs (rep {rep})"
        assert torch.equal(_views(lse), _views(lse0)), f"lse differs (rep {rep})"
        for name_, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(_views(a), _views(b)), f"{name_} differs (rep {rep})"
        del other
