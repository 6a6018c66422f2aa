"""attn_varlen_bwd_static, the backward that allocates nothing (its
workspace is the library's static device scratch), against attn_varlen_bwd
with a caller workspace: bit for bit, on two calls in a row, the second on a
smaller problem (the scratch keeps the first call's contents), and again
after an ordinary backward has run."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from synthetic import make_custom, make_microbatch  # noqa: E402

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import varlen_sliding_window_amd as attn  # noqa: E402
    from gpu_common import device_inputs  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bits(x):
    return x.view(torch.int16)


def _check(mb, window, label):
    q, k, v, do, cu = device_inputs(mb)
    ms, sc = mb.max_seqlen, mb.cfg.scale
    out, lse = attn.fwd(q, k, v, cu, ms, window, sc)
    ref = attn.bwd(q, k, v, out, lse, do, cu, ms, window, sc)
    dq, dk, dv = (torch.full_like(x, float("nan")) for x in (q, k, v))
    torch.cuda.synchronize()
    print(f"[case] bwd_static {label}: T={q.shape[0]} Hq={q.shape[1]} Hkv={k.shape[1]} "
          f"W={window}", flush=True)
    attn.bwd_static(q, k, v, out, lse, do, cu, ms, window, sc, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        assert torch.equal(_bits(a), _bits(b)), f"{label}: {name} differs from attn_varlen_bwd"


def test_static_backward_equals_the_workspace_backward():
    # a full workload microbatch, then a smaller problem over the same scratch
    _check(make_microbatch("ctx4096_w512", 0), 512, "ctx 4,096 window 512")
    _check(make_microbatch("tiny_ctx512_w512", 1), 512, "tiny")
    # other boundaries, heads and window, after ordinary calls have run
    lens = [1, 7, 33, 64, 65, 300, 2]
    cu = np.concatenate([[0, 0], np.cumsum(lens)]).astype(np.int32)
    _check(make_custom(cu, 6, 2, seed=9), 0, "edge segments 6q/2kv global")


def test_static_backward_refuses_a_problem_beyond_its_scratch():
    mb = make_microbatch("tiny_ctx512_w512", 2)
    q, k, v, do, cu = device_inputs(mb)
    out, lse = attn.fwd(q, k, v, cu, mb.max_seqlen, 512, mb.cfg.scale)
    cap = attn.load_library().attn_varlen_static_scratch_bytes()
    # a problem whose workspace exceeds the scratch: the host refuses it
    # before anything is enqueued (the pointers are never dereferenced)
    t_big = 1 << 20
    assert attn.workspace_size(t_big, 1, 64, 8, 128, t_big, 0) > cap
    lib = attn.load_library()
    st = lib.attn_varlen_bwd_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                    lse.data_ptr(), do.data_ptr(), cu.data_ptr(), 1, t_big, 64, 8,
                                    128, t_big, 0, 0.088, q.data_ptr(), k.data_ptr(),
                                    v.data_ptr(), None)
    assert st == -6, st
