"""Gated delta-rule backward (attn_delta_bwd) against the fp64 oracle's
gradients (oracle/delta.py: autograd of the token-by-token recurrence) on
seeded inputs: chunk-edge and empty documents, long documents whose state
gradient crosses many chunks, and documents sampled from the full
16,384-token microbatch (documents are independent, so the oracle runs on
each sampled document alone)."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle.delta import gated_delta_backward  # noqa: E402
from synthetic import CONFIGS, make_cu_seqlens, make_delta_dout, make_delta_inputs  # noqa: E402
from synthetic import bf16_bits_to_f32  # noqa: E402

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import varlen_sliding_window_amd as attn  # noqa: E402
    from gpu_common import FRO_REL, MAX_REL, bits_to_torch, rel_errors  # noqa: E402

NAMES = ("dq", "dk", "dv", "dg", "dbeta")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run(inp, dout_bits, scale, g=None):
    q, k, v = (bits_to_torch(getattr(inp, n + "_bits")) for n in ("q", "k", "v"))
    do = bits_to_torch(dout_bits)
    g = torch.from_numpy(inp.g if g is None else g).cuda()
    beta = torch.from_numpy(inp.beta).cuda()
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).cuda()
    grads = attn.delta_bwd(q, k, v, g, beta, do, cu, scale)
    torch.cuda.synchronize()
    return [x.float().cpu().numpy().astype(np.float64) for x in grads]


def reference(inp, dout_bits, scale, lo=None, hi=None, g=None):
    """Oracle gradients of tokens [lo, hi) taken as one document."""
    sl = slice(lo, hi)
    cu = inp.cu_seqlens if lo is None else np.array([0, hi - lo])
    g = inp.g if g is None else g
    ref = gated_delta_backward(inp.f32("q")[sl], inp.f32("k")[sl], inp.f32("v")[sl],
                               g[sl], inp.beta[sl], bf16_bits_to_f32(dout_bits)[sl], cu, scale)
    return ref[:5]


def compare(got, ref, label):
    for name, x, y in zip(NAMES, got, ref):
        assert np.all(np.isfinite(x)), f"{label} {name}"
        mr, fr = rel_errors(x, y)
        print(f"[parity] delta bwd {label} {name}: max-rel {mr:.2e} fro-rel {fr:.2e}", flush=True)
        assert mr <= MAX_REL and fr <= FRO_REL, f"{label} {name}: max-rel {mr:.3e} fro-rel {fr:.3e}"


EDGE = [1, 63, 64, 65, 2, 128, 129, 7, 300, 1, 33]


def test_delta_bwd_edge_documents():
    c = np.cumsum(EDGE)
    cu = np.concatenate([[0, 0], c[:4], [c[3]], c[4:]]).astype(np.int32)
    inp = make_delta_inputs(cu, 2, 128, seed=21)
    dout = make_delta_dout(int(cu[-1]), 2, 128, seed=22)
    compare(run(inp, dout, 128 ** -0.5), reference(inp, dout, 128 ** -0.5),
            f"edge T={int(cu[-1])}")


@pytest.mark.parametrize("length,heads", [(1000, 1), (400, 4)])
def test_delta_bwd_long_document(length, heads):
    inp = make_delta_inputs(np.array([0, length], dtype=np.int32), heads, 128, seed=23 + heads)
    dout = make_delta_dout(length, heads, 128, seed=24 + heads)
    compare(run(inp, dout, 128 ** -0.5), reference(inp, dout, 128 ** -0.5),
            f"one {length}-token document, H={heads}")


def test_delta_bwd_workload_microbatch_sampled():
    cu, _ = make_cu_seqlens(CONFIGS["ctx4096_w512"], 0)
    t = int(cu[-1])
    inp = make_delta_inputs(cu, 8, 128, seed=0)
    dout = make_delta_dout(t, 8, 128, seed=1)
    got = run(inp, dout, 128 ** -0.5)
    for x in got:
        assert np.all(np.isfinite(x))
    lens = np.diff(cu)
    # the shortest document and those nearest 300 and 600 tokens (the oracle's
    # token loop keeps longer ones out of a test's time)
    picks = {int(np.argmin(np.where(lens > 0, lens, 1 << 30))),
             int(np.argmin(np.abs(lens - 300))), int(np.argmin(np.abs(lens - 600)))}
    for s in sorted(picks):
        lo, hi = int(cu[s]), int(cu[s + 1])
        ref = reference(inp, dout, 128 ** -0.5, lo, hi)
        compare([x[lo:hi] for x in got], ref, f"T=16,384 H=8, document {s} ({hi - lo} tokens)")


def test_delta_bwd_workload_longest_document():
    """The longest document of the 16,384-token workload microbatch (3,678
    tokens, 58 chunks at seed 0), all 8 heads, against the oracle run on that
    document alone (documents are independent)."""
    cu, _ = make_cu_seqlens(CONFIGS["ctx4096_w512"], 0)
    t = int(cu[-1])
    inp = make_delta_inputs(cu, 8, 128, seed=0)
    dout = make_delta_dout(t, 8, 128, seed=1)
    got = run(inp, dout, 128 ** -0.5)
    s = int(np.argmax(np.diff(cu)))
    lo, hi = int(cu[s]), int(cu[s + 1])
    print(f"[case] delta bwd longest document {s}: {hi - lo} tokens", flush=True)
    compare([x[lo:hi] for x in got], reference(inp, dout, 128 ** -0.5, lo, hi),
            f"T=16,384 H=8, longest document {s} ({hi - lo} tokens)")


def test_delta_bwd_strong_decay():
    """Per-token decays down to 0.05 (whole chunks' decays underflow)."""
    inp = make_delta_inputs(np.array([0, 150, 300, 700], dtype=np.int32), 2, 128, seed=31)
    g = np.log(np.random.default_rng(32).uniform(0.05, 1.0, size=inp.g.shape)).astype(np.float32)
    dout = make_delta_dout(700, 2, 128, seed=33)
    compare(run(inp, dout, 0.2, g), reference(inp, dout, 0.2, g=g), "strong decay")


def test_delta_bwd_repeatable_and_scale():
    cu = np.array([0, 70, 200], dtype=np.int32)
    inp = make_delta_inputs(cu, 2, 128, seed=25)
    dout = make_delta_dout(200, 2, 128, seed=26)
    a = run(inp, dout, 0.3)
    b = run(inp, dout, 0.3)
    for name, x, y in zip(NAMES, a, b):   # fixed-order sums everywhere: bit for bit
        assert np.array_equal(x, y), name
    compare(a, reference(inp, dout, 0.3), "scale 0.3")


def _device(inp, dout_bits):
    q, k, v = (bits_to_torch(getattr(inp, n + "_bits")) for n in ("q", "k", "v"))
    g = torch.from_numpy(inp.g).cuda()
    beta = torch.from_numpy(inp.beta).cuda()
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).cuda()
    return q, k, v, g, beta, bits_to_torch(dout_bits), cu


def test_delta_bwd_reusing_a_saving_forward():
    cu = np.array([0, 130, 131, 400], dtype=np.int32)
    inp = make_delta_inputs(cu, 3, 128, seed=27)
    q, k, v, g, beta, do, cu_d = _device(inp, make_delta_dout(400, 3, 128, seed=28))
    plain = attn.delta_fwd(q, k, v, g, beta, cu_d)
    ref = attn.delta_bwd(q, k, v, g, beta, do, cu_d)
    ws = torch.empty(attn.delta_bwd_workspace_size(400, 3, 3, 128), dtype=torch.uint8,
                     device="cuda")
    saved = attn.delta_fwd(q, k, v, g, beta, cu_d, workspace=ws, save=True)
    assert torch.equal(saved, plain), "saving changes the forward's output"
    for rep in range(2):   # a reusing backward leaves the saved data as it was
        got = attn.delta_bwd(q, k, v, g, beta, do, cu_d, workspace=ws, reuse=True)
        torch.cuda.synchronize()
        for name, x, y in zip(NAMES, got, ref):
            assert torch.equal(x, y), (rep, name)


def test_delta_bwd_reuse_is_refused_without_a_matching_save():
    cu = np.array([0, 70, 200], dtype=np.int32)
    inp = make_delta_inputs(cu, 2, 128, seed=29)
    q, k, v, g, beta, do, cu_d = _device(inp, make_delta_dout(200, 2, 128, seed=30))
    ws = torch.empty(attn.delta_bwd_workspace_size(200, 2, 2, 128), dtype=torch.uint8,
                     device="cuda")
    attn.delta_fwd(q, k, v, g, beta, cu_d, workspace=ws, save=True)
    attn.delta_fwd(q, k, v, g, beta, cu_d, workspace=ws)           # a forward that saves nothing
    with pytest.raises(ValueError):                                # the binding's own record
        attn.delta_bwd(q, k, v, g, beta, do, cu_d, workspace=ws, reuse=True)
    # the device-side check: every output becomes NaN
    got = attn.delta_bwd(q, k, v, g, beta, do, cu_d, workspace=ws, reuse=True, check_reuse=False)
    torch.cuda.synchronize()
    assert all(torch.isnan(x.float()).all() for x in got), "ran on a workspace not saved for it"
    # saved for another segment count (same tokens and heads): refused too
    one = torch.tensor([0, 200], dtype=torch.int32, device="cuda")
    attn.delta_fwd(q, k, v, g, beta, one, workspace=ws, save=True)
    with pytest.raises(ValueError):
        attn.delta_bwd(q, k, v, g, beta, do, cu_d, workspace=ws, reuse=True)
    got = attn.delta_bwd(q, k, v, g, beta, do, cu_d, workspace=ws, reuse=True, check_reuse=False)
    torch.cuda.synchronize()
    assert all(torch.isnan(x.float()).all() for x in got)
    # without the flag the backward recomputes and fills them
    got = attn.delta_bwd(q, k, v, g, beta, do, cu_d, workspace=ws)
    torch.cuda.synchronize()
    assert all(torch.count_nonzero(x) > 0 and torch.isfinite(x.float()).all() for x in got)
