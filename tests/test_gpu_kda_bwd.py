"""Kimi Delta Attention backward (attn_kda_bwd) against the fp64 oracle's
gradients (oracle/kimi_delta.py, autograd of the token loop) on seeded
inputs: chunk-edge and empty documents, a long document, documents sampled
from the full 16,384-token microbatch (each run through the oracle alone),
strong per-channel decays, and a gate equal on every channel against the
Gated DeltaNet backward kernel (whose dg is then the channel sum)."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle.kimi_delta import kimi_delta_backward  # noqa: E402
from synthetic import CONFIGS, bf16_bits_to_f32, make_cu_seqlens, make_delta_dout  # noqa: E402
from synthetic import make_kda_inputs  # noqa: E402

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
    gt = torch.from_numpy(inp.g if g is None else g).cuda()
    beta = torch.from_numpy(inp.beta).cuda()
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).cuda()
    grads = attn.kda_bwd(q, k, v, gt, beta, bits_to_torch(dout_bits), cu, scale)
    torch.cuda.synchronize()
    return [x.float().cpu().numpy().astype(np.float64) for x in grads]


def reference(inp, dout_bits, scale, lo=None, hi=None, g=None):
    sl = slice(lo, hi)
    gg = inp.g if g is None else g
    cu = inp.cu_seqlens if lo is None else np.array([0, hi - lo])
    return kimi_delta_backward(inp.f32("q")[sl], inp.f32("k")[sl], inp.f32("v")[sl], gg[sl],
                               inp.beta[sl], bf16_bits_to_f32(dout_bits)[sl], cu, scale)[:5]


def compare(got, ref, label):
    for name, x, y in zip(NAMES, got, ref):
        assert np.all(np.isfinite(x)), f"{label} {name}"
        mr, fr = rel_errors(x, y)
        print(f"[parity] kda bwd {label} {name}: max-rel {mr:.2e} fro-rel {fr:.2e}", flush=True)
        assert mr <= MAX_REL and fr <= FRO_REL, f"{label} {name}: max-rel {mr:.3e} fro-rel {fr:.3e}"


EDGE = [1, 63, 64, 65, 2, 128, 129, 7, 300, 1, 33]


def test_kda_bwd_edge_documents():
    c = np.cumsum(EDGE)
    cu = np.concatenate([[0, 0], c[:4], [c[3]], c[4:]]).astype(np.int32)
    inp = make_kda_inputs(cu, 2, 128, seed=41)
    dout = make_delta_dout(int(cu[-1]), 2, 128, seed=42)
    compare(run(inp, dout, 128 ** -0.5), reference(inp, dout, 128 ** -0.5), f"edge T={int(cu[-1])}")


def test_kda_bwd_long_document():
    inp = make_kda_inputs(np.array([0, 700], dtype=np.int32), 2, 128, seed=43)
    dout = make_delta_dout(700, 2, 128, seed=44)
    compare(run(inp, dout, 128 ** -0.5), reference(inp, dout, 128 ** -0.5), "one 700-token document, H=2")


def test_kda_bwd_workload_microbatch_sampled():
    cu, _ = make_cu_seqlens(CONFIGS["ctx4096_w512"], 0)
    t = int(cu[-1])
    inp = make_kda_inputs(cu, 8, 128, seed=0)
    dout = make_delta_dout(t, 8, 128, seed=1)
    got = run(inp, dout, 128 ** -0.5)
    for x in got:
        assert np.all(np.isfinite(x))
    lens = np.diff(cu)
    picks = {int(np.argmin(np.where(lens > 0, lens, 1 << 30))), int(np.argmin(np.abs(lens - 300)))}
    for s in sorted(picks):
        lo, hi = int(cu[s]), int(cu[s + 1])
        compare([x[lo:hi] for x in got], reference(inp, dout, 128 ** -0.5, lo, hi),
                f"T=16,384 H=8, document {s} ({hi - lo} tokens)")


def test_kda_bwd_workload_longest_document():
    """The longest document of the workload microbatch (3,678 tokens at seed
    0), all 8 heads, against the oracle run on that document alone."""
    cu, _ = make_cu_seqlens(CONFIGS["ctx4096_w512"], 0)
    t = int(cu[-1])
    inp = make_kda_inputs(cu, 8, 128, seed=0)
    dout = make_delta_dout(t, 8, 128, seed=1)
    got = run(inp, dout, 128 ** -0.5)
    s = int(np.argmax(np.diff(cu)))
    lo, hi = int(cu[s]), int(cu[s + 1])
    print(f"[case] kda bwd longest document {s}: {hi - lo} tokens", flush=True)
    compare([x[lo:hi] for x in got], reference(inp, dout, 128 ** -0.5, lo, hi),
            f"T=16,384 H=8, longest document {s} ({hi - lo} tokens)")


def test_kda_bwd_repeatable():
    cu = np.array([0, 70, 200], dtype=np.int32)
    inp = make_kda_inputs(cu, 2, 128, seed=52)
    dout = make_delta_dout(200, 2, 128, seed=53)
    a = run(inp, dout, 0.3)
    b = run(inp, dout, 0.3)
    for name, x, y in zip(NAMES, a, b):   # fixed-order sums everywhere: bit for bit
        assert np.array_equal(x, y), name


def test_kda_bwd_strong_decay():
    inp = make_kda_inputs(np.array([0, 150, 300], dtype=np.int32), 2, 128, seed=45)
    g = np.log(np.random.default_rng(46).uniform(0.05, 1.0, size=inp.g.shape)).astype(np.float32)
    dout = make_delta_dout(300, 2, 128, seed=47)
    compare(run(inp, dout, 0.2, g), reference(inp, dout, 0.2, g=g), "strong decay")


def test_kda_bwd_equal_channels_match_the_scalar_gate_kernel():
    inp = make_kda_inputs(np.array([0, 90, 300], dtype=np.int32), 2, 128, seed=48)
    gs = inp.g[..., 0].copy()
    g = np.repeat(gs[..., None], 128, axis=-1)
    dout = make_delta_dout(300, 2, 128, seed=49)
    got = run(inp, dout, 0.1, g)
    q, k, v = (bits_to_torch(getattr(inp, n + "_bits")) for n in ("q", "k", "v"))
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).cuda()
    ref = attn.delta_bwd(q, k, v, torch.from_numpy(gs).cuda(), torch.from_numpy(inp.beta).cuda(),
                         bits_to_torch(dout), cu, 0.1)
    ref = [x.float().cpu().numpy().astype(np.float64) for x in ref]
    got[3] = got[3].sum(axis=-1)          # a shared gate's gradient is the channel sum
    for name, x, y in zip(NAMES, got, ref):
        mr, fr = rel_errors(x, y)
        print(f"[parity] kda bwd equal channels vs delta_bwd {name}: max-rel {mr:.2e} fro-rel {fr:.2e}",
              flush=True)
        assert mr <= MAX_REL and fr <= FRO_REL, name


def test_kda_bwd_reusing_a_saving_forward():
    cu = np.array([0, 130, 131, 400], dtype=np.int32)
    inp = make_kda_inputs(cu, 3, 128, seed=50)
    q, k, v = (bits_to_torch(getattr(inp, n + "_bits")) for n in ("q", "k", "v"))
    g = torch.from_numpy(inp.g).cuda()
    beta = torch.from_numpy(inp.beta).cuda()
    do = bits_to_torch(make_delta_dout(400, 3, 128, seed=51))
    cu_d = torch.from_numpy(cu).cuda()
    plain = attn.kda_fwd(q, k, v, g, beta, cu_d)
    ref = attn.kda_bwd(q, k, v, g, beta, do, cu_d)
    ws = torch.empty(attn.kda_bwd_workspace_size(400, 3, 3, 128), dtype=torch.uint8, device="cuda")
    saved = attn.kda_fwd(q, k, v, g, beta, cu_d, workspace=ws, save=True)
    assert torch.equal(saved, plain), "saving changes the forward's output"
    for rep in range(2):   # a reusing backward leaves the saved data as it was
        got = attn.kda_bwd(q, k, v, g, beta, do, cu_d, workspace=ws, reuse=True)
        torch.cuda.synchronize()
        for name, x, y in zip(NAMES, got, ref):
            assert torch.equal(x, y), (rep, name)
    attn.kda_fwd(q, k, v, g, beta, cu_d, workspace=ws)           # saves nothing
    with pytest.raises(ValueError):                              # the binding's own record
        attn.kda_bwd(q, k, v, g, beta, do, cu_d, workspace=ws, reuse=True)
    got = attn.kda_bwd(q, k, v, g, beta, do, cu_d, workspace=ws, reuse=True, check_reuse=False)
    torch.cuda.synchronize()
    assert all(torch.isnan(x.float()).all() for x in got), "ran on a workspace not saved for it"
