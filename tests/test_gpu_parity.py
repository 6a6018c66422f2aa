"""HIP path (through the C ABI) against the fp64 CPU oracle on seeded inputs."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import attention_backward  # noqa: E402
from synthetic import CONFIGS, make_custom, make_microbatch  # noqa: E402

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_common import assert_parity, raw_outputs, run_hip  # noqa: E402


def oracle(mb, window, cu=None):
    cu = mb.cu_seqlens if cu is None else cu
    dq, dk, dv, out, lse, _ = attention_backward(mb.f32("q"), mb.f32("k"), mb.f32("v"),
                                                 mb.f32("dout"), cu, window, mb.cfg.scale)
    return {"dq": dq, "dk": dk, "dv": dv, "out": out, "lse": lse}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# --- whole-array parity on the workload configs ----------------------------------

@pytest.mark.parametrize("name", ["tiny_ctx512_w512", "ctx512_w512", "ctx4096_w512",
                                  "ctx4096_global", "ctx1024_global", "ctx2048_global",
                                  "ctx4096_w512_h16", "ctx4096_global_h16"])
def test_parity_config(name):
    cfg = CONFIGS[name]
    mb = make_microbatch(cfg, 0)
    print(f"[case] {name} seed 0 T={cfg.total_tokens} segs={mb.num_seqs} W={cfg.window}",
          flush=True)
    got = run_hip(mb, cfg.window)
    assert_parity(got, oracle(mb, cfg.window), f"{name}/seed0")


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_parity_tiny_seeds(seed):
    mb = make_microbatch("tiny_ctx512_w512", seed)
    got = run_hip(mb, 512)
    assert_parity(got, oracle(mb, 512), f"tiny/seed{seed}")


# --- edge cases: odd, 1-token, empty segments, windows ----------------------------

EDGE_LENGTHS = [1, 7, 8, 9, 63, 64, 65, 127, 128, 129, 333, 1, 511, 512, 513, 2, 31, 32, 33]


@pytest.mark.parametrize("window", [0, 1, 3, 33, 64, 512])
def test_edge_segments(window):
    lens = EDGE_LENGTHS
    cu = np.concatenate([[0], np.cumsum(lens)])
    # insert empty segments at the front, middle and end
    cu = np.concatenate([[0, 0], cu[1:6], [cu[5]], cu[6:], [cu[-1]]]).astype(np.int32)
    mb = make_custom(cu, 8, 2, seed=100 + window)
    print(f"[case] edge window={window} T={int(cu[-1])} segs={len(cu) - 1}", flush=True)
    got = run_hip(mb, window)
    assert_parity(got, oracle(mb, window), f"edge/W{window}")


@pytest.mark.parametrize("window", [0, 100])
def test_more_tiles_than_scheduler_threads(window):
    """Over 1,024 tiles: the scheduler's multi-pass path (one thread per tile
    no longer suffices), on 40,000 tokens of documents of 1 to 700 tokens."""
    rng = np.random.default_rng(77)
    lens = []
    while sum(lens) < 40000:
        lens.append(int(rng.integers(1, 701)))
    lens[-1] -= sum(lens) - 40000
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    tiles = int(np.sum((np.diff(cu) + 31) // 32))
    assert tiles > 1024
    mb = make_custom(cu, 4, 1, seed=78 + window)
    print(f"[case] {tiles} tiles, {len(lens)} segments, W={window}", flush=True)
    got = run_hip(mb, window)
    assert_parity(got, oracle(mb, window), f"{tiles} tiles/W{window}")


def test_single_token_microbatch():
    mb = make_custom([0, 1], 4, 1, seed=5)
    got = run_hip(mb, 0)
    ref = oracle(mb, 0)
    assert_parity(got, ref, "T=1")
    # P = 1 so dS = dP - D is zero up to fp32 rounding: dP (MFMA) and
    # D = dO.O (vector sum) add the same products in different orders.
    assert np.max(np.abs(got["dq"])) < 1e-5 and np.max(np.abs(got["dk"])) < 1e-5
    np.testing.assert_array_equal(got["out"], ref["out"])   # out = v exactly


# --- bitwise properties ---------------------------------------------------------------

def _bitwise_equal(a, b, label):
    for name in ("out", "lse", "dq", "dk", "dv"):
        x, y = a[name], b[name]
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32)), \
            f"{label}: {name} differs"


def test_deterministic_repeat():
    mb = make_microbatch("ctx512_w512", 4)
    a = raw_outputs(mb, 512)
    b = raw_outputs(mb, 512)
    _bitwise_equal(a, b, "repeat")


def test_empty_segment_padding_is_bitwise_neutral():
    mb = make_microbatch("ctx512_w512", 5)
    cu = mb.cu_seqlens
    a = raw_outputs(mb, 512)
    for cap in (len(cu) + 1, 96):
        padded = np.concatenate([cu, np.full(cap - len(cu), cu[-1], dtype=np.int32)])
        b = raw_outputs(mb, 512, cu=padded)
        _bitwise_equal(a, b, f"padded to {cap - 1} docs")


def test_window_at_least_longest_equals_global():
    mb = make_microbatch("ctx1024_global", 6)
    a = raw_outputs(mb, 0)
    for w in (mb.max_seqlen, 1024, 100000):
        b = raw_outputs(mb, w)
        _bitwise_equal(a, b, f"window {w}")


def test_segment_permutation_permutes_outputs():
    mb = make_custom(np.cumsum([0, 40, 1, 300, 77, 129]), 8, 2, seed=7, window=64)
    cu = mb.cu_seqlens
    lens = np.diff(cu)
    order = [3, 0, 4, 2, 1]
    idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in order])
    cu_p = np.concatenate([[0], np.cumsum(lens[order])]).astype(np.int32)
    mb_p = make_custom(cu_p, 8, 2, seed=7, window=64)
    for name in ("q_bits", "k_bits", "v_bits", "dout_bits"):
        setattr(mb_p, name, getattr(mb, name)[idx])
    a = raw_outputs(mb, 64)
    b = raw_outputs(mb_p, 64)
    idx_t = torch.as_tensor(idx, device="cuda")
    for name in ("out", "dq", "dk", "dv"):
        assert torch.equal(a[name][idx_t].view(torch.int16), b[name].view(torch.int16)), name
    assert torch.equal(a["lse"][:, idx_t].view(torch.int32), b["lse"].view(torch.int32))


def test_outputs_leave_guard_regions_untouched():
    import varlen_sliding_window_amd as attn
    from gpu_common import device_inputs
    mb = make_microbatch("tiny_ctx512_w512", 8)
    q, k, v, do, cu = device_inputs(mb)
    t, hq, d = q.shape
    hkv = k.shape[1]
    guard = 4096

    def guarded(shape, dtype):
        n = int(np.prod(shape))
        buf = torch.full((n + 2 * guard,), float("nan"), dtype=dtype, device="cuda")
        return buf, buf[guard:guard + n].view(shape)

    ob, out = guarded((t, hq, d), torch.bfloat16)
    lb, lse = guarded((hq, t), torch.float32)
    qb_, dq = guarded((t, hq, d), torch.bfloat16)
    kb_, dk = guarded((t, hkv, d), torch.bfloat16)
    vb_, dv = guarded((t, hkv, d), torch.bfloat16)
    attn.fwd(q, k, v, cu, mb.max_seqlen, 512, mb.cfg.scale, out=out, lse=lse)
    attn.bwd(q, k, v, out, lse, do, cu, mb.max_seqlen, 512, mb.cfg.scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for buf, view in ((ob, out), (lb, lse), (qb_, dq), (kb_, dk), (vb_, dv)):
        assert torch.isnan(buf[:guard].float()).all() and torch.isnan(buf[-guard:].float()).all()
        assert torch.isfinite(view.float()).all()
