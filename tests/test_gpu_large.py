"""Microbatches far above the workload's 16,384 tokens, up to the largest
k the ABI accepts (T x Hkv x D bf16 just under 4 GiB, the limit of the
kernels' 32-bit row offsets): forward and backward through the C ABI, with
sampled outputs checked against the oracle's single-row (out, lse, dq) and
single-key (dk, dv) functions.  Documents are packed as in the workload at
context 4,096; tensors are seeded N(0,1) draws rounded to bf16 on the
device (host copies are made only of the sampled rows' segments)."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import attention_key, attention_row  # noqa: E402
from synthetic import Config, make_cu_seqlens  # noqa: E402

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import varlen_sliding_window_amd as attn  # noqa: E402
    from gpu_common import FRO_REL, LSE_ABS, MAX_REL  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _draw(shape, gen):
    return torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)


def _host(t, lo, hi):
    return t[lo:hi].float().cpu().numpy().astype(np.float64)


def _check(pairs, label):
    x = np.concatenate([a.ravel() for a, _ in pairs])
    y = np.concatenate([b.ravel() for _, b in pairs])
    max_rel = np.max(np.abs(x - y)) / np.max(np.abs(y))
    fro_rel = np.linalg.norm(x - y) / np.linalg.norm(y)
    print(f"[parity] {label}: max-rel {max_rel:.2e} fro-rel {fro_rel:.2e}", flush=True)
    assert max_rel <= MAX_REL and fro_rel <= FRO_REL, label


@pytest.mark.parametrize("total,window", [(1 << 20, 512), (1 << 20, 0), ((1 << 23) - 65536, 512)])
def test_large_microbatch_sampled(total, window):
    hq, hkv, d = 8, 2, 128
    need = total * (3 * hq + 4 * hkv + hq) * d * 2 + total * hq * 16
    if torch.cuda.mem_get_info()[0] < need * 1.3:
        pytest.skip(f"needs {need / 2**30:.0f} GiB of free device memory")
    cfg = Config("large", total, 4096, window, hq, hkv, d)
    cu, _ = make_cu_seqlens(cfg, 3)
    print(f"[case] T={total} W={window} segments={len(cu) - 1} "
          f"k bytes={total * hkv * d * 2}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(1234 + window)
    q, k, v, do = (_draw((total, h, d), gen) for h in (hq, hkv, hkv, hq))
    cu_dev = torch.from_numpy(cu.astype(np.int32)).cuda()
    ms = int(np.diff(cu).max())
    scale = cfg.scale
    out, lse = attn.fwd(q, k, v, cu_dev, ms, window, scale)
    dq, dk, dv = attn.bwd(q, k, v, out, lse, do, cu_dev, ms, window, scale)
    torch.cuda.synchronize()

    rng = np.random.default_rng(total + window)
    seg = lambda i: (int(cu[np.searchsorted(cu, i, side="right") - 1]),
                     int(cu[np.searchsorted(cu, i, side="right")]))
    rows = [0, total - 1, int(cu[len(cu) // 2]), int(cu[-2])]
    rows += [int(x) for x in rng.integers(0, total, 8)]
    outs, dqs = [], []
    lse_err = 0.0
    for n, i in enumerate(rows):
        a, b = seg(i)
        loc = [_host(t, a, i + 1) for t in (q, k, v, do)]
        h = n % hq
        o, l, g = attention_row(*loc, [0, i + 1 - a], window, scale, h, i - a)
        outs.append((out[i, h].float().cpu().numpy(), o))
        dqs.append((dq[i, h].float().cpu().numpy(), g))
        lse_err = max(lse_err, abs(float(lse[h, i]) - l))
    _check(outs, f"T={total} W={window} sampled out")
    _check(dqs, f"T={total} W={window} sampled dq")
    assert lse_err <= LSE_ABS, f"sampled lse error {lse_err:.2e}"

    keys = [0, total - 1, int(cu[len(cu) // 3])] + [int(x) for x in rng.integers(0, total, 3)]
    dks, dvs = [], []
    for n, j in enumerate(keys):
        a, b = seg(j)
        hi = min(b, j + window) if window > 0 else b
        loc = [_host(t, a, hi) for t in (q, k, v, do)]
        g = n % hkv
        rk, rv = attention_key(*loc, [0, hi - a], window, scale, g, j - a)
        dks.append((dk[j, g].float().cpu().numpy(), rk))
        dvs.append((dv[j, g].float().cpu().numpy(), rv))
    _check(dks, f"T={total} W={window} sampled dk")
    _check(dvs, f"T={total} W={window} sampled dv")
