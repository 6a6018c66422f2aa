"""Helpers shared by the GPU tests: seeded inputs onto the device, the HIP
path through the C ABI, and the parity metrics against the oracle."""
from __future__ import annotations

import numpy as np
import torch

import varlen_sliding_window_amd as attn
from synthetic import Microbatch

# Parity bar (per tensor, over the whole array): the kernel benchmarks page
# (research.dws.rip/llm/kernels, section 01) accepts 0.2% to 0.5% relative
# error against a 32-bit reference; we require norm-wise
# max|x - y| / max|y| <= 1e-2 and ||x - y||_F / ||y||_F <= 5e-3.
MAX_REL = 1e-2
FRO_REL = 5e-3
LSE_ABS = 2e-3


def bits_to_torch(bits: np.ndarray, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device)


def device_inputs(mb: Microbatch, device="cuda"):
    q = bits_to_torch(mb.q_bits, device)
    k = bits_to_torch(mb.k_bits, device)
    v = bits_to_torch(mb.v_bits, device)
    do = bits_to_torch(mb.dout_bits, device)
    cu = torch.from_numpy(mb.cu_seqlens.astype(np.int32)).to(device)
    return q, k, v, do, cu


def raw_outputs(mb: Microbatch, window: int, cu=None, max_seqlen=None, softcap: float = 0.0,
                scale: float | None = None):
    """Forward then backward through the C ABI; the raw torch tensors."""
    q, k, v, do, cu_dev = device_inputs(mb)
    if cu is not None:
        cu_dev = torch.as_tensor(np.asarray(cu, dtype=np.int32)).cuda()
    ms = mb.max_seqlen if max_seqlen is None else max_seqlen
    sc = mb.cfg.scale if scale is None else scale
    out, lse = attn.fwd(q, k, v, cu_dev, ms, window, sc, softcap=softcap)
    dq, dk, dv = attn.bwd(q, k, v, out, lse, do, cu_dev, ms, window, sc, softcap=softcap)
    torch.cuda.synchronize()
    return {"out": out, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def run_hip(mb: Microbatch, window: int, max_seqlen: int | None = None, cu=None,
            softcap: float = 0.0, scale: float | None = None):
    """Same as raw_outputs, as float64 numpy arrays."""
    r = raw_outputs(mb, window, cu=cu, max_seqlen=max_seqlen, softcap=softcap, scale=scale)
    return {name: t.float().cpu().numpy().astype(np.float64) for name, t in r.items()}


def rel_errors(x: np.ndarray, y: np.ndarray) -> tuple[float, float]:
    d = x - y
    ymax = np.max(np.abs(y))
    yfro = np.linalg.norm(y)
    max_rel = float(np.max(np.abs(d)) / ymax) if ymax > 0 else float(np.max(np.abs(d)))
    fro_rel = float(np.linalg.norm(d) / yfro) if yfro > 0 else float(np.linalg.norm(d))
    return max_rel, fro_rel


def assert_parity(got: dict, ref: dict, label: str, rows=None):
    """got: HIP results; ref: oracle (dq, dk, dv, out, lse).  rows: optional token index set."""
    report = {}
    for name in ("out", "dq", "dk", "dv"):
        x, y = got[name], ref[name]
        if rows is not None:
            x, y = x[rows], y[rows]
        mr, fr = rel_errors(x, y)
        report[name] = (mr, fr)
    x, y = got["lse"], ref["lse"]
    if rows is not None:
        x, y = x[:, rows], y[:, rows]
    lse_err = float(np.max(np.abs(x - y)))
    print(f"[parity] {label}: " + " ".join(f"{n} max {m:.2e} fro {f:.2e}"
                                           for n, (m, f) in report.items())
          + f" lse {lse_err:.2e}", flush=True)
    for name, (mr, fr) in report.items():
        assert mr <= MAX_REL, f"{label} {name}: max-rel {mr:.3e} > {MAX_REL}"
        assert fr <= FRO_REL, f"{label} {name}: fro-rel {fr:.3e} > {FRO_REL}"
        assert np.all(np.isfinite(got[name])), f"{label} {name}: non-finite values"
    assert lse_err <= LSE_ABS, f"{label} lse: max abs err {lse_err:.3e}"
