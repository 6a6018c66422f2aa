#!/usr/bin/env python3
"""Throughput of document-masked causal GQA attention, forward + backward, on MI355X.

One step is one pass of the whole hot path over one seeded 16,384-token
microbatch packed at context 4,096 (8 query / 2 key-value heads of 128): a
local layer with a 512-token window, then a global layer, each forward +
backward through the C ABI (schedule, forward, dQ + D, dK/dV kernels).  The
two layers share the microbatch's cu_seqlens and draw their own q/k/v/dout.
This is the workload the kernel benchmarks page times in its Figs. 3 and 4
(research.dws.rip/llm/kernels), with synthetic documents standing in for the
page's real token shards.

Throughput counts 4*d flops per unmasked (query, key) pair per query head
forward and 10*d backward, pairs counted exactly from cu_seqlens and the
window.  Prints one JSON line.

    python bench.py [--steps 20] [--warmup 50] [--workload ctx4096_w512+global]
                    [--softcap C] [--head-dim D] [--band] [--seeds 8] [--settle-ms 300]

Before the W warm-up steps the step runs untimed for --settle-ms of wall time
(the GPU clock needs a few tens of ms of load to leave its idle state); the
timed region is exactly K steps.  The line also carries the per-layer and
per-kernel times, the dominant kernel's roofline, a graph-replay timing,
the same step on seeds 0..7 (K steps each, with their aggregate), the CPU
oracle's rate, and the timed outputs' errors against the oracle ("parity").

--softcap C times the same step with every logit soft-capped to
C tanh(logit / C) (attn_varlen_fwd_ex / attn_varlen_bwd_ex); the counted
flops are the same.  --head-dim D (64, 128 or 256) runs the workload with
that head width (scale 1 / sqrt(D)); flops scale with D.  --band runs the
windowed layers through the band-block calls (attn_varlen_band_fwd /
attn_varlen_band_bwd: each W-token query block against the keys of its own
block and the one before, results equal to the plain calls); the counted
flops stay those of the visible pairs.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published

WORKLOADS = {
    # name: (list of (layer label, config name)), shared cu_seqlens from the first config
    "ctx4096_w512+global": [("window512", "ctx4096_w512"), ("global", "ctx4096_global")],
    "ctx4096_w512+global_h16": [("window512", "ctx4096_w512_h16"),
                                ("global", "ctx4096_global_h16")],
    "ctx512_w512": [("window512", "ctx512_w512")],
    "ctx4096_w512": [("window512", "ctx4096_w512")],
    "ctx4096_global": [("global", "ctx4096_global")],
    "ctx1024_global": [("global", "ctx1024_global")],
    "ctx2048_global": [("global", "ctx2048_global")],
    "ctx1024_w512": [("window512", "ctx1024_w512")],
    "ctx2048_w512": [("window512", "ctx2048_w512")],
    "stack_ctx4096": [("window512", "ctx4096_w512")] * 15 + [("global", "ctx4096_global")] * 5,
    "stack_ctx4096_h16": [("window512", "ctx4096_w512_h16")] * 15
    + [("global", "ctx4096_global_h16")] * 5,
}

# Flops each kernel must execute per unmasked pair per query head, in units of d
# (each product of a d-long row pair is 2d flops): forward S and PV; dQ kernel
# recomputes S and dP, then dQ; dK/dV kernel recomputes S and dP, then dV and dK.
KERNEL_FLOPS_PER_PAIR_D = {"forward": 4, "dq": 6, "dkdv": 8}


def cpu_info():
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model


def build_layers(workload: str, seed: int, device, softcap: float = 0.0, head_dim: int = 0,
                 band: bool = False):
    import dataclasses
    import torch
    from synthetic import CONFIGS, make_cu_seqlens, make_layer
    from varlen_sliding_window_amd.flops import attention_flops
    import varlen_sliding_window_amd as attn

    spec = WORKLOADS[workload]
    cu, _ = make_cu_seqlens(CONFIGS[spec[0][1]], seed)
    layers = []
    # Layers that share the microbatch's cu_seqlens and a window share one
    # workspace: the first of them builds the tile schedule, the others reuse
    # it (ATTN_FWD_REUSE_SCHEDULE), as a training step over a layer stack can.
    shared_ws = {}
    for idx, (label, cname) in enumerate(spec):
        cfg = CONFIGS[cname]
        if head_dim:
            cfg = dataclasses.replace(cfg, head_dim=head_dim)
        mb = make_layer(cfg, seed, idx, cu)

        def dev(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
                torch.bfloat16).to(device)

        q, k, v, do = dev(mb.q_bits), dev(mb.k_bits), dev(mb.v_bits), dev(mb.dout_bits)
        t, hq, d = q.shape
        key = (cfg.window, hq)
        reuse_fwd = key in shared_ws and not band
        if key not in shared_ws:
            shared_ws[key] = attn.new_workspace(t, len(cu) - 1, hq, k.shape[1], d,
                                                mb.max_seqlen, cfg.window, device)
        lay = {
            "label": label, "cfg": cfg, "mb": mb, "q": q, "k": k, "v": v, "do": do,
            "cu": torch.from_numpy(cu.astype(np.int32)).to(device),
            "max_seqlen": mb.max_seqlen, "window": cfg.window, "scale": cfg.scale,
            "out": torch.empty_like(q), "lse": torch.empty((hq, t), dtype=torch.float32,
                                                           device=device),
            "dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
            "reuse_fwd": reuse_fwd,
            "ws": shared_ws[key],
            "flops": attention_flops(cu, cfg.window, hq, d),
            "softcap": softcap,
            "band": band and cfg.window > 0,
        }
        layers.append(lay)
    return cu, layers


def run_layer(attn, L):
    attn.fwd(L["q"], L["k"], L["v"], L["cu"], L["max_seqlen"], L["window"], L["scale"],
             out=L["out"], lse=L["lse"], workspace=L["ws"], softcap=L["softcap"], band=L["band"],
             reuse_schedule=L["reuse_fwd"])
    # the backward of a layer reuses the tile schedule its forward just built
    # (the band-block backward always rebuilds its own)
    attn.bwd(L["q"], L["k"], L["v"], L["out"], L["lse"], L["do"], L["cu"], L["max_seqlen"],
             L["window"], L["scale"], dq=L["dq"], dk=L["dk"], dv=L["dv"], workspace=L["ws"],
             softcap=L["softcap"], reuse_schedule=not L["band"], band=L["band"])


def cpu_baseline(layers, seed, min_seconds=10.0, max_reps=4):
    """The CPU oracle, as it stands, on the step's layers (fwd+bwd each),
    repeated until at least min_seconds of CPU work (bounded by max_reps).
    Also returns the oracle's results of the first repetition, per layer."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import attention_backward

    cores = len(os.sched_getaffinity(0))
    reps = 0
    flops = 0
    results = []
    t0 = time.perf_counter()
    with threadpool_limits(limits=cores):
        used = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        while reps < max_reps and (reps == 0 or time.perf_counter() - t0 < min_seconds):
            for L in layers:
                mb = L["mb"]
                r = attention_backward(mb.f32("q"), mb.f32("k"), mb.f32("v"), mb.f32("dout"),
                                       mb.cu_seqlens, L["window"], L["scale"], L["softcap"])
                if reps == 0:
                    results.append(r)
                flops += L["flops"]["fwd_bwd"]
            reps += 1
    secs = time.perf_counter() - t0
    labels = "+".join(L["label"] for L in layers)
    mb = layers[0]["mb"]
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": int(used), "kind": "oracle",
            "seconds": secs, "cpu": cpu_info(),
            "sample": (f"{reps} x one step ({labels}, forward+backward) of the seed-{seed} "
                       f"microbatch, {mb.num_seqs} segments, all {mb.cfg.num_q_heads} query heads; "
                       f"fp64 NumPy oracle; counted flops / wall seconds")}, results


def parity_report(layers, oracle_results):
    """The timed step's outputs (every layer's out, lse, dq, dk, dv as the last
    timed step left them) against the oracle's: norm-wise max-rel and
    Frobenius-rel per tensor, worst over the layers of each label, and
    whether every one meets the bar (max-rel <= 1e-2, Fro-rel <= 5e-3)."""
    report = {}
    ok = True
    for L, (dq, dk, dv, out, lse, _) in zip(layers, oracle_results):
        rep = report.setdefault(L["label"], {})
        for name, ref in (("out", out), ("dq", dq), ("dk", dk), ("dv", dv)):
            x = L[name].float().cpu().numpy().astype(np.float64)
            d = x - ref
            mr = float(np.max(np.abs(d)) / np.max(np.abs(ref)))
            fr = float(np.linalg.norm(d) / np.linalg.norm(ref))
            prev = rep.get(name, {"max_rel": 0.0, "fro_rel": 0.0})
            rep[name] = {"max_rel": max(prev["max_rel"], mr), "fro_rel": max(prev["fro_rel"], fr)}
            ok = ok and mr <= 1e-2 and fr <= 5e-3 and bool(np.all(np.isfinite(x)))
        le = float(np.max(np.abs(L["lse"].cpu().numpy().astype(np.float64) - lse)))
        rep["lse_max_abs"] = max(rep.get("lse_max_abs", 0.0), le)
    return {"bar": {"max_rel": 1e-2, "fro_rel": 5e-3}, "pass": ok, "layers": report,
            "reference": "CPU oracle (fp64) on the same seeded inputs"}


def sources_sha256() -> str:
    """Hash of the sources the attention kernels are compiled from: every file
    under csrc/ except delta.hip, the translation unit that holds only the
    delta-rule kernels (it changes none of the attention kernels' code)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "varlen_sliding_window_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name == "delta.hip":
            continue
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def load_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (profiles/*.md, a 'traffic-json:' line), provided the counters
    were taken on the current kernel sources; else None."""
    pdir = os.path.join(ROOT, "profiles")
    if not os.path.isdir(pdir):
        return None
    sha = sources_sha256()
    for name in sorted(os.listdir(pdir)):
        if not name.endswith(".md"):
            continue
        with open(os.path.join(pdir, name)) as f:
            for line in f:
                if line.startswith("traffic-json:"):
                    data = json.loads(line.split(":", 1)[1])
                    if data.get("sources_sha256") == sha and data.get("kernel") == kernel:
                        return data.get("bytes_per_launch")
    return None


def load_counters():
    """Per-kernel counter summary (MFMA utilisation, executed/counted MFMA
    flops) from the committed rocprofv3 summary (a 'summary-json:' line),
    provided it was taken on the current kernel sources; else None."""
    pdir = os.path.join(ROOT, "profiles")
    if not os.path.isdir(pdir):
        return None
    sha = sources_sha256()
    for name in sorted(os.listdir(pdir)):
        if not name.endswith(".md"):
            continue
        with open(os.path.join(pdir, name)) as f:
            for line in f:
                if line.startswith("summary-json:"):
                    data = json.loads(line.split(":", 1)[1])
                    if data.get("sources_sha256") == sha:
                        return data.get("kernels")
    return None


def delta_bench(args, device):
    """Gated delta-rule layer step on the workload microbatch (one layer, H = 8
    heads of 128, the documents of the attention workload's cu_seqlens): the
    forward, saving its chunk records and states, then the backward reusing
    them, as a training step runs them.  Also times the plain forward and the
    recomputing backward alone; prints one JSON line."""
    import torch
    import varlen_sliding_window_amd as attn
    from synthetic import CONFIGS, make_cu_seqlens, make_delta_dout, make_delta_inputs

    cu, _ = make_cu_seqlens(CONFIGS["ctx4096_w512"], args.seed)
    heads, d = 8, 128
    inp = make_delta_inputs(cu, heads, d, args.seed)
    t = int(cu[-1])

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)

    q, k, v = dev_bf16(inp.q_bits), dev_bf16(inp.k_bits), dev_bf16(inp.v_bits)
    dout = dev_bf16(make_delta_dout(t, heads, d, args.seed + 1))
    g = torch.from_numpy(inp.g).to(device)
    beta = torch.from_numpy(inp.beta).to(device)
    cu_dev = torch.from_numpy(cu.astype(np.int32)).to(device)
    nseq = len(cu) - 1
    ws = torch.empty(attn.delta_bwd_workspace_size(t, nseq, heads, d), dtype=torch.uint8,
                     device=device)
    out = torch.zeros_like(q)

    def fwd():
        attn.delta_fwd(q, k, v, g, beta, cu_dev, d ** -0.5, out=out, workspace=ws)

    def bwd():
        attn.delta_bwd(q, k, v, g, beta, dout, cu_dev, d ** -0.5, workspace=ws)

    def step():
        attn.delta_fwd(q, k, v, g, beta, cu_dev, d ** -0.5, out=out, workspace=ws, save=True)
        attn.delta_bwd(q, k, v, g, beta, dout, cu_dev, d ** -0.5, workspace=ws, reuse=True)

    def timed(fn, steps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    for _ in range(args.warmup):
        step()
    ms = timed(step, args.steps)
    ms_fwd = timed(fwd, args.steps)
    ms_bwd = timed(bwd, args.steps)
    attn.profile_start()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kern = attn.profile_stop()
    print(json.dumps({
        "metric": "gated delta-rule layer step (forward + backward) per 16,384-token microbatch, 8 heads of 128",
        "value": ms, "unit": "ms", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": False, "dtype": "bf16 in, fp32 arithmetic",
        "data": "synthetic (seeded lognormal document packing; unit q, k; N(0,1) v and dout)",
        "vs_baseline": None,
        "config": {"workload": "delta_ctx4096", "total_tokens": t, "num_heads": heads,
                   "head_dim": d, "num_seqs": nseq, "seed": args.seed},
        "forward_ms": ms_fwd, "backward_recomputing_ms": ms_bwd,
        "forward_tflops": 6.0 * d * d * t * heads / (ms_fwd * 1e-3) / 1e12,
        "kernels": {kk: {"avg_ms": vv["avg_ms"]} for kk, vv in kern.items()},
    }))


def kda_bench(args, device):
    """Kimi Delta Attention layer step on the workload microbatch (one layer,
    H = 8 heads of 128, the attention workload's documents): the forward,
    saving its chunk records and states, then the backward reusing them;
    also times the plain forward alone; one JSON line."""
    import torch
    import varlen_sliding_window_amd as attn
    from synthetic import CONFIGS, make_cu_seqlens, make_delta_dout, make_kda_inputs

    cu, _ = make_cu_seqlens(CONFIGS["ctx4096_w512"], args.seed)
    heads, d = 8, 128
    inp = make_kda_inputs(cu, heads, d, args.seed)
    t = int(cu[-1])

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)

    q, k, v = dev_bf16(inp.q_bits), dev_bf16(inp.k_bits), dev_bf16(inp.v_bits)
    g = torch.from_numpy(inp.g).to(device)
    beta = torch.from_numpy(inp.beta).to(device)
    cu_dev = torch.from_numpy(cu.astype(np.int32)).to(device)
    dout = dev_bf16(make_delta_dout(t, heads, d, args.seed + 1))
    ws = torch.empty(attn.kda_bwd_workspace_size(t, len(cu) - 1, heads, d), dtype=torch.uint8,
                     device=device)
    out = torch.zeros_like(q)

    def fwd():
        attn.kda_fwd(q, k, v, g, beta, cu_dev, d ** -0.5, out=out, workspace=ws)

    def step():
        attn.kda_fwd(q, k, v, g, beta, cu_dev, d ** -0.5, out=out, workspace=ws, save=True)
        attn.kda_bwd(q, k, v, g, beta, dout, cu_dev, d ** -0.5, workspace=ws, reuse=True)

    def timed(fn):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps

    for _ in range(args.warmup):
        step()
    ms = timed(step)
    ms_fwd = timed(fwd)
    attn.profile_start()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kern = attn.profile_stop()
    print(json.dumps({
        "metric": "Kimi Delta Attention layer step (forward + backward) per 16,384-token microbatch, 8 heads of 128",
        "value": ms, "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": False, "dtype": "bf16 in, fp32 arithmetic",
        "data": "synthetic (seeded lognormal document packing; unit q, k; N(0,1) v and dout; per-channel gates)",
        "vs_baseline": None,
        "config": {"workload": "kda_ctx4096", "total_tokens": t, "num_heads": heads,
                   "head_dim": d, "num_seqs": len(cu) - 1, "seed": args.seed},
        "forward_ms": ms_fwd,
        "kernels": {kk: {"avg_ms": vv["avg_ms"]} for kk, vv in kern.items()},
    }))


def copy_calibration(device, mib: int = 256, reps: int = 3):
    """Plain device copies of a known size, for scaling the FETCH_SIZE and
    WRITE_SIZE counters (each copy reads and writes exactly mib MiB)."""
    import torch
    src = torch.ones(mib * 1024 * 1024 // 4, dtype=torch.float32, device=device)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_copy": src.numel() * 4, "copies": reps}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps first (the GPU clock takes a few tens of ms of load to settle)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--workload", default="ctx4096_w512+global",
                    choices=sorted(WORKLOADS) + ["delta_ctx4096", "kda_ctx4096"])
    ap.add_argument("--softcap", type=float, default=0.0,
                    help="logit soft-cap C > 0 (every logit becomes C tanh(logit / C))")
    ap.add_argument("--head-dim", type=int, default=0, choices=[0, 64, 128, 256],
                    help="head width (default: the workload's, 128)")
    ap.add_argument("--band", action="store_true",
                    help="windowed layers through the band-block calls")
    ap.add_argument("--print-sources-sha", action="store_true",
                    help="print the kernel-source hash the traffic summary is keyed on")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip timing the CPU oracle (profiling runs)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-replay timing (profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain copies of a known size (counter calibration)")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed steps before the warm-up until this much wall time has "
                         "passed: the GPU clock leaves its idle state only after a few tens "
                         "of ms of load (0: none)")
    ap.add_argument("--seeds", type=int, default=8,
                    help="also time seeds 0 .. N-1 of the workload (K steps each) and report "
                         "each and their aggregate (0 or 1: the headline seed only)")
    args = ap.parse_args()
    if args.print_sources_sha:
        print(sources_sha256())
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import varlen_sliding_window_amd as attn

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    attn.load_library()
    device = torch.device("cuda", 0)
    if args.copy_calibration:
        copy_calibration(device)
        return
    if args.workload == "delta_ctx4096":
        delta_bench(args, device)
        return
    if args.workload == "kda_ctx4096":
        kda_bench(args, device)
        return
    cu, layers = build_layers(args.workload, args.seed, device, args.softcap, args.head_dim,
                              args.band)
    print(f"[bench] workload {args.workload}: {len(layers)} layer(s), {len(cu) - 1} segments, "
          f"max_seqlen {layers[0]['max_seqlen']}", file=sys.stderr, flush=True)

    def step(events=None):
        for i, L in enumerate(layers):
            if events is not None:
                events[i][0].record()
            run_layer(attn, L)
            if events is not None:
                events[i][1].record()

    # The clock settles first (untimed, reported), then the W warm-up steps.
    settle_steps = 0
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        step()
        torch.cuda.synchronize()
        settle_steps += 1
    settle_s = time.perf_counter() - t_settle
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps, nothing but the library's calls
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps

    step_flops = sum(L["flops"]["fwd_bwd"] for L in layers)
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    # per-layer durations: a separate pass of K steps with an event pair
    # around each layer (event records in the stream cost time of their own,
    # so they stay out of the timed region)
    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
           for _ in layers] for _ in range(args.steps)]
    for s in range(args.steps):
        step(ev[s])
    torch.cuda.synchronize()
    per_label = {}
    for i, L in enumerate(layers):
        times = [ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)]
        d = per_label.setdefault(L["label"], {"times": [], "flops": 0, "count": 0})
        d["times"].extend(times)
        d["flops"] += L["flops"]["fwd_bwd"]
        d["count"] += 1
    layer_report = {}
    for label, d in per_label.items():
        med = statistics.median(d["times"])
        fl = d["flops"] / d["count"]
        layer_report[label] = {"ms_fwd_bwd_median": med,
                               "ms_p10": float(np.percentile(d["times"], 10)),
                               "ms_p90": float(np.percentile(d["times"], 90)),
                               "gflop": fl / 1e9, "tflops": fl / (med * 1e-3) / 1e12}

    # per-kernel durations: HIP events around each launch, one pass per layer label
    kernels = {}
    for label in per_label:
        attn.profile_start()
        for _ in range(args.steps):
            for L in layers:
                if L["label"] == label:
                    run_layer(attn, L)
        torch.cuda.synchronize()
        stats = attn.profile_stop()
        lay = next(L for L in layers if L["label"] == label)
        for kname, st in stats.items():
            entry = dict(st)
            per_d = KERNEL_FLOPS_PER_PAIR_D.get(kname)
            if per_d is not None:
                fl = per_d * lay["cfg"].head_dim * lay["flops"]["pairs"] * lay["cfg"].num_q_heads
                entry["flops_per_launch"] = fl
                entry["tflops"] = fl / (st["avg_ms"] * 1e-3) / 1e12
            kernels[f"{label}/{kname}"] = entry

    # Dominant kernel over the whole step (every launch of it, all layers):
    # achieved = its algorithmic flops / its summed event durations.  A
    # rocprofv3 --stats run of the same command averages the same launches.
    by_kernel = {}
    for key, entry in kernels.items():
        kname = key.split("/")[1]
        agg = by_kernel.setdefault(kname, {"ms": 0.0, "flops": 0.0, "launches": 0.0})
        # a label's profile pass ran every layer of that label once per step
        per_step = entry["launches"] / args.steps
        agg["ms"] += entry["total_ms"] / args.steps
        agg["flops"] += entry.get("flops_per_launch", 0.0) * per_step
        agg["launches"] += per_step
    dom_name = max(by_kernel, key=lambda k: by_kernel[k]["ms"])
    dom = by_kernel[dom_name]
    achieved = dom["flops"] / (dom["ms"] * 1e-3) / 1e12 if dom["ms"] > 0 else 0.0
    traffic = load_traffic(dom_name)
    counters = load_counters() if args.workload == "ctx4096_w512+global" else None
    roofline = {"bound": "mfma", "kernel": dom_name, "achieved": achieved,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": traffic,
                "avg_ms": dom["ms"] / dom["launches"], "launches_per_step": dom["launches"],
                "flops_per_launch": dom["flops"] / dom["launches"],
                "share_of_step": dom["ms"] / ms_per_step,
                "counters": counters}

    # The same step captured once as a HIP graph and replayed (the library
    # allocates nothing and never waits on the host, so the whole step is
    # capturable); replays remove the per-launch gaps between kernels.
    graph_report = None
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(max(args.warmup, 1)):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        graph_report = {"ms_per_step": graph_ms, "tflops": step_flops / (graph_ms * 1e-3) / 1e12,
                        "speedup_vs_eager": ms_per_step / graph_ms, "steps": args.steps}
        del graph

    # Other seeds of the same workload (other document mixes), K timed steps
    # each after a few warm-up steps; the headline seed's figure is the one
    # measured above.  The aggregate is total flops over total time.
    seeds_report = None
    if args.seeds > 1:
        per_seed = {str(args.seed): {"ms_per_step": ms_per_step, "gflop": step_flops / 1e9,
                                     "tflops": value, "num_seqs": len(cu) - 1}}
        for sd in range(args.seeds):
            if sd == args.seed:
                continue
            print(f"[bench] seed {sd}", file=sys.stderr, flush=True)
            cu_s, lay_s = build_layers(args.workload, sd, device, args.softcap, args.head_dim,
                                       args.band)
            for _ in range(max(args.warmup, 3)):
                for L in lay_s:
                    run_layer(attn, L)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                for L in lay_s:
                    run_layer(attn, L)
            torch.cuda.synchronize()
            ms_s = (time.perf_counter() - t0) * 1e3 / args.steps
            fl = sum(L["flops"]["fwd_bwd"] for L in lay_s)
            per_seed[str(sd)] = {"ms_per_step": ms_s, "gflop": fl / 1e9,
                                 "tflops": fl / (ms_s * 1e-3) / 1e12, "num_seqs": len(cu_s) - 1}
            del lay_s
        tot_fl = sum(v["gflop"] for v in per_seed.values()) * 1e9
        tot_ms = sum(v["ms_per_step"] for v in per_seed.values())
        seeds_report = {"per_seed": per_seed, "steps_each": args.steps,
                        "aggregate_tflops": tot_fl / (tot_ms * 1e-3) / 1e12,
                        "aggregate_frac_of_peak": tot_fl / (tot_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                        "mean_ms_per_step": tot_ms / len(per_seed)}

    result = {
        "metric": "fwd+bwd TFLOPS per 16,384-token microbatch (window-512 and global layers, "
                  "context 4,096)",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded lognormal document packing, N(0,1) bf16 tensors)",
        "config": {
            "workload": args.workload,
            "total_tokens": int(cu[-1]),
            "ctx": layers[0]["cfg"].ctx,
            "num_q_heads": layers[0]["cfg"].num_q_heads,
            "num_kv_heads": layers[0]["cfg"].num_kv_heads,
            "head_dim": layers[0]["cfg"].head_dim,
            "layers": [L["label"] for L in layers],
            "seed": args.seed,
            "num_seqs": len(cu) - 1,
            "max_seqlen": layers[0]["max_seqlen"],
            "gflop_per_step": step_flops / 1e9,
            "softcap": args.softcap if args.softcap > 0 else None,
            "band": True if args.band else None,
        },
        "frac_of_peak": value / PEAK_BF16_TFLOPS,
        "clock_settle": {"steps": settle_steps, "seconds": settle_s,
                         "note": "untimed steps before the W warm-up steps"},
        "layers": layer_report,
        "kernels": kernels,
        "roofline": roofline,
        "graph_replay": graph_report,
        "seeds": seeds_report,
        "gpu": torch.cuda.get_device_name(0),
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"], oracle_results = cpu_baseline(layers, args.seed)
        # the outputs the timed steps produced, against the oracle's
        result["parity"] = parity_report(layers, oracle_results)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
