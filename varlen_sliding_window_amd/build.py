"""Build libattn_varlen.so in-tree with hipcc for gfx950.

    python -m varlen_sliding_window_amd.build

Every call recompiles.  Packed fp32 instructions are switched off
(``-packed-fp32-ops``) for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["schedule.hip", "fwd.hip", "bwd.hip", "delta.hip", "api.hip"]
OUTPUT = os.path.join(HERE, "libattn_varlen.so")


def hipcc_command(output: str = OUTPUT) -> list[str]:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    return [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"),
            *[os.path.join(HERE, "csrc", s) for s in SOURCES], "-o", output]


def build(verbose: bool = False) -> str:
    tmp = OUTPUT + ".tmp"
    cmd = hipcc_command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libattn_varlen.so")
    if verbose:
        sys.stderr.write(res.stderr)
    os.replace(tmp, OUTPUT)
    return OUTPUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
