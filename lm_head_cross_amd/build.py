"""Build the HIP library ``libflce.so`` for gfx950 in-tree.

    python -m lm_head_cross_amd.build

Every HIP source is compiled with packed fp32 ops turned off.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", "flce.hip"), os.path.join(PKG, "csrc", "chunked_ce.hip")]
OUTPUT = os.path.join(PKG, "libflce.so")
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def command(output: str = OUTPUT) -> list[str]:
    return [
        hipcc(),
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-shared",
        "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        *SOURCES,
        "-o", output,
    ]


def build(verbose: bool = False) -> str:
    """Compile the library (always) and return its path."""
    tmp = OUTPUT + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, OUTPUT)
    return OUTPUT


if __name__ == "__main__":
    print(build(verbose=True))
