"""Build ``libada.so`` (HIP kernels + C ABI) for gfx950 with hipcc, in place.

Usage: ``python autoregressive_decode_attention_amd/build.py`` (a plain script: it does
not import the package, which needs the built library).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG_DIR = Path(__file__).resolve().parent
ROOT = PKG_DIR.parent
CSRC = PKG_DIR / "csrc"
INCLUDE = ROOT / "include"
LIBRARY = PKG_DIR / "libada.so"
SOURCES = [CSRC / "ada_kernels.hip", CSRC / "ada_prefill.hip", CSRC / "ada_graph.hip", CSRC / "ada_measure.hip",
           CSRC / "ada_noalloc.hip", CSRC / "ada_api.cpp"]
ARCH = os.environ.get("ADA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and Path(cand).exists():
            return cand
    raise FileNotFoundError("hipcc not found (ROCm is required to build libada)")


def command(output: Path = LIBRARY) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Wall", "-Wno-unused-result",
        # packed fp32 arithmetic stays off: plain fp32 ops only
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{INCLUDE}", f"-I{CSRC}",
        *[str(s) for s in SOURCES],
        "-o", str(output),
    ]


def build(verbose: bool = False) -> Path:
    tmp = LIBRARY.with_name(LIBRARY.name + ".tmp")
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
