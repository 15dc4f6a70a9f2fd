"""Build libvidattn.so in-tree with hipcc for gfx950.

    python video_diffusion_transformer_rope3d_amd/build.py

(run by path: importing the package loads the library, which may not be
built yet).

Packed fp32 VALU instructions are disabled for all device code
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host pass
warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libvidattn.so")
SOURCES = [os.path.join(CSRC, "vidattn.hip")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libvidattn)")


def command(out: str = LIB, extra=()) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
            "-I", INCLUDE, "-I", CSRC, *SOURCES, "-o", out, *extra]


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile the library to ``out``; ``defines`` are extra -D options
    (tile-shape knobs of the kernels)."""
    tmp = out + ".tmp"
    cmd = command(tmp, extra=[f"-D{d}" for d in defines])
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(line for line in r.stderr.splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


def assembly(out: str) -> None:
    """Write the gfx950 assembly of the library (for register and
    instruction inspection)."""
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-S", "--cuda-device-only",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC,
           *SOURCES, "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)


if __name__ == "__main__":
    print(build(verbose=True))
