"""Builds libfadecode.so (the HIP decode library) in-tree for gfx950 with hipcc."""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfadecode.so")
SOURCES = [os.path.join(CSRC, "fa_decode.hip")]
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed-FP32 instructions: plain scalar f32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def build(verbose: bool = False) -> str:
    cmd = [HIPCC, *FLAGS, "-o", LIB + ".tmp", *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        sys.stderr.write("\n".join(noise) + "\n")
        raise RuntimeError(f"hipcc failed ({r.returncode})")
    if verbose and noise:
        sys.stderr.write("\n".join(noise) + "\n")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
