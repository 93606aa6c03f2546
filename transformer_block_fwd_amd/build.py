"""Builds the HIP library libpblock.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "pblock.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpblock.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-shared",
    "-fPIC",
    # no packed-fp32 (v_pk_*_f32) instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the pblock library)")


def build(verbose: bool = True) -> str:
    """Compile csrc/pblock.hip into transformer_block_fwd_amd/libpblock.so (always recompiles)."""
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, SRC, "-o", tmp]
    if verbose:
        print("[build]", " ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature: harmless
    noise = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed:\n" + "\n".join(noise))
    if verbose and noise:
        print("\n".join(noise), file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
