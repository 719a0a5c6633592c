"""Build libq3moe.so (HIP, gfx950) in-tree with hipcc.

    python -m sparse_moe_decode_q3moe_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
LIB = PKG / "libq3moe.so"
SOURCES = ["api.hip", "route.hip", "group.hip", "ffn.hip", "ffn_decode.hip", "prefill.hip", "norm.hip", "layer.hip", "model.hip", "attn_prefill.hip", "noalloc.hip"]
ARCH = "gfx950"

# Packed-FP32 instructions are disabled for all device code.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found; the q3moe library needs ROCm's hipcc")


def build(verbose: bool = False) -> Path:
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc(), *HIP_FLAGS, "-shared", "-o", str(tmp), *[str(CSRC / s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
