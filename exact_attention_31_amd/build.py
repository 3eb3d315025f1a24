"""Build the HIP library ``libfa.so`` in-tree for gfx950 with hipcc.

``python -m exact_attention_31_amd.build`` (or ``build()``) always recompiles.
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfa.so")
SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_fwd_fp8.hip", "fa_decode.hip", "fa_bwd.hip"]
ARCH = os.environ.get("FA_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    # no packed fp32 arithmetic anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libfa.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, "-o", tmp, *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(
        ln for ln in (res.stdout + res.stderr).splitlines()
        if "packed-fp32-ops" not in ln  # the host pass does not know this device feature
    ).strip()
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if out and verbose:
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
