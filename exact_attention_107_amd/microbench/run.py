"""Build and run the gfx950 issue-rate microbenchmarks of this directory.

    python exact_attention_107_amd/microbench/run.py [co_issue] [fp8_acc] [lds_read] ...

Each probe is a stand-alone HIP program (hipcc, gfx950, the library's
compile flags) built into a temporary directory and run once; its table is
printed as is.  The probes measure the limits the forward kernel's design
rests on: how MFMA and VALU instructions share a SIMD, the issue cost of the
softmax's VALU instructions, LDS read bandwidth, and the accumulation error
of the FP8 matrix product (which sets the FP8 forward's error bound).
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
PROBES = [f[:-4] for f in sorted(os.listdir(HERE)) if f.endswith(".hip")]


def main(argv) -> int:
    names = argv or PROBES
    with tempfile.TemporaryDirectory(prefix="fa_probe_") as tmp:
        for name in names:
            exe = os.path.join(tmp, name)
            subprocess.run([HIPCC, *FLAGS, os.path.join(HERE, name + ".hip"), "-o", exe], check=True,
                           stderr=subprocess.DEVNULL)
            print(f"## {name}", flush=True)
            rc = subprocess.run([exe]).returncode
            if rc != 0:
                return rc
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
