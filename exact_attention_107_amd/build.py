"""Build libfa.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

One translation unit per head dimension is compiled in parallel, then linked
with the C ABI unit into exact_attention_107_amd/libfa.so.
"""
from __future__ import annotations

import json
import os
import re
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libfa.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
# Keep MFMA accumulators in architectural VGPRs, where the softmax rescale and
# the epilogue operate on them in place.  At d = 256 (one wave per SIMD) the
# values that do not fit then spill into the accumulation registers instead
# of scratch; with the accumulators there instead, every score tile and every
# rescale of O went through accvgpr moves (~900 per key tile; measured 15 %
# slower).
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
UNITS = [
    ("fa_kernels_d64.hip", VGPR_FORM),
    ("fa_kernels_d128.hip", VGPR_FORM),
    ("fa_kernels_d256.hip", VGPR_FORM),
    ("fa_bwd_d64.hip", VGPR_FORM),
    ("fa_bwd_d128.hip", VGPR_FORM),
    # d = 256 backward, one wave per SIMD: the 256 dK/dV accumulator values
    # live in the accumulation registers, which the MFMAs read and write in
    # place (neither form spills to scratch)
    ("fa_bwd_d256.hip", []),
    # FP8: d = 64 and 128 allocate the same either way; at d = 256 (one wave
    # per SIMD) the VGPR form keeps the O accumulators where the rescale and
    # the epilogue use them
    ("fa_fp8.hip", VGPR_FORM),
    ("fa_merge.hip", []),
    ("fa_api.hip", []),
]
SOURCES = [os.path.join(CSRC, u) for u, _ in UNITS] + [os.path.join(CSRC, "fa_kernel.hpp"),
                                                       os.path.join(CSRC, "fa_bwd_kernel.hpp"),
                                                       os.path.join(CSRC, "fa_fp8_kernel.hpp"),
                                                       os.path.join(CSRC, "fa_internal.h")]


def _clean(stderr: str) -> str:
    return "\n".join(l for l in stderr.splitlines()
                     if "packed-fp32-ops' is not a recognized feature" not in l)


# Per-kernel register, scratch and LDS use reported by the compiler
# (kernel-resource-usage remarks), written next to the library by build().
RESOURCES_PATH = os.path.join(os.path.dirname(LIB_PATH), "libfa.resources.json")


def _resources(stderr: str) -> dict:
    """Kernel name -> resource fields from hipcc's kernel-resource-usage
    remarks (demangled with c++filt when it is available)."""
    rows, cur = {}, None
    for line in stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = rows.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z][A-Za-z \[\]/]*?): (\w+) \[", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = int(m.group(2)) if m.group(2).isdigit() else m.group(2)
    names = list(rows)
    try:
        out = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True,
                             check=True).stdout.splitlines()
        if len(out) == len(names):
            return {d: rows[n] for n, d in zip(names, out)}
    except (OSError, subprocess.CalledProcessError):
        pass
    return rows


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="fa_build_") as tmp:
        procs, objs = [], []
        for unit, extra in UNITS:
            obj = os.path.join(tmp, unit.replace(".hip", ".o"))
            cmd = [HIPCC, *COMMON, *extra, "-Rpass-analysis=kernel-resource-usage", "-c",
                   os.path.join(CSRC, unit), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((unit, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                 stderr=subprocess.PIPE, text=True)))
            objs.append(obj)
        failed, resources = [], {}
        for unit, p in procs:
            _, err = p.communicate()
            if p.returncode != 0:
                failed.append(f"{unit}:\n{_clean(err)}")
            else:
                resources.update({k: dict(v, unit=unit) for k, v in _resources(err).items()})
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join(failed))
        out_tmp = LIB_PATH + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out_tmp]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed:\n{_clean(res.stderr)}")
        os.replace(out_tmp, LIB_PATH)
    with open(RESOURCES_PATH, "w") as f:
        json.dump(resources, f, indent=1, sort_keys=True)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
