"""Build libw4a4.so: the HIP kernels and the C ABI, for gfx950 only.

    python -m mixed_precision_integer_amd.build

hipcc cross-compiles without a GPU. Packed-FP32 instructions are disabled
for the device code (-packed-fp32-ops); hipcc's host pass warns that it does
not know that target feature, which is harmless. MFMA accumulators are kept
in architectural VGPRs (-amdgpu-mfma-vgpr-form).
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libw4a4.so")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # MFMA accumulators in ordinary VGPRs: the fp32 epilogue reads them
           # with plain VALU ops instead of v_accvgpr_read copies
           "-mllvm", "-amdgpu-mfma-vgpr-form",
           "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"),
           *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
