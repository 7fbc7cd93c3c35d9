"""Build libw4a4.so: the HIP kernels and the C ABI, for gfx950 only.

    python -m mixed_precision_integer_amd.build

hipcc cross-compiles without a GPU. Each source is compiled to an object with
its own flags, then the objects are linked into one shared library.
Packed-FP32 instructions are disabled for all device code (-packed-fp32-ops);
hipcc's host pass warns that it does not know that target feature, which is
harmless. The 64 x 64 and 128 x 128 GEMM keeps MFMA accumulators in
architectural VGPRs (-amdgpu-mfma-vgpr-form), since its fp32 epilogue reads
them every scale group; the 256 x 256 GEMMs (i8 and FP6) hold 256 accumulator
registers per lane, which only fit as AGPRs, and are built without that option.
Sources are compiled in parallel (at most MAX_JOBS, else the CPU count).

The streaming-read probe (probe/read_probe.hip, a measurement tool that
bench.py --read-probe calls) is built into a library of its own,
libw4a4_probe.so, so that nothing of it enters the layer's library.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libw4a4.so")
PROBE_LIB = os.path.join(HERE, "libw4a4_probe.so")

COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]
# per-source extra flags (default: accumulators in architectural VGPRs)
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
EXTRA = {"gemm_big.hip": [], "gemm_fp6.hip": []}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed")


def build(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    tmp = LIB + ".tmp"
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with tempfile.TemporaryDirectory(prefix="w4a4_build_") as objdir:
        cmds, objs = [], []
        for src in srcs:
            name = os.path.basename(src)
            obj = os.path.join(objdir, name + ".o")
            cmds.append([hipcc(), *COMMON, *EXTRA.get(name, VGPR_FORM), *inc, "-c", src, "-o", obj])
            objs.append(obj)
        # one process per source, at most MAX_JOBS (or the CPU count) at a time
        with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
            for f in [pool.submit(_run, c, verbose) for c in cmds]:
                f.result()
        _run([hipcc(), "--offload-arch=gfx950", "-fPIC", "-shared", *objs, "-o", tmp], verbose)
        probe_tmp = PROBE_LIB + ".tmp"
        _run([hipcc(), *COMMON, "-shared", os.path.join(HERE, "probe", "read_probe.hip"), "-o", probe_tmp], verbose)
    os.replace(tmp, LIB)
    os.replace(probe_tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
