"""The kernel names the library reports (w4a4_outlier_gemm_kernel_name,
w4a4_outlier_gemm_fp6_kernel_name, w4a4_quant_gemm_kernel_name) against the
kernel traces committed under profiles/: for every GEMM summary, the name the
bench recorded for its shape is the one the library reports now, and a kernel
of that name appears in the summary's rocprofv3 trace. CPU only (the name
calls are host functions)."""
import glob
import os
import re

import pytest

import mixed_precision_integer_amd as w4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SHAPE = re.compile(r"\(M=(\d+), N=(\d+), K=(\d+), n_out=(\d+), group=(\d+)\).*"
                   r"GEMM kernel for this shape: `([^`]+)`")


def gemm_summaries():
    out = []
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        text = open(path, encoding="utf-8").read()
        m = SHAPE.search(text)
        if m:
            out.append((os.path.basename(path), tuple(int(v) for v in m.groups()[:5]), m.group(6), text))
    return out


SUMMARIES = gemm_summaries()


def trace_names(text):
    """Kernel names (the part after the last ::) of the trace table."""
    names = []
    for line in text.splitlines():
        if line.startswith("| `w4a4::"):
            full = line.split("`")[1]
            names.append(full.split("(")[0].split("::")[-1] if "(" in full else full.rsplit("::", 1)[-1])
    return names


def test_there_are_gemm_summaries():
    assert len(SUMMARIES) >= 4


@pytest.mark.parametrize("name,shape,kernel,text", SUMMARIES, ids=[s[0] for s in SUMMARIES])
def test_reported_kernel_name_matches_the_trace(name, shape, kernel, text):
    reported = {w4.outlier_gemm_kernel_name(*shape), w4.outlier_gemm_fp6_kernel_name(*shape),
                w4.quant_gemm_kernel_name(*shape)}
    assert kernel in reported, (name, kernel, reported)
    names = trace_names(text)
    assert any(n == kernel or n.startswith(kernel + "<") for n in names), (name, kernel, names)
