"""The HIP quantizer replaces the per-element IEEE division x / s by
q0 = x * r, e = fma(-q0, s, x), q1 = fma(e, r, q0) with r = fl32(1 / s)
computed once per block (Markstein's correction step). Codes must stay
bit-identical to the definition q = rint(fl32(x / s)), so this test proves
q1 == fl32(x / s) exhaustively for every input the quantizer can see: every
positive fp16 block absmax a, every fp16 x with |x| <= a, and both qmax = 7
(INT4) and qmax = 127 (INT8). It also proves |rint(q1)| <= qmax on the same domain, so the clamp of
the definition never fires and the kernel may omit it. About 2e9 cases, a few
seconds with OpenMP.
"""
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))


def test_markstein_quotient_is_exact_for_all_fp16_blocks():
    src = os.path.join(HERE, "csrc", "exact_quotient_check.c")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "eqc")
        subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", src,
                        "-o", exe, "-lm"], check=True)
        res = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    print(res.stdout)
    assert res.returncode == 0, res.stdout
    assert res.stdout.count("mismatches=0") == 2
    assert res.stdout.count("beyond_qmax=0") == 2
