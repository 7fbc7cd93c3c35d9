"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* the C oracle, compiled with -fsanitize=address,undefined, driven through
  every function on small and edge-case inputs (tests/csrc/oracle_san_driver.c);
* the host side of the C ABI (csrc/abi.hip, host code instrumented with
  -Xarch_host -fsanitize=...), driven through the layout helpers, queries,
  empty calls and argument rejects (tests/csrc/abi_host_san.cpp), linked
  ahead of libw4a4.so so that its own, instrumented, entry points run.
No kernel is launched. A sanitizer report aborts the driver (nonzero exit).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tests", "csrc")
PKG = os.path.join(ROOT, "mixed_precision_integer_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, (cmd[0], r.stdout[-2000:], r.stderr[-4000:])
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(ROOT, "oracle", "w4a4_oracle.c"), os.path.join(CSRC, "oracle_san_driver.c"),
          "-o", exe, "-lm"])
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:abort_on_error=1")
    r = _run([exe], env=env)
    assert "all checks passed" in r.stdout


def test_abi_host_checks_under_asan_ubsan(tmp_path):
    lib = os.path.join(PKG, "libw4a4.so")
    if not os.path.exists(HIPCC) or not os.path.exists(lib):
        pytest.skip("hipcc or the built library missing")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-Wno-unused-command-line-argument", *HOST_SAN]
    abi_o, drv_o, exe = (str(tmp_path / n) for n in ("abi_san.o", "drv.o", "abi_san"))
    _run([HIPCC, *common, *inc, "-c", os.path.join(PKG, "csrc", "abi.hip"), "-o", abi_o])
    _run([HIPCC, *common, *inc, "-c", os.path.join(CSRC, "abi_host_san.cpp"), "-o", drv_o])
    _run([HIPCC, "--offload-arch=gfx950", *HOST_SAN, drv_o, abi_o, "-L", PKG, "-lw4a4",
          "-Wl,-rpath," + PKG, "-o", exe])
    syms = _run(["nm", exe]).stdout
    assert " T w4a4_quant_reorder_act\n" in syms, "the driver must run its own instrumented entry points"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = _run([exe], env=env)
    assert "all checks passed" in r.stdout
