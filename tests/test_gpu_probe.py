"""The streaming-read probe (bench.py --read-probe-mib) runs through its C
call for every depth and load kind on a small buffer, including a size that
is not a whole number of rounds and more workgroups than rounds. It reads
only; the output buffer is written only in a case a seeded buffer of this
size does not produce, so it stays as it was filled."""
import ctypes
import os
import sys

import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "mixed_precision_integer_amd", "libw4a4_probe.so")


@pytest.mark.parametrize("nbytes,wgs", [(1 << 20, 256), ((1 << 20) + 48, 512), (4096, 64)])
def test_read_probe_runs(nbytes, wgs):
    sys.stderr.write(f"\n[gpu case] read probe {nbytes} bytes, {wgs} workgroups\n")
    sys.stderr.flush()
    L = ctypes.CDLL(PROBE)
    L.w4a4_read_probe.restype = ctypes.c_int32
    L.w4a4_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    L.w4a4_read_probe_out_words.restype = ctypes.c_int64
    L.w4a4_read_probe_out_words.argtypes = [ctypes.c_int32]
    g = torch.Generator().manual_seed(7)
    buf = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, generator=g).to("cuda:0")
    out = torch.full((int(L.w4a4_read_probe_out_words(wgs)),), -1, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()
    for depth in (1, 2, 4, 8, 16):
        for nt in (0, 1):
            assert L.w4a4_read_probe(buf.data_ptr(), nbytes, wgs, depth, nt, out.data_ptr(),
                                     ctypes.c_void_p(stream.cuda_stream)) == 0
    torch.cuda.synchronize()
    assert bool((out == -1).all())
