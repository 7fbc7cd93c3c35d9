"""The fused layer call with the library's static workspace
(w4a4_quant_gemm_static, for callers that cannot allocate), through the C
ABI: on calls in a row with different shapes (split K, then a smaller decode
batch, then split K again, reusing the array's counters) its Y equals
w4a4_quant_gemm's with a fresh workspace bit for bit, and matches the oracle.
"""
import ctypes
import sys

import numpy as np
import pytest

import mixed_precision_integer_amd as w4
from mixed_precision_integer_amd import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    sys.stderr.write(f"\n[gpu case] {msg}\n")
    sys.stderr.flush()


def test_static_workspace_calls_in_a_row(oracle):
    L = w4.lib()
    assert L.w4a4_quant_gemm_static_max_bytes() == 32 << 20
    N, K, n_out, group = 384, 4224, 128, 128
    X, W, o = wl.draw(200, N, K, n_out, seed=4242, outlier_factor=30.0)
    perm = torch.from_numpy(w4.make_perm(K, o)).to(DEV)
    w = w4.pack_int4_weights(torch.from_numpy(W).to(DEV), perm, n_out, group)
    perm_o = oracle.make_perm(K, o)
    qw = oracle.quantize_rows(W, perm_o, n_out, group)
    for M in (200, 37, 160):                  # split K, decode kernel (smaller), split K again
        _say(f"static workspace M={M} kernel={w4.quant_gemm_kernel_name(M, N, K, n_out, group)}")
        Xd = torch.from_numpy(np.ascontiguousarray(X[:M])).to(DEV)
        ref = w4.quant_gemm(Xd, perm, w)      # fresh zeroed workspace
        y = torch.full_like(ref, float("nan"))
        st = L.w4a4_quant_gemm_static(Xd.data_ptr(), K, perm.data_ptr(), w.q4.data_ptr(), w.q8.data_ptr(),
                                      w.s4.data_ptr(), w.s8.data_ptr(), M, N, K, n_out, group, y.data_ptr(), N,
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0, w4.STATUS.get(st, st)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"M={M}: the static-workspace call differs from w4a4_quant_gemm"
        qa = oracle.quantize_rows(X[:M], perm_o, n_out, group)
        _, _, ystar = oracle.linear_dense(qa, qw, group)
        want = oracle.to_fp16(ystar).astype(np.float64)
        got = y.cpu().numpy().astype(np.float64)
        assert np.abs(got - want).max() <= 1e-2 * np.abs(want).max()
    assert w4.outlier_gemm_workspace_bytes(200, N, K, n_out, group) > 0      # the shapes really split K
    assert w4.outlier_gemm_workspace_bytes(37, N, K, n_out, group) == 0


def test_static_workspace_rejects_oversized_shapes():
    L = w4.lib()
    # the down_proj activation codes alone exceed the array: rejected on the host
    M, N, K, n_out = 8192, 8192, 22016, 256
    assert w4.quant_gemm_workspace_bytes(M, N, K, n_out, 0) > L.w4a4_quant_gemm_static_max_bytes()
    fake = 1 << 20
    st = L.w4a4_quant_gemm_static(fake, K, fake, fake, fake, fake, fake, M, N, K, n_out, 0, fake, N, None)
    assert w4.STATUS[st] == "W4A4_ERR_UNSUPPORTED"
