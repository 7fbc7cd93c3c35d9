"""GPU parity of the W4A8 GEMM (w4a4_w4a8_gemm / _i32 through the C ABI)
against the oracle's W4A8 layer: per-token INT8 activation codes and scales,
packed INT4 weight codes and scales, and the exported group accumulators
bit-exact; Y within 1e-2 * max |Y_oracle|. W4A8 per channel and per group
follows the QQQ abstract on the "smoothquant" tag page (4-bit weights, 8-bit activations).
"""
import sys

import numpy as np
import pytest

import mixed_precision_integer_amd as w4
from mixed_precision_integer_amd import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 1e-2


def _say(msg):
    sys.stderr.write(f"\n[gpu case] {msg}\n")
    sys.stderr.flush()


def u32(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def operands(oracle, X, W, group):
    a = w4.quant_act_int8(torch.from_numpy(X).to(DEV))
    w = w4.pack_int4_weights_w4a8(torch.from_numpy(W).to(DEV), group)
    (qa8, sa8), (qw4, sw4) = oracle.w4a8_quantize(X, W, group)
    torch.cuda.synchronize()
    assert np.array_equal(a.q.cpu().numpy(), qa8), "INT8 activation codes"
    assert np.array_equal(u32(a.s.cpu().numpy()), u32(sa8)), "token scales"
    assert np.array_equal(w.q.cpu().numpy(), oracle.pack_nibbles(qw4, X.shape[1] // 2)), "INT4 weight codes"
    assert np.array_equal(u32(w.s.cpu().numpy()), u32(sw4)), "weight scales"
    return a, w, ((qa8, sa8), (qw4, sw4))


def check_y(got, ref):
    got, ref = got.astype(np.float64), ref.astype(np.float64)
    assert np.all(np.isfinite(got))
    assert np.abs(got - ref).max() <= TOL * np.abs(ref).max()


W4A8 = [
    # M, N, K, group
    (16, 256, 256, 0),
    (200, 300, 1024, 0),        # ragged M and N
    (130, 257, 1152, 128),      # group 128, G = 9, ragged N
    (300, 130, 2048, 256),      # group 256: two K-tiles per group
    (37, 200, 640, 0),
    (1, 128, 512, 0),           # one token
    (70, 90, 384, 128),
    (512, 512, 4096, 128),      # several full tiles each way
]


@pytest.mark.parametrize("M,N,K,group", W4A8)
def test_w4a8_parity(oracle, M, N, K, group):
    _say(f"w4a8 M={M} N={N} K={K} group={group}")
    X, W, _ = wl.draw(M, N, K, 0, seed=M + N + K + group)
    a, w, (qa, qw) = operands(oracle, X, W, group)
    mm, nn = np.meshgrid(np.arange(M, dtype=np.int32), np.arange(N, dtype=np.int32), indexing="ij")
    acc, ystar = oracle.w4a8_linear_at(qa, qw, group, mm.reshape(-1), nn.reshape(-1))
    G = acc.shape[1]
    g = w4.w4a8_gemm_i32(a, w)
    y = w4.w4a8_gemm(a, w)
    torch.cuda.synchronize()
    assert np.array_equal(g.cpu().numpy(), acc.reshape(M, N, G).transpose(2, 0, 1)), "group accumulators"
    check_y(y.cpu().numpy(), oracle.to_fp16(ystar).reshape(M, N))


def test_w4a8_extreme_codes(oracle):
    """Codes at the ends of both ranges (activations +-127, weights -8 .. 7
    from hand-set rows), accumulated over the longest K the int32 guard allows
    in this test's budget."""
    _say("w4a8 extreme codes")
    M, N, K = 64, 64, 8192
    rng = np.random.default_rng(9)
    X = (rng.choice([-1.0, 1.0], (M, K)) * 127).astype(np.float16)
    W = rng.choice([-7.0, 7.0], (N, K)).astype(np.float16)
    a, w, (qa, qw) = operands(oracle, X, W, 0)
    mm, nn = np.meshgrid(np.arange(M, dtype=np.int32), np.arange(N, dtype=np.int32), indexing="ij")
    acc, ystar = oracle.w4a8_linear_at(qa, qw, 0, mm.reshape(-1), nn.reshape(-1))
    g = w4.w4a8_gemm_i32(a, w)
    torch.cuda.synchronize()
    assert np.array_equal(g.cpu().numpy()[0], acc.reshape(M, N))


@pytest.mark.parametrize("M,N,K,group", [(2048, 4096, 4096, 128), (4096, 11008, 4096, 0)],
                         ids=["qproj_g128", "upproj_per_channel"])
def test_w4a8_full_size(oracle, M, N, K, group):
    _say(f"w4a8 full size M={M} N={N} K={K} group={group}")
    X, W, _ = wl.draw(M, N, K, 0, seed=M + N + group)
    a, w, (qa, qw) = operands(oracle, X, W, group)
    rng = np.random.default_rng(1)
    mi = rng.integers(0, M, 4096).astype(np.int32)
    ni = rng.integers(0, N, 4096).astype(np.int32)
    acc, ystar = oracle.w4a8_linear_at(qa, qw, group, mi, ni)
    g = w4.w4a8_gemm_i32(a, w)
    y = w4.w4a8_gemm(a, w)
    mt, nt = torch.from_numpy(mi).long().to(DEV), torch.from_numpy(ni).long().to(DEV)
    got = g[:, mt, nt].cpu().numpy().T
    ys = y[mt, nt].cpu().numpy()
    assert np.array_equal(got, acc), "group accumulators (sampled)"
    check_y(ys, oracle.to_fp16(ystar))
