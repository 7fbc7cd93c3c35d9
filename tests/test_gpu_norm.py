"""GPU parity of the producer fused with the preceding RMSNorm.

The HIP path (w4a4_rmsnorm_quant_reorder_act / w4a4_rmsnorm_quant_gemm,
through the C ABI) against the oracle's rmsnorm_quantize_rows: the norm
factor rstd, codes, padding bytes and scales bit-exact; the fused layer's fp16
output within 1e-2 * max |Y_oracle| and bit-identical to norm-producer +
GEMM run as two calls. The norm follows the standard RMSNorm of the Llama
models the Atom summary page evaluates; fusing it with the quantizer follows
that page's Summary paragraph 2 and Interesting ideas I2.
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


def pitch4(K_n):
    return ((K_n + 127) // 128) * 128 // 2


def pitch8(n_out):
    return ((n_out + 63) // 64) * 64


def u32(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def to_dev(X, ld=None):
    """X on the device, with row pitch ld (>= K, a multiple of 8) when given."""
    rows, K = X.shape
    ld = ld or K
    buf = torch.zeros((rows, ld), dtype=torch.float16, device=DEV)
    buf[:, :K] = torch.from_numpy(X).to(DEV)
    return buf[:, :K]


def check_norm_producer(oracle, X, gamma, eps, outliers, group, ld=None):
    rows, K = X.shape
    n_out = len(outliers)
    perm_h = oracle.make_perm(K, outliers)                  # the oracle's own permutation
    perm = torch.from_numpy(w4.make_perm(K, outliers)).to(DEV)
    op, rstd = w4.rmsnorm_quant_reorder_act(to_dev(X, ld), torch.from_numpy(gamma).to(DEV), eps,
                                            perm, n_out, group, want_rstd=True)
    q4, s4, q8, s8 = oracle.rmsnorm_quantize_rows(X, gamma, eps, perm_h, n_out, group)
    r = oracle.rms_rstd(X, eps)
    torch.cuda.synchronize()
    assert np.array_equal(u32(rstd.cpu().numpy()), u32(r)), "rstd"
    assert np.array_equal(op.q4.cpu().numpy(), oracle.pack_nibbles(q4, pitch4(K - n_out))), "INT4 codes"
    if n_out:
        p8 = np.zeros((rows, pitch8(n_out)), np.int8)
        p8[:, :n_out] = q8
        assert np.array_equal(op.q8.cpu().numpy(), p8), "INT8 codes"
    assert np.array_equal(u32(op.s4.cpu().numpy()), u32(s4)), "INT4 scales"
    assert np.array_equal(u32(op.s8.cpu().numpy()), u32(s8 if n_out else np.zeros(rows, np.float32))), "INT8 scales"
    return op


NORM_PRODUCER = [
    # rows, K, n_out, group, eps
    (2048, 4096, 128, 128, 1e-6),   # the Llama-7B q_proj activations, every row
    (37, 4608, 512, 512, 1e-5),     # 512-channel groups, 8192 bucket
    (65, 1152, 128, 0, 1e-6),       # per-row scales
    (3, 8192, 128, 128, 1e-6),      # decode-length batch: the row kernel (the norm needs whole rows)
    (5, 16384, 256, 0, 1e-5),       # 1024-lane bucket
    (2, 24576, 256, 128, 1e-6),     # the longest row
    (6, 3200, 1100, 0, 1e-6),       # tail of 1100: more than one tail word per lane
    (7, 1024, 0, 128, 0.0),         # no outliers, eps = 0
    (2, 256, 256, 128, 1e-6),       # no INT4 head
]


@pytest.mark.parametrize("rows,K,n_out,group,eps", NORM_PRODUCER)
def test_norm_producer_parity(oracle, rows, K, n_out, group, eps):
    _say(f"norm producer rows={rows} K={K} n_out={n_out} group={group} eps={eps}")
    X, _, o = wl.draw(rows, 1, K, n_out, seed=rows + K + n_out + 17, outlier_factor=30.0)
    g = wl.draw_norm_weight(K, seed=K)
    check_norm_producer(oracle, X, g, eps, o, group)


def test_norm_ragged_row_and_pitch(oracle):
    """K not a multiple of 8 (the row's last channels come by plain loads) and
    a row pitch larger than K."""
    _say("norm producer ragged K=1004 ld=1016")
    X, _, o = wl.draw(9, 1, 1004, 44, seed=3, outlier_factor=30.0)
    check_norm_producer(oracle, X, wl.draw_norm_weight(1004, seed=3), 1e-6, o, 0, ld=1016)


@pytest.mark.parametrize("group", [0, 128])
def test_norm_special_rows(oracle, group):
    """A zero row (rstd = 0 at eps = 0), a row of equal magnitudes 2^-20 (fp16
    subnormals: exact sum of squares far below fp32's reach), one huge entry
    among small ones, gamma with negative and zero entries."""
    _say(f"norm special rows group={group}")
    K, n_out = 1152, 128
    rng = np.random.default_rng(8)
    X = np.zeros((5, K), np.float16)
    X[1] = (rng.choice([-1.0, 1.0], K) * 2.0 ** -20).astype(np.float16)
    X[2] = (rng.standard_normal(K) * 2.0 ** -6).astype(np.float16)
    X[2, 7] = 60000.0
    X[3] = rng.standard_normal(K).astype(np.float16)
    X[4] = 1.0
    g = wl.draw_norm_weight(K, seed=1)
    g[::5] = -g[::5]
    g[3] = 0.0
    o = rng.choice(K, n_out, replace=False).astype(np.int32)
    check_norm_producer(oracle, X, g, 0.0, o, group)


def test_norm_fused_layer(oracle):
    """rmsnorm_quant_gemm: every output of a mid-size layer against the oracle,
    and bit-identical to the norm producer followed by the GEMM."""
    M, N, K, n_out, group = 130, 257, 1152, 128, 128
    _say(f"norm fused layer M={M} N={N} K={K}")
    X, W, o = wl.draw(M, N, K, n_out, seed=41, outlier_factor=30.0)
    g = wl.draw_norm_weight(K, seed=41)
    perm_h = oracle.make_perm(K, o)
    perm = torch.from_numpy(w4.make_perm(K, o)).to(DEV)
    Xd, gd = torch.from_numpy(X).to(DEV), torch.from_numpy(g).to(DEV)
    w = w4.pack_int4_weights(torch.from_numpy(W).to(DEV), perm, n_out, group)
    y = w4.rmsnorm_quant_gemm(Xd, gd, 1e-6, perm, w)
    a = w4.rmsnorm_quant_reorder_act(Xd, gd, 1e-6, perm, n_out, group)
    y2 = w4.w4a4_outlier_gemm(a, w)
    qa = oracle.rmsnorm_quantize_rows(X, g, 1e-6, perm_h, n_out, group)
    qw = oracle.quantize_rows(W, perm_h, n_out, group)
    mm, nn = np.meshgrid(np.arange(M, dtype=np.int32), np.arange(N, dtype=np.int32), indexing="ij")
    _, _, ystar = oracle.linear_at(qa, qw, group, mm.reshape(-1), nn.reshape(-1))
    ref = oracle.to_fp16(ystar).reshape(M, N).astype(np.float64)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "fused layer differs from norm producer + GEMM"
    got = y.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    assert np.abs(got - ref).max() <= TOL * np.abs(ref).max()


def test_norm_full_size_qproj_layer(oracle):
    """The Llama-7B q_proj layer behind its RMSNorm at full size: every
    producer byte above, sampled outputs of the fused layer here."""
    work = wl.QPROJ_7B
    _say(f"norm fused layer {work.name}")
    X, W, o = wl.draw_workload(work)
    g = wl.draw_norm_weight(work.K, seed=work.seed)
    perm_h = oracle.make_perm(work.K, o)
    perm = torch.from_numpy(w4.make_perm(work.K, o)).to(DEV)
    w = w4.pack_int4_weights(torch.from_numpy(W).to(DEV), perm, work.n_out, work.group)
    y = w4.rmsnorm_quant_gemm(torch.from_numpy(X).to(DEV), torch.from_numpy(g).to(DEV), 1e-6,
                              perm, w)
    rng = np.random.default_rng(2)
    mi = rng.integers(0, work.M, 4096).astype(np.int32)
    ni = rng.integers(0, work.N, 4096).astype(np.int32)
    rows = np.unique(mi)
    qa = oracle.rmsnorm_quantize_rows(X[rows], g, 1e-6, perm_h, work.n_out, work.group)
    qw = oracle.quantize_rows(W, perm_h, work.n_out, work.group)
    _, _, ystar = oracle.linear_at(qa, qw, work.group, np.searchsorted(rows, mi).astype(np.int32), ni)
    got = y[torch.from_numpy(mi).long().to(DEV), torch.from_numpy(ni).long().to(DEV)].cpu().numpy()
    ref = oracle.to_fp16(ystar).astype(np.float64)
    assert np.all(np.isfinite(got))
    assert np.abs(got.astype(np.float64) - ref).max() <= TOL * np.abs(ref).max()


def test_norm_layer_object(oracle):
    """W4A4Linear with a norm weight runs the fused RMSNorm layer."""
    M, N, K, n_out, group = 24, 96, 512, 128, 128
    _say("norm W4A4Linear")
    X, W, o = wl.draw(M, N, K, n_out, seed=77, outlier_factor=30.0)
    g = wl.draw_norm_weight(K, seed=77)
    gd = torch.from_numpy(g).to(DEV)
    layer = w4.W4A4Linear(torch.from_numpy(W).to(DEV), o, group, norm_weight=gd, eps=1e-6)
    Xd = torch.from_numpy(X).to(DEV)
    y = layer(Xd)
    y2 = w4.rmsnorm_quant_gemm(Xd, gd, 1e-6, layer.perm, layer.weight)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)


def test_norm_empty_batch():
    K = 256
    X = torch.zeros((0, K), dtype=torch.float16, device=DEV)
    perm = torch.arange(K, dtype=torch.int32, device=DEV)
    op = w4.rmsnorm_quant_reorder_act(X, torch.ones(K, dtype=torch.float16, device=DEV), 1e-6,
                                      perm, 16, 0)
    assert op.q4.shape[0] == 0


@pytest.mark.parametrize("rows,K,n_out,group,eps", [c for c in NORM_PRODUCER if c[1] > c[2]] + [
    (1100, 22016, 256, 0, 1e-6),    # the Llama-65B down_proj rows, several per workgroup
])
def test_norm_producer_u6_parity(oracle, rows, K, n_out, group, eps):
    """The FP6 path's norm producer (w4a4_rmsnorm_quant_reorder_act_u6): the
    u6 head equals the oracle's pack_u6 of its normalized codes byte for byte
    (rows past the last one up to the end of their block included), and the
    rstd, the scales and the INT8 tail equal the oracle's."""
    _say(f"norm producer u6 rows={rows} K={K} n_out={n_out} group={group} eps={eps}")
    X, _, o = wl.draw(rows, 1, K, n_out, seed=rows + K + n_out + 17, outlier_factor=30.0)
    gamma = wl.draw_norm_weight(K, seed=K)
    perm_h = oracle.make_perm(K, o)
    perm = torch.from_numpy(perm_h).to(DEV)
    a, rstd = w4.rmsnorm_quant_reorder_act_u6(to_dev(X), torch.from_numpy(gamma).to(DEV), eps, perm, n_out, group,
                                              want_rstd=True)
    q4, s4, q8, s8 = oracle.rmsnorm_quantize_rows(X, gamma, eps, perm_h, n_out, group)
    r = oracle.rms_rstd(X, eps)
    torch.cuda.synchronize()
    assert np.array_equal(u32(rstd.cpu().numpy()), u32(r)), "rstd"
    assert np.array_equal(a.u6.cpu().numpy(), oracle.pack_u6(q4, pitch4(K - n_out))), "u6 head"
    if n_out:
        assert np.array_equal(a.q8.cpu().numpy()[:, :n_out], q8), "INT8 codes"
        assert not a.q8.cpu().numpy()[:, n_out:].any(), "INT8 padding"
    assert np.array_equal(u32(a.s4.cpu().numpy().reshape(s4.shape)), u32(s4)), "INT4 scales"
    assert np.array_equal(u32(a.s8.cpu().numpy()), u32(s8 if n_out else np.zeros(rows, np.float32))), "INT8 scales"
