"""GPU parity of the FP6 prefill path (INT4 codes q held as the FP6 E2M3 values q / 8)
through the C ABI, against the CPU oracle.

* The u6 conversion (w4a4_repack_u6) is checked byte for byte against the
  oracle's pack_u6 of the oracle's own codes.
* The FP6 GEMM's integer sums are the layer's accumulators: its export
  (w4a4_outlier_gemm_fp6_i32, the same kernel and main loop as the product)
  must equal the oracle's acc4 / acc8 exactly, and its Y the product's Y bit
  for bit; Y is within 1e-2 * max |Y_oracle| of the oracle's fp64 dequant.
* The fused FP6 layer call equals producer + repack + FP6 GEMM bit for bit.
Every case compares every output.
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


@pytest.fixture(autouse=True)
def _name_the_case(request):
    sys.stderr.write(f"\n[gpu case] {request.node.nodeid}\n")
    sys.stderr.flush()
    yield
    torch.cuda.synchronize()


def check_y(y_gpu, y_ref_fp16):
    ref = y_ref_fp16.astype(np.float64)
    got = y_gpu.astype(np.float64)
    amax = np.abs(ref).max()
    err = np.abs(got - ref).max()
    assert np.all(np.isfinite(got))
    assert err <= TOL * amax, f"max err {err} vs bound {TOL * amax}"
    return err / max(amax, 1e-30)


def fp6_compare(oracle, X, W, outliers, group=0):
    M, K = X.shape
    N = W.shape[0]
    n_out = len(outliers)
    K_n = K - n_out
    perm = torch.from_numpy(w4.make_perm(K, outliers)).to(DEV)
    Xd, Wd = torch.from_numpy(X).to(DEV), torch.from_numpy(W).to(DEV)
    a = w4.quant_reorder_act(Xd, perm, n_out, group)
    wq = w4.pack_int4_weights(Wd, perm, n_out, group)
    af, wf = w4.to_fp6(a), w4.to_fp6(wq)
    perm_o = oracle.make_perm(K, outliers)
    qa = oracle.quantize_rows(X, perm_o, n_out, group)
    qw = oracle.quantize_rows(W, perm_o, n_out, group)
    torch.cuda.synchronize()
    # the u6 conversion, byte for byte, for both operands
    for op, q, rows in ((af, qa[0], M), (wf, qw[0], N)):
        want = oracle.pack_u6(q, w4.pitch4_bytes(K_n))
        assert op.u6.numel() == want.size == w4.u6_bytes(rows, K_n)
        assert np.array_equal(op.u6.cpu().numpy(), want), "u6 bytes"
    # the producer that writes u6 directly: the same bytes, codes and scales
    au = w4.quant_reorder_act_u6(Xd, perm, n_out, group)
    assert torch.equal(au.u6, af.u6), "u6 producer differs from producer + repack"
    assert torch.equal(au.s4, af.s4) and torch.equal(au.s8, af.s8)
    if n_out:
        assert torch.equal(au.q8, af.q8)
    acc4, acc8, ystar = oracle.linear_dense(qa, qw, group)
    g4, g8, y_exp = w4.outlier_gemm_fp6_i32(af, wf)
    y = w4.outlier_gemm_fp6(af, wf)
    yf = w4.quant_gemm_fp6(Xd, perm, wf)
    y_i8 = w4.w4a4_outlier_gemm(a, wq)
    torch.cuda.synchronize()
    assert torch.equal(y, y_exp), "the accumulator export's launch wrote a different Y"
    assert np.array_equal(g4.cpu().numpy(), acc4), "acc4 (every group)"
    if n_out:
        assert np.array_equal(g8.cpu().numpy(), acc8), "acc8"
    rel = check_y(y.cpu().numpy(), oracle.to_fp16(ystar))
    assert torch.equal(yf, y), "fused FP6 call differs from producer + repack + FP6 GEMM"
    # the i8 path forms the same integer sums; Y may differ only by the fp32 order
    check_y(y_i8.cpu().numpy(), y.cpu().numpy())
    return rel


CASES = [
    # M, N, K, n_out
    (256, 256, 320, 64),            # one tile, K_n = 256: two K-tiles, one tail tile
    (300, 520, 1152, 128),          # ragged M and N (edge tiles), two tail tiles
    (37, 200, 640, 100),            # one partial tile, tail of 100 padded to 128
    (1, 128, 512, 0),               # one token, no outliers
    (512, 768, 2304, 256),          # several tiles, four tail tiles
    (513, 257, 4160, 64),           # ragged by one in both directions, 65 K-tiles (odd)
    (96, 160, 21760 + 256, 256),    # the longest K of the workloads
]


@pytest.mark.parametrize("M,N,K,n_out", CASES)
def test_fp6_parity(oracle, M, N, K, n_out):
    X, W, o = wl.draw(M, N, K, n_out, seed=M + 5 * N + K, outlier_factor=40.0)
    fp6_compare(oracle, X, W, o)


GROUP_CASES = [
    # M, N, K, n_out (group 128: K_n a multiple of 128)
    (256, 128, 384, 128),           # one tile, two groups, two tail tiles
    (300, 200, 1152, 128),          # ragged M and N, eight groups
    (37, 520, 640, 0),              # one partial row tile, no outliers, four groups
    (513, 257, 4352, 256),          # ragged by one, 32 groups, four tail tiles
    (64, 96, 21760 + 256, 256),     # the longest K: 170 groups
]


@pytest.mark.parametrize("M,N,K,n_out", GROUP_CASES)
def test_fp6_group_parity(oracle, M, N, K, n_out):
    """The 128-channel group kernel: every group's exact integer sums, the
    tail sums, Y, the fused call, the u6 producer with group scales."""
    X, W, o = wl.draw(M, N, K, n_out, seed=M + 3 * N + K, outlier_factor=40.0)
    fp6_compare(oracle, X, W, o, group=128)


DECODE_CASES = [
    # M, N, K, n_out (group 128; 33 to 128 rows: the FP6 decode kernel)
    (33, 512, 1152, 128),           # two row blocks (the second holds one row), nine groups
    (70, 100, 2176, 128),           # three row blocks, ragged N (a partial last workgroup)
    (128, 256, 8320, 128),          # four row blocks, the longest K it takes (64 groups)
    (100, 64, 640, 0),              # no outliers, five groups: some group ranges are empty
    (65, 32, 384, 256),             # one group, four tail tiles, one workgroup
    (250, 96, 2176, 128),           # eight row blocks (the last one partial), 16 groups
]


@pytest.mark.parametrize("M,N,K,n_out", DECODE_CASES)
def test_fp6_decode_parity(oracle, M, N, K, n_out):
    """The FP6 decode kernel: every group's exact sums and the tail sums from
    its main loop, Y, the fused call and the i8 path's Y."""
    assert w4.outlier_gemm_fp6_kernel_name(M, N, K, n_out, 128).startswith("gemm_fp6_decode_kernel")
    X, W, o = wl.draw(M, N, K, n_out, seed=M + 7 * N + K, outlier_factor=40.0)
    fp6_compare(oracle, X, W, o, group=128)


@pytest.mark.parametrize("M", [64, 128, 256])
def test_fp6_decode_full_size(oracle, M):
    """The Llama-65B decode shape (N = K = 8192, 128 outliers, group 128) at
    64, 128 and 256 token rows, every output compared."""
    X, W, o = wl.draw_workload(wl.DECODE_65B, M)
    fp6_compare(oracle, X, W, o, group=128)


def test_fp6_extreme_codes(oracle):
    """All -8 codes (magnitude 8, the largest value used: E2M3 1 times 8) and random
    full-range codes over the longest K: the sums reach 21760 * 64."""
    rng = np.random.default_rng(321)
    M, N, K_n, n_out = 64, 96, 21760, 256
    for mode in ("all_min", "random"):
        if mode == "all_min":
            qa4 = np.full((M, K_n), -8, np.int8); qw4 = np.full((N, K_n), -8, np.int8)
        else:
            qa4 = rng.integers(-8, 8, (M, K_n), dtype=np.int8); qw4 = rng.integers(-8, 8, (N, K_n), dtype=np.int8)
        qa8 = rng.integers(-128, 128, (M, n_out), dtype=np.int8)
        qw8 = rng.integers(-128, 128, (N, n_out), dtype=np.int8)
        sa4 = rng.uniform(0.5, 2, (M, 1)).astype(np.float32); sw4 = rng.uniform(1e-3, 2e-3, (N, 1)).astype(np.float32)
        sa8 = rng.uniform(0.5, 2, M).astype(np.float32); sw8 = rng.uniform(1e-4, 2e-4, N).astype(np.float32)
        t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)  # noqa: E731

        def operand(q4, s4, q8, s8):
            rows = q4.shape[0]
            u6 = t(oracle.pack_u6(q4, w4.pitch4_bytes(K_n)))
            p8 = np.zeros((rows, 256), np.int8); p8[:, :n_out] = q8
            return w4.Fp6Operand(u6, t(p8), t(s4), t(s8), K_n + n_out, n_out, 0)

        a = operand(qa4, sa4, qa8, sa8)
        w = operand(qw4, sw4, qw8, sw8)
        acc4, acc8, ystar = oracle.linear_dense((qa4, sa4, qa8, sa8), (qw4, sw4, qw8, sw8), 0)
        g4, g8, y = w4.outlier_gemm_fp6_i32(a, w)
        torch.cuda.synchronize()
        assert np.array_equal(g4[0].cpu().numpy(), acc4[0]), mode
        assert np.array_equal(g8.cpu().numpy(), acc8), mode
        check_y(y.cpu().numpy(), oracle.to_fp16(ystar))


@pytest.mark.parametrize("work", [wl.UPPROJ_7B, wl.DOWNPROJ_65B, wl.QPROJ_7B], ids=lambda w: w.name)
def test_fp6_full_size_workload(oracle, work):
    X, W, o = wl.draw_workload(work)
    sys.stderr.write(f"[gpu case] FP6 full size {work.name}: "
                     f"{w4.outlier_gemm_fp6_kernel_name(work.M, work.N, work.K, work.n_out, work.group)}\n")
    sys.stderr.flush()
    fp6_compare(oracle, X, W, o, work.group)


@pytest.mark.parametrize("M,K,n_out,group", [
    (37, 640, 100, 0),         # rows past M in the last block; tail of 100, ragged head chunk
    (64, 1003, 11, 0),         # K and K_n not multiples of 8 (ragged row end: the row kernel)
    (1, 256, 0, 0),            # one row, no outliers
    (200, 4096, 128, 0),       # the 4096 row bucket, several row blocks
    (3000, 4096, 512, 0),      # more rows than resident workgroups; a tail word on every lane
    (300, 8192, 64, 0),        # the 8192 bucket
    (70, 16384, 7, 0),         # the 16384 bucket, ragged head and tail words
    (33, 22016, 256, 0),       # the longest rows (24576 bucket)
    (5, 24576, 3072, 0),       # the longest row; one tail word per lane of the 768-lane workgroup
    (37, 768, 128, 128),       # 128-channel group scales
    (2048, 4096, 128, 128),    # q_proj-shaped rows with group scales
    (9, 24576, 128, 128),      # group scales on the longest rows
    (1100, 22016, 256, 0),     # several rows per workgroup of the 24576 bucket
    (700, 20096, 128, 128),    # the same with group scales
])
def test_u6_producer(oracle, M, K, n_out, group):
    """w4a4_quant_reorder_act_u6 against the oracle: u6 bytes (rows past M up
    to the end of their block written as code 0 over garbage), INT8 tail and
    scales bit-exact."""
    sys.stderr.write(f"[gpu case] u6 producer M={M} K={K} n_out={n_out} group={group}\n")
    sys.stderr.flush()
    X, _, o = wl.draw(M, 8, K, n_out, seed=M * 7 + K, outlier_factor=40.0)
    perm_o = oracle.make_perm(K, o)
    perm = torch.from_numpy(perm_o).to(DEV)
    K_n = K - n_out
    out = w4.alloc_fp6_operand(M, K, n_out, group, DEV)
    out.u6.fill_(0xFF)
    out.s4.fill_(float("nan"))
    if n_out:
        out.q8.fill_(0x55)
    ld = (K + 7) // 8 * 8                  # row pitch: a multiple of 8 halves
    Xd = torch.zeros((M, ld), dtype=torch.float16, device=DEV)
    Xd[:, :K] = torch.from_numpy(X).to(DEV)
    a = w4.quant_reorder_act_u6(Xd[:, :K], perm, n_out, group, out=out)
    torch.cuda.synchronize()
    q4, s4, q8, s8 = oracle.quantize_rows(X, perm_o, n_out, group)
    assert np.array_equal(a.u6.cpu().numpy(), oracle.pack_u6(q4, w4.pitch4_bytes(K_n)))
    assert np.array_equal(a.s4.cpu().numpy().reshape(s4.shape), s4)
    assert np.array_equal(a.s8.cpu().numpy(), s8)
    if n_out:
        assert np.array_equal(a.q8.cpu().numpy()[:, :n_out], q8)
        assert not a.q8.cpu().numpy()[:, n_out:].any()


def test_fp6_kernel_names():
    assert w4.outlier_gemm_fp6_kernel_name(2048, 4096, 4096, 128, 128) == "gemm_fp6_group_kernel<false>"
    assert w4.outlier_gemm_fp6_kernel_name(128, 8192, 8192, 128, 128) == "gemm_fp6_decode_kernel<4, false>"
    assert w4.outlier_gemm_fp6_kernel_name(64, 8192, 8192, 128, 128) == "gemm_fp6_decode_kernel<2, false>"
    assert w4.outlier_gemm_fp6_kernel_name(256, 8192, 8192, 128, 128) == "gemm_fp6_decode_kernel<8, false>"
    assert w4.outlier_gemm_fp6_kernel_name(160, 8192, 8192, 128, 128) == "gemm_fp6_group_kernel<false>"
    assert w4.outlier_gemm_fp6_kernel_name(257, 8192, 8192, 128, 128) == "gemm_fp6_group_kernel<false>"
    assert w4.outlier_gemm_fp6_kernel_name(4096, 11008, 4096, 256, 0) == "gemm_fp6_big_kernel<false>"
    assert w4.outlier_gemm_fp6_kernel_name(2048, 4096, 4352, 256, 256) is None    # groups of 256


@pytest.mark.parametrize("M,N,K,n_out,group", [
    (512, 512, 640, 64, 0),         # 256 x 256 kernel: interior tiles
    (300, 520, 1152, 128, 0),       # 256 x 256 kernel: edge tiles
    (384, 384, 1152, 128, 128),     # group kernel, interior tiles
    (200, 264, 1152, 128, 128),     # group kernel, edge tiles
    (96, 256, 1152, 128, 128),      # decode kernel
])
@pytest.mark.parametrize("pad,col", [(8, 0), (4, 0), (1, 1), (0, 3)], ids=["ld16B", "ld8B", "ld2B", "off2B"])
def test_fp6_strided_output(M, N, K, n_out, group, pad, col):
    """Y written into a view with another row stride or a start that is only
    8- or 2-byte aligned takes the epilogues' narrower store paths; it must
    equal the contiguous result bit for bit, and nothing outside the view may
    change."""
    rng = np.random.default_rng(M + N + pad)
    X = (rng.standard_normal((M, K)) * 2).astype(np.float16)
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float16)
    outliers = np.sort(rng.choice(K, n_out, replace=False)) if n_out else np.zeros(0, np.int64)
    perm = torch.from_numpy(w4.make_perm(K, outliers)).to(DEV)
    Xd, Wd = torch.from_numpy(X).to(DEV), torch.from_numpy(W).to(DEV)
    af = w4.to_fp6(w4.quant_reorder_act(Xd, perm, n_out, group))
    wf = w4.to_fp6(w4.pack_int4_weights(Wd, perm, n_out, group))
    ref = w4.outlier_gemm_fp6(af, wf)
    big = torch.full((M, N + pad + col), float("nan"), dtype=torch.float16, device=DEV)
    view = big[:, col:col + N]
    w4.outlier_gemm_fp6(af, wf, out=view)
    torch.cuda.synchronize()
    assert torch.equal(view, ref)
    outside = torch.cat([big[:, :col].flatten(), big[:, col + N:].flatten()])
    assert bool(torch.isnan(outside).all())


@pytest.mark.parametrize("M,N,K,n_out,group,norm", [
    (2048, 4096, 4224, 128, 128, False),   # group kernel (512 tiles)
    (1024, 4096, 2304, 256, 0, False),     # 256 x 256 kernel (64 tiles: below one per CU, i8 path)
    (4096, 4096, 2304, 256, 0, True),      # 256 x 256 kernel with the norm in front (256 tiles)
    (96, 8192, 1152, 128, 128, False),     # FP6 decode kernel (256 stripes)
    (8, 8192, 1152, 128, 128, False),      # decode batch below the FP6 kernels: i8 path
])
def test_layer_object_fp6(M, N, K, n_out, group, norm):
    """W4A4Linear(fp6=True) runs the FP6 GEMM where it fills the chip: its Y
    equals the explicit FP6 launches bit for bit there, and the i8 layer's Y
    within the fp32-order tolerance everywhere."""
    sys.stderr.write(f"[gpu case] layer object fp6 M={M} N={N} K={K} n_out={n_out} group={group} norm={norm}\n")
    sys.stderr.flush()
    X, W, o = wl.draw(M, N, K, n_out, seed=M + N + K, outlier_factor=30.0)
    Xd, Wd = torch.from_numpy(X).to(DEV), torch.from_numpy(W).to(DEV)
    g = torch.from_numpy(wl.draw_norm_weight(K, seed=K)).to(DEV) if norm else None
    layer = w4.W4A4Linear(Wd, o, group, norm_weight=g, fp6=True)
    ref_layer = w4.W4A4Linear(Wd, o, group, norm_weight=g)
    y, y_i8 = layer(Xd), ref_layer(Xd)
    fills = w4.fp6_path_fills_chip(M, N, K, n_out, group)
    if fills:
        perm = layer.perm
        a = (w4.rmsnorm_quant_reorder_act_u6(Xd, g, 1e-6, perm, n_out, group) if norm
             else w4.quant_reorder_act_u6(Xd, perm, n_out, group))
        y_fp6 = w4.outlier_gemm_fp6(a, layer.weight_fp6)
        torch.cuda.synchronize()
        assert torch.equal(y, y_fp6), "the layer's FP6 call"
    torch.cuda.synchronize()
    assert fills == ((M, N) != (1024, 4096) and M != 8), "shape classes of the cases"
    check_y(y.cpu().numpy(), y_i8.cpu().numpy())
