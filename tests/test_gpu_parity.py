"""GPU parity: the HIP path against the CPU oracle, through the C ABI.

Bars (from the layer's definition; the oracle is pinned separately):
* codes, padding bytes and fp32 scales of the producer: bit-exact;
* int32 accumulators of the GEMM: bit-exact. They come from
  w4a4_outlier_gemm_i32, which launches the kernel w4a4_outlier_gemm launches
  for the shape (one shape-only plan serves both) and writes the same Y; the
  tests check that Y bit for bit;
* fp16 output: max |Y - Y_oracle| <= 1e-2 * max |Y_oracle| (the GPU sums the
  scaled groups in fp32 in its own order; the oracle sums in fp64).

The oracle side always takes its own permutation (oracle.make_perm), so a
wrong permutation from the library's host helper would show.

Mid-size cases span several tiles with ragged M, N and K edges. The five
named workloads and the large-tile and group-tile shapes run at full size.
Every case compares every output: accumulators against the oracle's
whole-matrix GEMM (oracle.linear_dense, pinned to the per-position C oracle)
and Y against its fp64 dequant.
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


def pitch4(K_n):
    return ((K_n + 127) // 128) * 128 // 2


def pitch8(n_out):
    return ((n_out + 63) // 64) * 64


def as_u32(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def oracle_quant(oracle, A, perm, n_out, group):
    q4, s4, q8, s8 = oracle.quantize_rows(A, perm, n_out, group)
    p4 = oracle.pack_nibbles(q4, pitch4(q4.shape[1]))
    p8 = np.zeros((A.shape[0], pitch8(n_out)), np.int8)
    p8[:, :n_out] = q8
    return (q4, s4, q8, s8), p4, p8


def check_producer(oracle, gpu_op, A, perm, n_out, group):
    ref, p4, p8 = oracle_quant(oracle, A, perm, n_out, group)
    torch.cuda.synchronize()
    assert np.array_equal(gpu_op.q4.cpu().numpy(), p4), "INT4 codes / padding"
    if n_out:
        assert np.array_equal(gpu_op.q8.cpu().numpy(), p8), "INT8 codes / padding"
    assert np.array_equal(as_u32(gpu_op.s4.cpu().numpy()), as_u32(ref[1])), "INT4 scales"
    s8 = ref[3] if n_out else np.zeros(A.shape[0], np.float32)
    assert np.array_equal(as_u32(gpu_op.s8.cpu().numpy()), as_u32(s8)), "INT8 scales"
    return ref


def run_layer(X, W, outliers, group):
    K = X.shape[1]
    perm = torch.from_numpy(w4.make_perm(K, outliers)).to(DEV)
    Xd = torch.from_numpy(X).to(DEV)
    Wd = torch.from_numpy(W).to(DEV)
    n_out = len(outliers)
    a = w4.quant_reorder_act(Xd, perm, n_out, group)
    w = w4.pack_int4_weights(Wd, perm, n_out, group)
    return perm, Xd, a, w


def check_y(y_gpu, y_ref_fp16):
    ref = y_ref_fp16.astype(np.float64)
    got = y_gpu.astype(np.float64)
    amax = np.abs(ref).max()
    err = np.abs(got - ref).max()
    assert np.all(np.isfinite(got))
    assert err <= TOL * amax, f"max err {err} vs bound {TOL * amax}"
    return err / max(amax, 1e-30), int((y_gpu != y_ref_fp16).sum())


def full_compare(oracle, X, W, outliers, group):
    """Every output position: producer, accumulators, Y and the fused call."""
    M, K = X.shape
    N = W.shape[0]
    n_out = len(outliers)
    perm, Xd, a, w = run_layer(X, W, outliers, group)
    perm_o = oracle.make_perm(K, outliers)
    qa = check_producer(oracle, a, X, perm_o, n_out, group)
    qw = check_producer(oracle, w, W, perm_o, n_out, group)
    acc4, acc8, ystar = oracle.linear_dense(qa, qw, group)
    g4, g8, y_exp = w4.w4a4_outlier_gemm_i32(a, w)
    y = w4.w4a4_outlier_gemm(a, w)
    yf = w4.quant_gemm(Xd, perm, w)
    torch.cuda.synchronize()
    assert torch.equal(y, y_exp), "the accumulator export's launch wrote a different Y"
    G = acc4.shape[0]
    for t in range(G):                      # one group at a time (bounded host memory)
        assert np.array_equal(g4[t].cpu().numpy(), acc4[t]), f"acc4 group {t}"
    del g4
    if n_out:
        assert np.array_equal(g8.cpu().numpy(), acc8), "acc8"
    rel, ndiff = check_y(y.cpu().numpy(), oracle.to_fp16(ystar))
    assert torch.equal(yf, y), "fused call differs from producer + GEMM"
    return rel, ndiff


MID = [
    # M, N, K, n_out, group                 kernel the shape runs
    (16, 256, 256, 16, 0),          # decode kernel: the tiny workload's shape, other seed
    (200, 300, 1024, 32, 0),        # 128 x 128 generic kernel, ragged M and N, K_n = 992
    (130, 257, 1152, 128, 128),     # group-tile kernel, G = 8, ragged N
    (300, 130, 2176, 128, 256),     # 128 x 128 generic kernel: group 256 spans two K-tiles
    (37, 200, 640, 100, 0),         # row-block decode kernel (2 blocks): tail of 100 padded to 128
    (1, 128, 512, 0, 0),            # decode kernel: one token, no outliers
    (64, 64, 256, 256, 0),          # 64 x 64 generic kernel: every channel an outlier (plain W8A8)
    (70, 90, 384, 0, 128),          # row-block decode kernel (3 blocks): group mode, no outliers
    (512, 512, 4096, 128, 128),     # group-tile kernel, several full tiles each way
    (600, 300, 2304, 256, 0),       # 128 x 128 generic kernel (under 256 large tiles), ragged
    (520, 260, 1664, 128, 128),     # group-tile kernel with ragged M and N
]


@pytest.mark.parametrize("M,N,K,n_out,group", MID)
def test_mid_size_parity(oracle, M, N, K, n_out, group):
    X, W, o = wl.draw(M, N, K, n_out, seed=M * 7 + K, outlier_factor=40.0)
    full_compare(oracle, X, W, o, group)


# Shapes with few output tiles and long K: the GEMM splits K across workgroups
# (fp32 partials in the workspace, added in split order by the last split).
SPLIT_K = [
    # M, N, K, n_out, group (M <= 128 takes the decode kernel unless K_n > 16384)
    (48, 384, 17536, 128, 128),     # group mode, 64 x 64 tiles, K_n past the decode kernel's range
    (40, 1000, 16832, 64, 0),       # per-row scales, ragged N, split inside the one group
    (160, 384, 4224, 128, 128),     # 128 x 128 tiles, ragged M
    (150, 640, 4224, 128, 256),     # group of two K-tiles cut by splits
]


@pytest.mark.parametrize("M,N,K,n_out,group", SPLIT_K)
def test_split_k_parity(oracle, M, N, K, n_out, group):
    assert w4.outlier_gemm_workspace_bytes(M, N, K, n_out, group) > 0, "shape does not split K"
    X, W, o = wl.draw(M, N, K, n_out, seed=M * 11 + K, outlier_factor=30.0)
    full_compare(oracle, X, W, o, group)


def test_split_k_workspace_reuse(oracle):
    """One workspace for shapes with different tile and split counts, in turn:
    every call must leave the tile counters at zero for the next one."""
    shapes = [(48, 384, 17536, 128, 128), (40, 1000, 16832, 64, 0), (48, 384, 17536, 128, 128)]
    need = max(w4.outlier_gemm_workspace_bytes(*s) for s in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for i, (M, N, K, n_out, group) in enumerate(shapes):
        X, W, o = wl.draw(M, N, K, n_out, seed=50 + i)
        perm, Xd, a, w = run_layer(X, W, o, group)
        fresh = w4.w4a4_outlier_gemm(a, w)
        y = torch.empty_like(fresh)
        for _ in range(3):
            y.fill_(float("nan"))          # a split that never reduces would leave NaN
            st = w4.lib().w4a4_outlier_gemm(*w4._gemm_args(a, w, y, ws))
            assert st == 0
            torch.cuda.synchronize()
            assert torch.equal(y, fresh), f"shape {i}: reused workspace gives a different Y"


# Decode batches (M <= 128): the weights stream once through the decode
# kernel (eight waves per 32 output columns take the K-tiles in turn, the
# partial blocks are added in wave order).
DECODE = [
    # M, N, K, n_out, group
    (4, 384, 4224, 128, 128),       # group mode
    (3, 1000, 4096, 64, 0),         # per-row scales, ragged N
    (1, 640, 2176, 128, 256),       # one token, group of two K-tiles
    (32, 2048, 2176, 128, 128),     # a full 32-row block
    (17, 300, 1536, 0, 0),          # no outlier tail, ragged N
    (9, 96, 8320, 128, 128),        # one workgroup short of columns, 64 groups
    # token rows moved in runs of eight (XI = ceil(M / 8) DMA instructions per
    # pair); the slot rows past them hold stale bytes whose results are dropped
    (13, 256, 2176, 128, 128),      # two runs, the second ragged
    (24, 520, 4224, 128, 0),        # three full runs, per-row scales, ragged N
    (27, 64, 8320, 128, 128),       # four runs, the last ragged, 64 groups
    # 32 < M <= 128: two to four row blocks per wave, token fragments from L2
    (48, 384, 4224, 128, 128),      # two blocks, the second ragged
    (64, 1000, 4096, 64, 0),        # two full blocks, per-row scales, ragged N
    (65, 300, 1536, 0, 0),          # three blocks (one row in the third), no tail
    (96, 96, 8320, 128, 128),       # three full blocks, 64 groups
    (100, 640, 2176, 128, 256),     # four blocks, group of two K-tiles
    (128, 2048, 2176, 128, 128),    # four full blocks
]


@pytest.mark.parametrize("M,N,K,n_out,group", DECODE)
def test_decode_parity(oracle, M, N, K, n_out, group):
    assert w4.outlier_gemm_workspace_bytes(M, N, K, n_out, group) == 0
    assert w4.outlier_gemm_kernel_name(M, N, K, n_out, group).startswith("gemm_decode")
    X, W, o = wl.draw(M, N, K, n_out, seed=M * 13 + K, outlier_factor=30.0)
    full_compare(oracle, X, W, o, group)


def test_laplace_inputs(oracle):
    X, W, o = wl.draw(96, 160, 896, 64, seed=9, x_dist="laplace", outlier_factor=50.0)
    full_compare(oracle, X, W, o, 0)


def test_tiny_workload(oracle):
    X, W, o = wl.draw_workload(wl.TINY)
    full_compare(oracle, X, W, o, wl.TINY.group)


def test_special_values(oracle):
    """Zero rows, fp16 extremes and subnormals through the whole layer."""
    M, N, K, n_out = 40, 70, 512, 32
    X, W, o = wl.draw(M, N, K, n_out, seed=77)
    X[3] = 0                                      # all-zero token: s = 0, codes 0
    X[5, :8] = np.float16(65504)                   # fp16 max on a few channels (the
    X[6, 8:16] = -np.float16(65504)                # output itself stays finite)
    X[7, :] = np.float16(6e-8)                     # subnormal fp16
    X[8, ::2] = np.float16(-6e-8)
    W[2] = 0
    W[4, :] = np.float16(1e-7)
    full_compare(oracle, X, W, o, 0)


# ---------------------------------------------------------------------------
# the GEMM on hand-made operands: extreme codes (-8, -128) and int32 range
# ---------------------------------------------------------------------------
def upload_codes(oracle, q4, s4, q8, s8):
    rows = q4.shape[0]
    p4 = oracle.pack_nibbles(q4, pitch4(q4.shape[1]))
    p8 = np.zeros((rows, pitch8(q8.shape[1])), np.int8)
    p8[:, :q8.shape[1]] = q8
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)  # noqa: E731
    return w4.QuantizedOperand(t(p4), t(p8) if q8.shape[1] else None, t(s4), t(s8),
                               q4.shape[1] + q8.shape[1], q8.shape[1], 0)


@pytest.mark.parametrize("mode", ["random_full_range", "all_min"])
def test_gemm_extreme_codes(oracle, mode):
    rng = np.random.default_rng(123)
    M, N, K_n, n_out = 96, 160, 21760, 256          # the largest K_n of the workloads
    if mode == "all_min":
        qa4 = np.full((M, K_n), -8, np.int8); qw4 = np.full((N, K_n), -8, np.int8)
        qa8 = np.full((M, n_out), -128, np.int8); qw8 = np.full((N, n_out), -128, np.int8)
    else:
        qa4 = rng.integers(-8, 8, (M, K_n), dtype=np.int8); qw4 = rng.integers(-8, 8, (N, K_n), dtype=np.int8)
        qa8 = rng.integers(-128, 128, (M, n_out), dtype=np.int8)
        qw8 = rng.integers(-128, 128, (N, n_out), dtype=np.int8)
    sa4 = rng.uniform(0.5, 2, (M, 1)).astype(np.float32); sw4 = rng.uniform(1e-3, 2e-3, (N, 1)).astype(np.float32)
    sa8 = rng.uniform(0.5, 2, M).astype(np.float32); sw8 = rng.uniform(1e-4, 2e-4, N).astype(np.float32)
    a = upload_codes(oracle, qa4, sa4, qa8, sa8)
    w = upload_codes(oracle, qw4, sw4, qw8, sw8)
    mm, nn = np.meshgrid(np.arange(M, dtype=np.int32), np.arange(N, dtype=np.int32), indexing="ij")
    acc4, acc8, ystar = oracle.linear_at((qa4, sa4, qa8, sa8), (qw4, sw4, qw8, sw8), 0,
                                         mm.reshape(-1), nn.reshape(-1))
    g4, g8, y_exp = w4.w4a4_outlier_gemm_i32(a, w)
    y = w4.w4a4_outlier_gemm(a, w)
    torch.cuda.synchronize()
    assert torch.equal(y, y_exp)
    assert np.array_equal(g4.cpu().numpy()[0], acc4[:, 0].reshape(M, N))
    assert np.array_equal(g8.cpu().numpy(), acc8.reshape(M, N))
    check_y(y.cpu().numpy(), oracle.to_fp16(ystar).reshape(M, N))


# ---------------------------------------------------------------------------
# full-size workloads: every producer byte and every GEMM output
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("work", [wl.QPROJ_7B, wl.UPPROJ_7B, wl.DOWNPROJ_65B],
                         ids=lambda w: w.name)
def test_full_size_workload(oracle, work):
    X, W, o = wl.draw_workload(work)
    sys.stderr.write(f"[gpu case] full size {work.name}: "
                     f"{w4.outlier_gemm_kernel_name(work.M, work.N, work.K, work.n_out, work.group)}\n")
    sys.stderr.flush()
    full_compare(oracle, X, W, o, work.group)


# The activation producer on its own (codes, scales and padding bit-exact
# against the oracle). Batches of up to 64 rows with group sizes of 128 to
# 1024 channels take the wave-worker kernel (head chunks of 1024 channels, one
# wave for the outlier tail); longer batches, other group sizes, per-row
# scales and tails over 1024 channels take the row kernel.
PRODUCER = [
    # rows, K, n_out, group
    (1, 8192, 128, 128),        # one decode row over eight head chunks
    (5, 2176, 128, 256),        # 256-channel groups: 32-lane segments
    (37, 4608, 512, 512),       # 512-channel groups: whole-wave segments
    (9, 3072, 1024, 1024),      # group = the whole chunk; 1024 outliers (four tail words per lane)
    (64, 1152, 128, 128),       # the longest batch of the wave-worker kernel
    (65, 1152, 128, 128),       # one row more: row kernel
    (11, 1408, 256, 384),       # 384-channel groups: row kernel
    (6, 3200, 1100, 0),         # per-row scales: row kernel
    (3, 2112, 1088, 128),       # tail of 1088 channels: row kernel
    (7, 1024, 0, 128),          # no outliers
    (2, 256, 256, 128),         # no INT4 head at all
]


@pytest.mark.parametrize("rows,K,n_out,group", PRODUCER)
def test_producer_parity(oracle, rows, K, n_out, group):
    sys.stderr.write(f"[gpu case] producer rows={rows} K={K} n_out={n_out} group={group}\n")
    sys.stderr.flush()
    X, _, o = wl.draw(rows, 1, K, n_out, seed=rows + K + n_out, outlier_factor=30.0)
    perm = torch.from_numpy(w4.make_perm(K, o)).to(DEV)
    a = w4.quant_reorder_act(torch.from_numpy(X).to(DEV), perm, n_out, group)
    check_producer(oracle, a, X, oracle.make_perm(K, o), n_out, group)


# The longest row the producer takes (24576 channels, the 1024-lane bucket)
# through the producer alone and through the whole layer (a short batch: K
# past the decode kernels' range, so split K).
@pytest.mark.parametrize("n_out,group", [(256, 0), (256, 128), (0, 128)])
def test_longest_row(oracle, n_out, group):
    K = 24576
    sys.stderr.write(f"[gpu case] longest row K={K} n_out={n_out} group={group}\n")
    sys.stderr.flush()
    X, W, o = wl.draw(3, 200, K, n_out, seed=K + n_out + group, outlier_factor=30.0)
    full_compare(oracle, X, W, o, group)


# Per-row-scale shapes with at least 256 tiles of 256 x 256 take the
# large-tile kernel (accumulators in AGPRs, outlier tail folded in per block).
BIG_TILE = [
    # M, N, K, n_out, group
    (4096, 4096, 1152, 128, 0),     # 256 tiles exactly, two tail tiles
    (4000, 4100, 1304, 100, 0),     # ragged M, N and K_n (1204 -> 640-byte rows)
    (4096, 4096, 1024, 0, 0),       # no outlier tail
    (4096, 4352, 2048, 256, 1792),  # one group spanning the head, four tail tiles
]


@pytest.mark.parametrize("M,N,K,n_out,group", BIG_TILE)
def test_big_tile_parity(oracle, M, N, K, n_out, group):
    assert w4.outlier_gemm_kernel_name(M, N, K, n_out, group) == "gemm_big_kernel"
    X, W, o = wl.draw(M, N, K, n_out, seed=M + N + K, outlier_factor=40.0)
    full_compare(oracle, X, W, o, group)


# Shapes with 128-channel scale groups and more than 256 output tiles of
# 128 x 128 take the group-tile kernel (scale products on the matrix core,
# fp32 fold per group, the outlier tail as the first group).
GROUP_TILE = [
    # M, N, K, n_out, group
    (2048, 2100, 1280, 128, 128),   # ragged N, two tail tiles
    (2050, 2048, 1152, 0, 128),     # ragged M, no outlier tail
    (2176, 2112, 1344, 64, 128),    # one tail tile
    (2100, 2060, 1384, 104, 128),   # ragged M and N, tail of 104 padded to 128
    (2048, 2048, 4352, 256, 128),   # 32 groups, four tail tiles
]


@pytest.mark.parametrize("M,N,K,n_out,group", GROUP_TILE)
def test_group_tile_parity(oracle, M, N, K, n_out, group):
    assert w4.outlier_gemm_workspace_bytes(M, N, K, n_out, group) == 0, "shape splits K"
    assert w4.outlier_gemm_kernel_name(M, N, K, n_out, group) == "gemm_group_kernel<false>"
    X, W, o = wl.draw(M, N, K, n_out, seed=M + 3 * N + K, outlier_factor=30.0)
    rel, _ = full_compare(oracle, X, W, o, group)
    # The fp32 dequantization of every group adds far less than the fp16
    # rounding of the output (2^-11 of max |Y|), well inside the layer
    # tolerance: a fold that loses precision shows here first.
    assert rel <= 1e-3, f"group fold error {rel:.2e} of max |Y|"


@pytest.mark.parametrize("M", wl.DECODE_M)
def test_decode_sweep(oracle, M):
    """The 65B decode sweep at full size, every output, on the kernel each
    batch size runs in production (decode, row-block decode, split K)."""
    d = wl.DECODE_65B
    X, W, o = wl.draw_workload(d)
    sys.stderr.write(f"[gpu case] decode M={M}: {w4.outlier_gemm_kernel_name(M, d.N, d.K, d.n_out, d.group)}\n")
    sys.stderr.flush()
    full_compare(oracle, np.ascontiguousarray(X[:M]), W, o, d.group)


# Every production kernel class is reached by the cases of this file; the
# export runs the same plan, so its kernel is the production kernel.
PRODUCTION_KERNELS = {
    (16, 256, 256, 16, 0): "gemm_decode_kernel<2, false>",             # the tiny layer
    (2048, 4096, 4096, 128, 128): "gemm_group_kernel<false>",       # q_proj prefill
    (4096, 11008, 4096, 256, 0): "gemm_big_kernel",                 # up_proj prefill
    (8192, 8192, 22016, 256, 0): "gemm_big_kernel",                 # down_proj prefill
    (1, 8192, 8192, 128, 128): "gemm_decode_kernel<1, false>",         # decode sweep
    (8, 8192, 8192, 128, 128): "gemm_decode_kernel<1, false>",
    (32, 8192, 8192, 128, 128): "gemm_decode_kernel<4, false>",
    (128, 8192, 8192, 128, 128): "gemm_decode_rows_kernel<4, false>",
    (256, 8192, 8192, 128, 128): "gemm_kernel<128, 128, 2, 2, 4, false, true>",
}


def test_workload_kernels():
    for shape, name in PRODUCTION_KERNELS.items():
        assert w4.outlier_gemm_kernel_name(*shape) == name, shape


def test_quant_gemm_workspace_reuse(oracle):
    """One fused-call workspace for M = 256, 64, 200, 256 on the 65B decode
    shape (split K, decode kernel, split K): the activation codes of a
    non-split call must not land on the arrival counters of the next split
    one. Y starts as NaN so that a split that never reduces would show."""
    d = wl.DECODE_65B
    X, W, o = wl.draw_workload(d)
    perm = torch.from_numpy(w4.make_perm(d.K, o)).to(DEV)
    w = w4.pack_int4_weights(torch.from_numpy(W).to(DEV), perm, d.n_out, d.group)
    Ms = [256, 64, 200, 256]
    need = max(w4.quant_gemm_workspace_bytes(M, d.N, d.K, d.n_out, d.group) for M in Ms)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for M in Ms:
        Xd = torch.from_numpy(np.ascontiguousarray(X[:M])).to(DEV)
        fresh = w4.quant_gemm(Xd, perm, w)
        y = torch.full_like(fresh, float("nan"))
        w4.quant_gemm(Xd, perm, w, out=y, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y, fresh), f"M={M}: the reused workspace gives a different Y"


def test_layer_object_reuses_its_workspace(oracle):
    """W4A4Linear keeps one workspace across calls of different batch sizes."""
    d = wl.DECODE_65B
    X, W, o = wl.draw_workload(d)
    layer = w4.W4A4Linear(torch.from_numpy(W).to(DEV), o, d.group)
    for M in [256, 32, 200, 256, 1]:
        Xd = torch.from_numpy(np.ascontiguousarray(X[:M])).to(DEV)
        y = layer(Xd)
        ref = w4.quant_gemm(Xd, layer.perm, layer.weight)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"M={M}"


def test_repeatable(oracle):
    X, W, o = wl.draw(300, 260, 1280, 64, seed=5)
    perm, Xd, a, w = run_layer(X, W, o, 128 if (1280 - 64) % 128 == 0 else 0)
    y1 = w4.quant_gemm(Xd, perm, w)
    y2 = w4.quant_gemm(Xd, perm, w)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y3 = w4.quant_gemm(Xd, perm, w)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y1, y3)


def test_empty_batch():
    X = torch.zeros((0, 256), dtype=torch.float16, device=DEV)
    W = torch.randn((64, 256), device=DEV).half()
    perm = torch.from_numpy(w4.make_perm(256, [1, 2])).to(DEV)
    w = w4.pack_int4_weights(W, perm, 2, 0)
    y = w4.quant_gemm(X, perm, w)
    assert y.shape == (0, 64)
