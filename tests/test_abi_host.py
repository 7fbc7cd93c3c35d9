"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

* libw4a4.so loads and exports every function include/w4a4.h declares;
* the host helpers follow the layout contract of the header;
* invalid calls are rejected by the host checks before any device work.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import mixed_precision_integer_amd as w4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a4.h")

OK, INVALID, UNSUPPORTED, ALIGN, HIP, WS = range(6)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a4_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 12
    L = w4.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(w4.EXPORTED) == names


def test_status_strings():
    L = w4.lib()
    for code, name in w4.STATUS.items():
        assert L.w4a4_status_string(code).decode() == name
    assert L.w4a4_status_string(99).decode() == "W4A4_ERR_UNKNOWN"


@pytest.mark.parametrize("K_n", [0, 1, 127, 128, 129, 240, 3968, 21760])
def test_pitch4(K_n):
    assert w4.pitch4_bytes(K_n) == ((K_n + 127) // 128) * 128 // 2


@pytest.mark.parametrize("n_out", [0, 1, 16, 64, 65, 128, 256])
def test_pitch8(n_out):
    assert w4.pitch8_bytes(n_out) == ((n_out + 63) // 64) * 64


def test_num_groups():
    assert w4.num_groups(3968, 128) == 31
    assert w4.num_groups(240, 0) == 1
    assert w4.num_groups(0, 0) == 0
    assert w4.num_groups(100, 128) == -1
    assert w4.num_groups(100, -1) == -1


def test_make_perm_matches_definition():
    rng = np.random.default_rng(0)
    for K in (1, 7, 256, 4096):
        for n in (0, 1, K // 3, K):
            o = rng.choice(K, n, replace=False)
            p = w4.make_perm(K, o)
            assert sorted(p.tolist()) == list(range(K))
            assert p[K - n:].tolist() == sorted(o.tolist())
            assert np.all(np.diff(p[:K - n]) > 0)


@pytest.mark.parametrize("bad", [[1, 1], [-1], [9]])
def test_make_perm_rejects(bad):
    with pytest.raises(w4.W4A4Error) as e:
        w4.make_perm(9, bad)
    assert e.value.status == INVALID


# ---------------------------------------------------------------------------
# argument checks of the device entry points: every call below fails on the
# host, before any HIP call
# ---------------------------------------------------------------------------
FAKE = 1 << 20          # a 16-byte aligned non-null address; never dereferenced


def quant(**kw):
    args = dict(X=FAKE, ld=256, perm=FAKE, rows=4, K=256, n_out=16, group=0,
                q4=FAKE, q8=FAKE, s4=FAKE, s8=FAKE)
    args.update(kw)
    return w4.lib().w4a4_quant_reorder_act(*args.values(), None)


def gemm(**kw):
    args = dict(a4=FAKE, a8=FAKE, sa4=FAKE, sa8=FAKE, w4=FAKE, w8=FAKE, sw4=FAKE, sw8=FAKE,
                M=4, N=8, K=256, n_out=16, group=0, Y=FAKE, ldy=8, ws=None, ws_bytes=0)
    args.update(kw)
    return w4.lib().w4a4_outlier_gemm(*args.values(), None)


@pytest.mark.parametrize("kw,code", [
    (dict(K=0), INVALID), (dict(rows=-1), INVALID), (dict(n_out=300), INVALID),
    (dict(n_out=-1), INVALID), (dict(ld=100), INVALID), (dict(X=None), INVALID),
    (dict(q4=None), INVALID), (dict(q8=None), INVALID),
    (dict(s4=None), INVALID), (dict(s8=None), INVALID),
    (dict(group=100), INVALID),                    # does not divide K_n = 240
    (dict(K=272, ld=272, group=64), UNSUPPORTED),  # divides, but not a multiple of 128
    (dict(X=FAKE + 2), ALIGN), (dict(ld=260), ALIGN), (dict(perm=FAKE + 4), ALIGN),
    (dict(q4=FAKE + 8), ALIGN), (dict(s4=FAKE + 2), ALIGN),
    (dict(K=140000, ld=140000, n_out=0), UNSUPPORTED),  # int32 guard of the accumulators
    (dict(K=90000, ld=90000, n_out=0), UNSUPPORTED),    # row larger than LDS
    (dict(K=24584, ld=24584, n_out=0), UNSUPPORTED),    # one step past the longest row (24576)
])
def test_quant_rejects(kw, code):
    assert quant(**kw) == code


def quant_u6(**kw):
    args = dict(X=FAKE, ld=256, perm=FAKE, rows=4, K=256, n_out=16, group=0,
                u6=FAKE, q8=FAKE, s4=FAKE, s8=FAKE)
    args.update(kw)
    return w4.lib().w4a4_quant_reorder_act_u6(*args.values(), None)


@pytest.mark.parametrize("kw,code", [
    (dict(group=64, K=272, ld=272), UNSUPPORTED),     # groups are multiples of 128
    (dict(u6=None), INVALID), (dict(q8=None), INVALID), (dict(s4=None), INVALID),
    (dict(u6=FAKE + 8), ALIGN), (dict(X=FAKE + 2), ALIGN), (dict(K=0), INVALID),
    (dict(K=24584, ld=24584, n_out=0), UNSUPPORTED),
])
def test_quant_u6_rejects(kw, code):
    assert quant_u6(**kw) == code


def test_quant_u6_empty_is_ok():
    assert quant_u6(rows=0, X=None, u6=None, q8=None, s4=None, s8=None) == 0


def norm_quant(**kw):
    args = dict(X=FAKE, ld=256, gamma=FAKE, eps=1e-6, perm=FAKE, rows=4, K=256, n_out=16, group=0,
                q4=FAKE, q8=FAKE, s4=FAKE, s8=FAKE, rstd=None)
    args.update(kw)
    return w4.lib().w4a4_rmsnorm_quant_reorder_act(*args.values(), None)


@pytest.mark.parametrize("kw,code", [
    (dict(gamma=None), INVALID), (dict(eps=-1e-6), INVALID), (dict(eps=float("nan")), INVALID),
    (dict(eps=float("inf")), INVALID), (dict(gamma=FAKE + 1), ALIGN), (dict(rstd=FAKE + 2), ALIGN),
    (dict(K=0), INVALID), (dict(ld=100), INVALID), (dict(q4=None), INVALID),
    (dict(X=FAKE + 2), ALIGN), (dict(K=24584, ld=24584, n_out=0), UNSUPPORTED),
])
def test_norm_quant_rejects(kw, code):
    assert norm_quant(**kw) == code


def test_norm_quant_empty_is_ok():
    assert norm_quant(rows=0, X=None, gamma=None, perm=None, q4=None, q8=None, s4=None,
                      s8=None) == OK


def test_norm_quant_gemm_rejects():
    L = w4.lib()
    need = w4.quant_gemm_workspace_bytes(16, 256, 256, 16, 0)
    head = [FAKE, 256]
    tail = [FAKE, FAKE, FAKE, FAKE, FAKE, 16, 256, 256, 16, 0, FAKE, 256]
    assert L.w4a4_rmsnorm_quant_gemm(*head, None, 1e-6, *tail, FAKE, need, None) == INVALID
    assert L.w4a4_rmsnorm_quant_gemm(*head, FAKE, -1.0, *tail, FAKE, need, None) == INVALID
    assert L.w4a4_rmsnorm_quant_gemm(*head, FAKE, 1e-6, *tail, FAKE, need - 1, None) == WS
    assert L.w4a4_rmsnorm_quant_gemm(*head, FAKE, 1e-6, *tail, FAKE + 16, need, None) == ALIGN


def select(**kw):
    args = dict(X=FAKE, ld=256, rows=64, K=256, n_out=16, idx=FAKE, perm=FAKE, amax=None, ws=FAKE,
                ws_bytes=1 << 20)
    args.update(kw)
    return w4.lib().w4a4_select_outliers(*args.values(), None)


@pytest.mark.parametrize("kw,code", [
    (dict(K=0), INVALID), (dict(rows=-1), INVALID), (dict(n_out=-1), INVALID), (dict(n_out=257), INVALID),
    (dict(ld=200), INVALID), (dict(perm=None), INVALID), (dict(idx=None), INVALID), (dict(X=None), INVALID),
    (dict(K=40000, ld=40000), UNSUPPORTED), (dict(X=FAKE + 2), ALIGN), (dict(ld=260), ALIGN),
    (dict(perm=FAKE + 2), ALIGN), (dict(amax=FAKE + 1), ALIGN), (dict(ws_bytes=16), WS), (dict(ws=None), WS),
    (dict(ws=FAKE + 64), ALIGN),
])
def test_select_rejects(kw, code):
    assert select(**kw) == code


def test_select_workspace_query():
    assert w4.select_outliers_workspace_bytes(-1, 64) == 0
    assert w4.select_outliers_workspace_bytes(10, 0) == 0
    assert w4.select_outliers_workspace_bytes(10, 40000) == 0
    assert w4.select_outliers_workspace_bytes(0, 64) >= 64 * 2          # the keys alone
    big = w4.select_outliers_workspace_bytes(32768, 4096)
    assert 4096 * 2 < big < 64 << 20


def w4a8(**kw):
    args = dict(a8=FAKE, sa8=FAKE, w4=FAKE, sw4=FAKE, M=4, N=8, K=256, group=0, Y=FAKE, ldy=8)
    args.update(kw)
    return w4.lib().w4a4_w4a8_gemm(*args.values(), None)


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), INVALID), (dict(K=0), INVALID), (dict(group=100), INVALID), (dict(ldy=4), INVALID),
    (dict(a8=None), INVALID), (dict(sw4=None), INVALID), (dict(Y=None), INVALID),
    (dict(K=200), UNSUPPORTED), (dict(K=384, group=192), UNSUPPORTED), (dict(K=131072), UNSUPPORTED),
    (dict(a8=FAKE + 8), ALIGN), (dict(w4=FAKE + 4), ALIGN), (dict(Y=FAKE + 1), ALIGN),
])
def test_w4a8_rejects(kw, code):
    assert w4a8(**kw) == code


def test_w4a8_empty_is_ok():
    assert w4a8(M=0, a8=None, sa8=None, Y=None) == OK
    assert w4.lib().w4a4_w4a8_gemm_i32(None, None, 0, 8, 256, 0, None, None) == OK


def kvq(**kw):
    args = dict(X=FAKE, ldx=512, T=4, H=4, D=128, bits=4, slots=None, num_slots=8, cq=FAKE, cs=FAKE)
    args.update(kw)
    return w4.lib().w4a4_kv_quant(*args.values(), None)


@pytest.mark.parametrize("kw,code", [
    (dict(bits=5), INVALID), (dict(D=96), UNSUPPORTED), (dict(num_slots=0), INVALID), (dict(num_slots=3), INVALID),
    (dict(ldx=256), INVALID), (dict(X=None), INVALID), (dict(cq=None), INVALID), (dict(T=-1), INVALID),
    (dict(X=FAKE + 2), ALIGN), (dict(ldx=516), ALIGN), (dict(cq=FAKE + 4), ALIGN), (dict(cs=FAKE + 2), ALIGN),
])
def test_kv_quant_rejects(kw, code):
    assert kvq(**kw) == code


def test_kv_empty_is_ok():
    assert kvq(T=0, X=None, cq=None, cs=None) == OK
    assert w4.lib().w4a4_kv_dequant(None, None, 0, None, 0, 4, 128, 4, None, 512, None) == OK
    assert w4.lib().w4a4_kv_dequant(FAKE, FAKE, 8, None, 4, 4, 128, 8, FAKE, 256, None) == INVALID  # ldy < H D
    assert w4.lib().w4a4_kv_dequant(FAKE, FAKE, 8, None, 4, 4, 128, 8, FAKE + 2, 512, None) == ALIGN
    assert w4.lib().w4a4_kv_dequant(FAKE, FAKE, 8, None, 4, 4, 128, 8, FAKE, 516, None) == ALIGN


def test_quant_empty_is_ok():
    assert quant(rows=0, X=None, perm=None, q4=None, q8=None, s4=None, s8=None) == OK


@pytest.mark.parametrize("kw,code", [
    (dict(N=-1), INVALID), (dict(K=0), INVALID), (dict(ldy=4), INVALID),
    (dict(a4=None), INVALID), (dict(w8=None), INVALID), (dict(sa4=None), INVALID),
    (dict(sw8=None), INVALID), (dict(Y=None), INVALID),
    (dict(group=100), INVALID), (dict(group=48), UNSUPPORTED), (dict(K=272, group=64), UNSUPPORTED),
    (dict(a4=FAKE + 8), ALIGN), (dict(w8=FAKE + 4), ALIGN), (dict(Y=FAKE + 1), ALIGN),
    (dict(sa8=FAKE + 2), ALIGN),
])
def test_gemm_rejects(kw, code):
    assert gemm(**kw) == code


def test_gemm_empty_is_ok():
    assert gemm(M=0, a4=None, a8=None, sa4=None, sa8=None, Y=None) == OK
    assert gemm(N=0, w4=None, w8=None, sw4=None, sw8=None, Y=None, ldy=0) == OK


def test_gemm_no_outliers_needs_no_tail_pointers():
    # n_out = 0 must not require tail pointers; the call then reaches the
    # launch, which needs a GPU, so only check the empty-shape variant here
    assert gemm(M=0, n_out=0, a8=None, w8=None, sa8=None, sw8=None) == OK


def test_quant_gemm_workspace_rules():
    L = w4.lib()
    need = w4.quant_gemm_workspace_bytes(16, 256, 256, 16, 0)
    assert need >= 16 * 128 + 16 * 64 + 16 * 4 + 16 * 4
    args = [FAKE, 256, FAKE, FAKE, FAKE, FAKE, FAKE, 16, 256, 256, 16, 0, FAKE, 256]
    assert L.w4a4_quant_gemm(*args, FAKE, need - 1, None) == WS
    assert L.w4a4_quant_gemm(*args, None, need, None) == WS
    assert L.w4a4_quant_gemm(*args, FAKE + 16, need, None) == ALIGN


def test_device_calls_fail_loudly_without_gpu():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    X = torch.zeros((4, 256), dtype=torch.float16)
    perm = torch.arange(256, dtype=torch.int32)
    with pytest.raises(ValueError):
        w4.quant_reorder_act(X, perm, 16, 0)


@pytest.mark.parametrize("shape,name", [
    ((1, 8192, 8192, 128, 128), "gemm_decode_kernel<1, false>"),   # decode batch: weights streamed once
    ((32, 8192, 8192, 128, 128), "gemm_decode_kernel<4, false>"),
    ((16, 256, 256, 16, 0), "gemm_decode_kernel<2, false>"),       # the tiny per-row layer
    ((2048, 4096, 4096, 128, 128), "gemm_group_kernel<false>"), # 128-channel groups
    ((2048, 11008, 4096, 256, 0), "gemm_big_kernel"),           # per-row scales, >= 256 large tiles
    ((48, 384, 4224, 128, 128), "gemm_decode_rows_kernel<2, false>"),   # two row blocks
    ((96, 384, 4224, 128, 128), "gemm_decode_rows_kernel<3, false>"),
    ((128, 8192, 8192, 128, 128), "gemm_decode_rows_kernel<4, false>"),
    ((256, 8192, 8192, 128, 128), "gemm_kernel<128, 128, 2, 2, 4, false, true>"),   # split K
    ((48, 384, 17536, 128, 128), "gemm_kernel<64, 64, 2, 2, 4, false, true>"),      # K_n past the decode range
    ((200, 300, 1024, 32, 0), "gemm_kernel<128, 128, 2, 2, 4, false, false>"),
    ((0, 1, 1, 0, 0), None),                                    # rejected shapes
    ((4, 4, 130, 0, 128), None),
])
def test_gemm_kernel_name(shape, name):
    assert w4.outlier_gemm_kernel_name(*shape) == name


def test_gemm_rejects_rows_past_32bit_offsets():
    """Operand rows are addressed by 32-bit byte offsets: a shape whose last
    packed row would start at 4 GiB or more is rejected before any launch."""
    # K_n = 21760 -> 10880-byte rows; 394759 rows reach 2^32
    K, n_out = 22016, 256
    assert gemm(M=394800, N=8, K=K, n_out=n_out, ldy=8) == UNSUPPORTED
    assert gemm(M=4, N=394800, K=K, n_out=n_out, ldy=394800) == UNSUPPORTED
    L = w4.lib()
    need = w4.quant_gemm_workspace_bytes(394800, 8, K, n_out, 0)
    assert L.w4a4_quant_gemm(FAKE, K, FAKE, FAKE, FAKE, FAKE, FAKE, 394800, 8, K, n_out, 0, FAKE, 8,
                             FAKE, need, None) == UNSUPPORTED


def gemm_i32(**kw):
    args = dict(a4=FAKE, a8=FAKE, sa4=FAKE, sa8=FAKE, w4=FAKE, w8=FAKE, sw4=FAKE, sw8=FAKE,
                M=4, N=8, K=256, n_out=16, group=0, Y=FAKE, ldy=8, ws=None, ws_bytes=0,
                acc4=FAKE, acc8=FAKE)
    args.update(kw)
    return w4.lib().w4a4_outlier_gemm_i32(*args.values(), None)


@pytest.mark.parametrize("kw,code", [
    (dict(acc4=None), INVALID), (dict(acc8=None), INVALID), (dict(Y=None), INVALID),
    (dict(sa4=None), INVALID), (dict(acc4=FAKE + 2), ALIGN), (dict(K=272, group=64), UNSUPPORTED),
])
def test_gemm_i32_rejects(kw, code):
    assert gemm_i32(**kw) == code


def test_gemm_i32_empty_is_ok():
    assert gemm_i32(M=0, a4=None, a8=None, sa4=None, sa8=None, Y=None, acc4=None, acc8=None) == OK


def test_quant_gemm_workspace_keeps_the_counters_first():
    """The fused call's workspace reserves the GEMM's arrival-counter block at
    offset 0 for every shape, so the activation codes of one call never land
    on the counters of a later split-K call sharing the workspace."""
    for shape in [(256, 8192, 8192, 128, 128), (200, 8192, 8192, 128, 128), (64, 8192, 8192, 128, 128),
                  (16, 256, 256, 16, 0)]:
        M, N, K, n_out, g = shape
        gemm_ws = w4.outlier_gemm_workspace_bytes(*shape)
        act = (M * w4.pitch4_bytes(K - n_out) + M * w4.pitch8_bytes(n_out) + 4 * M * max(w4.num_groups(K - n_out, g), 0)
               + 4 * M)
        assert w4.quant_gemm_workspace_bytes(*shape) >= max(gemm_ws, 2048) + act
    assert w4.outlier_gemm_workspace_bytes(256, 8192, 8192, 128, 128) > 0      # these two split K
    assert w4.outlier_gemm_workspace_bytes(200, 8192, 8192, 128, 128) > 0


def test_one_launch_decode_path_bounds():
    """The fused layer call takes one launch for at most 2 rows, 128-channel
    groups, at most 128 outliers and K_n <= 16384; other shapes keep the
    producer + GEMM launches (a pure function of the shape)."""
    assert w4.quant_gemm_kernel_name(1, 8192, 8192, 128, 128) == "decode_fused_kernel"
    assert w4.quant_gemm_kernel_name(2, 256, 16384 + 64, 64, 128) == "decode_fused_kernel"
    assert w4.quant_gemm_kernel_name(3, 256, 1152, 128, 128) == "gemm_decode_kernel<1, false>"
    assert w4.quant_gemm_kernel_name(2, 256, 1152, 128, 0) == "gemm_decode_kernel<1, false>"
    assert w4.quant_gemm_kernel_name(2, 256, 1280, 256, 128) == "gemm_decode_kernel<1, false>"
    assert w4.quant_gemm_kernel_name(2, 256, 16384 + 256, 128, 128) != "decode_fused_kernel"
    assert w4.quant_gemm_kernel_name(2, 256, 1152, 128, 256) == "gemm_decode_kernel<1, false>"
    assert w4.quant_gemm_kernel_name(2048, 4096, 4096, 128, 128) == w4.outlier_gemm_kernel_name(2048, 4096, 4096, 128, 128)
    assert w4.quant_gemm_kernel_name(0, 256, 1152, 128, 128) is None


PROBE = os.path.join(ROOT, "mixed_precision_integer_amd", "libw4a4_probe.so")


def _probe():
    if not os.path.exists(PROBE):
        pytest.skip("libw4a4_probe.so is not built")
    L = ctypes.CDLL(PROBE)
    L.w4a4_read_probe.restype = ctypes.c_int32
    L.w4a4_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    L.w4a4_read_probe_out_words.restype = ctypes.c_int64
    L.w4a4_read_probe_out_words.argtypes = [ctypes.c_int32]
    return L


def test_read_probe_library_host_checks():
    """The streaming-read probe (a measurement tool in a library of its own)
    exports its two calls and rejects bad arguments before any launch."""
    L = _probe()
    assert L.w4a4_read_probe_out_words(256) == 256 * 256
    assert L.w4a4_read_probe_out_words(0) == -1
    fake = ctypes.c_void_p(1 << 20)          # never dereferenced: every call below is rejected
    assert L.w4a4_read_probe(None, 1024, 256, 4, 0, fake, None) == 1
    assert L.w4a4_read_probe(fake, 1000, 256, 4, 0, fake, None) == 1      # not a multiple of 16
    assert L.w4a4_read_probe(fake, 1024, 0, 4, 0, fake, None) == 1        # no workgroups
    assert L.w4a4_read_probe(fake, 1024, 256, 3, 0, fake, None) == 1      # depth not offered
    assert L.w4a4_read_probe(ctypes.c_void_p((1 << 20) + 4), 1024, 256, 4, 0, fake, None) == 1
