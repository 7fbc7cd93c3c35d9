"""CPU oracle for the W4A4 + INT8-outlier hybrid linear layer.

TEST INFRASTRUCTURE ONLY. The product package never imports this module. Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it. It shares no code with the HIP path.

The arithmetic lives in ``w4a4_oracle.c`` (plain C, gcc, OpenMP over rows and
output positions). This wrapper only converts dtypes and shapes:

* fp16 inputs are widened to fp32 with numpy (exact);
* the fp64 result y* is rounded to fp16 with numpy's float64 -> float16 cast
  (round to nearest even, pinned in ``tests/test_oracle_pins.py``).

Sources: "QUIK: Towards End-to-End 4-Bit Inference on Generative Large
Language Models" (abstract) and "Atom: Low-bit Quantization for Efficient and
Accurate LLM Serving" (research summary page: Summary paragraph 2, Key points
item 5, Interesting ideas I1 and I3). Readings R1-R8 are listed in the header
of ``w4a4_oracle.c``.

Every function here is pinned by ``tests/test_oracle_pins.py`` against facts
that do not come from the oracle (closed forms, brute force on tiny inputs,
invariances and a hand-worked fixture in ``tests/golden/``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "w4a4_oracle.c")
_LIB = os.path.join(_HERE, "libw4a4_oracle.so")
_lib = None

_i8p = np.ctypeslib.ndpointer(np.int8, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")


def build() -> str:
    """Compile the C oracle with gcc (no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-std=c11", "-Wall", "-shared", "-fPIC", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    c_i32, c_i64 = ctypes.c_int32, ctypes.c_int64
    lib.w4o_max_threads.argtypes = []
    lib.w4o_max_threads.restype = ctypes.c_int
    lib.w4o_make_perm.argtypes = [c_i32, _i32p, c_i32, _i32p]
    lib.w4o_make_perm.restype = ctypes.c_int
    lib.w4o_quantize_block.argtypes = [_f32p, c_i32, c_i32, _i8p, ctypes.POINTER(ctypes.c_float)]
    lib.w4o_quantize_block.restype = None
    lib.w4o_num_groups.argtypes = [c_i32, c_i32]
    lib.w4o_num_groups.restype = c_i32
    lib.w4o_quantize_rows.argtypes = [_f32p, c_i64, c_i32, c_i64, _i32p, c_i32, c_i32,
                                      _i8p, _f32p, _i8p, _f32p]
    lib.w4o_quantize_rows.restype = ctypes.c_int
    lib.w4o_rms_rstd_rows.argtypes = [_f32p, c_i64, c_i32, c_i64, ctypes.c_float, _f32p]
    lib.w4o_rms_rstd_rows.restype = ctypes.c_int
    lib.w4o_pack_nibbles.argtypes = [_i8p, c_i64, c_i32, c_i64, _u8p]
    lib.w4o_pack_nibbles.restype = None
    lib.w4o_linear_at.argtypes = [_i8p, _f32p, _i8p, _f32p, _i8p, _f32p, _i8p, _f32p,
                                  c_i32, c_i32, c_i32, _i32p, _i32p, c_i64,
                                  _i32p, _i32p, _f64p]
    lib.w4o_linear_at.restype = ctypes.c_int
    lib.w4o_w4a8_linear_at.argtypes = [_i8p, _f32p, _i8p, _f32p, c_i32, c_i32, _i32p, _i32p, c_i64,
                                       _i32p, _f64p]
    lib.w4o_w4a8_linear_at.restype = ctypes.c_int
    _lib = lib
    return lib


def max_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().w4o_max_threads())


def num_groups(K_n: int, group: int) -> int:
    return int(_load().w4o_num_groups(K_n, group))


def make_perm(K: int, outlier_idx) -> np.ndarray:
    """Stable outlier permutation (reading R6). Raises ValueError on bad indices."""
    o = np.ascontiguousarray(np.asarray(outlier_idx, dtype=np.int32).reshape(-1))
    perm = np.zeros(max(K, 1), dtype=np.int32)
    if _load().w4o_make_perm(K, o if o.size else np.zeros(1, np.int32), o.size, perm) != 0:
        raise ValueError("outlier indices out of range or repeated")
    return perm[:K]


def quantize_block(v, qmax: int):
    """Quantize one block; returns (codes int8, scale float32)."""
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float32).reshape(-1))
    q = np.zeros(max(v.size, 1), dtype=np.int8)
    s = ctypes.c_float(0.0)
    _load().w4o_quantize_block(v if v.size else np.zeros(1, np.float32), v.size, qmax, q,
                               ctypes.byref(s))
    return q[: v.size], np.float32(s.value)


def quantize_rows(X, perm, n_out: int, group: int):
    """Reorder + quantize every row of X [rows, K] (fp16 or fp32).

    Returns (q4 int8 [rows, K_n], s4 f32 [rows, G], q8 int8 [rows, n_out],
    s8 f32 [rows]), codes unpacked one per byte.
    """
    X = np.asarray(X)
    rows, K = X.shape
    Xf = np.ascontiguousarray(X.astype(np.float32))
    K_n = K - n_out
    G = num_groups(K_n, group) if K_n >= 0 else 0
    q4 = np.zeros((rows, K_n), np.int8)
    s4 = np.zeros((rows, G), np.float32)
    q8 = np.zeros((rows, n_out), np.int8)
    s8 = np.zeros(rows, np.float32)
    pad = lambda a, dt: a if a.size else np.zeros(1, dt)  # noqa: E731
    rc = _load().w4o_quantize_rows(pad(Xf, np.float32), rows, K, K,
                                   pad(np.ascontiguousarray(perm, np.int32), np.int32),
                                   n_out, group, pad(q4, np.int8), pad(s4, np.float32),
                                   pad(q8, np.int8), pad(s8, np.float32))
    if rc != 0:
        raise ValueError("group must divide K - n_out")
    return q4, s4, q8, s8


def rms_rstd(X, eps: float) -> np.ndarray:
    """RMSNorm factor of every row of X [rows, K] (fp16): float32 [rows].

    Readings N1-N3 in ``w4a4_oracle.c``: exact sum of squares, then
    fl32(1 / sqrt(fl64(fl64(S) / K) + eps)) in binary64; 0 for a zero row at
    eps = 0.
    """
    X = np.asarray(X)
    if X.dtype != np.float16:
        raise TypeError("rms_rstd takes fp16 rows")
    rows, K = X.shape
    Xf = np.ascontiguousarray(X.astype(np.float32))
    out = np.zeros(max(rows, 1), np.float32)
    if rows and _load().w4o_rms_rstd_rows(Xf, rows, K, K, float(eps), out) != 0:
        raise ValueError("K must be in [1, 32768] and eps finite and >= 0")
    return out[:rows]


def rmsnorm(X, gamma, eps: float) -> np.ndarray:
    """RMSNorm of fp16 rows as an fp16 model computes it: the row is scaled in
    fp32 by rstd and rounded to fp16, then multiplied by the fp16 weight gamma
    (the product of two fp16 values is exact in fp32, so one rounding to fp16).
    Both roundings are to nearest even (numpy's float32 -> float16 cast)."""
    X = np.asarray(X)
    g = np.asarray(gamma)
    if g.dtype != np.float16 or g.shape != (X.shape[1],):
        raise TypeError("gamma must be fp16 [K]")
    r = rms_rstd(X, eps)
    h = (X.astype(np.float32) * r[:, None]).astype(np.float16)
    return (h.astype(np.float32) * g.astype(np.float32)).astype(np.float16)


def rmsnorm_quantize_rows(X, gamma, eps: float, perm, n_out: int, group: int):
    """The fused producer's result: quantize_rows of rmsnorm(X, gamma, eps)."""
    return quantize_rows(rmsnorm(X, gamma, eps), perm, n_out, group)


def channel_absmax(Xcal) -> np.ndarray:
    """Per-channel max |x| over the rows of a calibration batch Xcal [R, K]
    (fp16): fp16 [K], exact (0 for R == 0)."""
    X = np.asarray(Xcal)
    if X.dtype != np.float16 or X.ndim != 2:
        raise TypeError("channel_absmax takes an fp16 [R, K] batch")
    if X.shape[0] == 0:
        return np.zeros(X.shape[1], np.float16)
    return np.abs(X).max(axis=0)


def select_outliers(Xcal, n_out: int) -> np.ndarray:
    """Offline outlier-channel selection (reading S1): the n_out channels with
    the largest calibration absmax, ties to the lower channel index, returned
    in ascending channel order (int32 [n_out]). The pages keep a small set of
    outlier channels in 8 bits (Atom summary page, Summary paragraph 2) but
    give no rule for choosing them; the absmax is the statistic the quantizer
    itself scales by."""
    a = channel_absmax(Xcal).astype(np.float32)
    K = a.size
    if not 0 <= n_out <= K:
        raise ValueError("n_out must be in [0, K]")
    order = np.lexsort((np.arange(K), -a))      # by score descending, then index ascending
    return np.sort(order[:n_out]).astype(np.int32)


def pack_nibbles(q4, pitch: int) -> np.ndarray:
    """Pack INT4 codes two per byte, low nibble first, zero padded to pitch."""
    q4 = np.ascontiguousarray(q4, dtype=np.int8)
    rows, K_n = q4.shape
    out = np.zeros((rows, pitch), np.uint8)
    if rows and pitch:
        _load().w4o_pack_nibbles(q4 if q4.size else np.zeros(1, np.int8), rows, K_n,
                                 pitch, out)
    return out


# ---------------------------------------------------------------------------
# FP6 (E2M3) packing of INT4 codes for the prefill GEMM
# ---------------------------------------------------------------------------
def e2m3_value(code: int) -> float:
    """Value of a 6-bit FP6 E2M3 code (OCP Microscaling Formats v1.0): sign
    bit 5, exponent bits 4..3 with bias 1, mantissa bits 2..0; exponent 0 is
    subnormal, 2^0 * m/8; no infinities or NaNs."""
    s, e, m = (code >> 5) & 1, (code >> 3) & 3, code & 7
    v = 2.0 ** (e - 1) * (1 + m / 8) if e else m / 8
    return -v if s else v


# The FP6 operand holds q / U6_DIV, and the matrix instruction's block scale
# U6_DIV on each operand restores q.
U6_DIV = 8


def e2m3_code(q: int) -> int:
    """The E2M3 code of the INT4 code q: the code whose value is q / 8 (|q| <=
    8 here; the multiples of 1/8 up to 1 in magnitude are exact in E2M3, the
    ones below 1 as subnormals). Zero is +0."""
    if q == 0:
        return 0
    hits = [c for c in range(64) if e2m3_value(c) == q / U6_DIV]
    if len(hits) != 1:
        raise ValueError(f"{q} / {U6_DIV} is not exactly representable in E2M3")
    return hits[0]


U6_BLOCK = 1536    # bytes of one 32-row x 64-channel block of a u6 operand


def u6_chunk_images(q4, pitch4: int) -> np.ndarray:
    """The 192-bit image of every 32-channel chunk of every row: code i of
    chunk c (channel 32c + i, code 0 past K_n up to 2 * pitch4 channels) at
    bits 6i .. 6i+5, little-endian. Returns uint8 [rows, chunks, 24]."""
    q4 = np.asarray(q4, np.int8)
    rows, K_n = q4.shape
    C = 2 * pitch4 // 32                      # chunks per row
    table = np.array([e2m3_code(v) for v in range(-8, 8)], np.uint64)
    codes = np.zeros((rows, C * 32), np.uint64)
    codes[:, :K_n] = table[q4.astype(np.int64) + 8]
    codes = codes.reshape(rows, C, 32)
    words = np.zeros((rows, C, 3), np.uint64)
    for i in range(32):
        bit = 6 * i
        w, off = bit // 64, bit % 64
        words[:, :, w] |= (codes[:, :, i] << np.uint64(off)) & np.uint64(0xFFFFFFFFFFFFFFFF)
        if off > 58:                          # the code straddles two 64-bit words
            words[:, :, w + 1] |= codes[:, :, i] >> np.uint64(64 - off)
    return words.astype("<u8").view(np.uint8).reshape(rows, C, 24)


def pack_u6(q4, pitch4: int) -> np.ndarray:
    """INT4 codes [rows, K_n] -> the u6 operand of the FP6 GEMM (uint8).

    Rows go in blocks of 32 (rows past the last one are code 0) and channels
    in tiles of 64 (two 32-channel chunks, h = 0, 1); the block of row block
    b and tile t is 1536 bytes at (b * T + t) * 1536, T = pitch4 / 32. Inside
    it, row r's chunk h has image bytes 0..15 at 512 h + 16 r and image bytes
    16..23 at 1024 + 256 h + 8 r.
    """
    img = u6_chunk_images(q4, pitch4)
    rows = img.shape[0]
    RB, T = (rows + 31) // 32, pitch4 // 32
    out = np.zeros((RB, T, U6_BLOCK), np.uint8)
    for r in range(rows):
        b, rr = divmod(r, 32)
        for t in range(T):
            for h in range(2):
                c = img[r, 2 * t + h]
                out[b, t, 512 * h + 16 * rr:512 * h + 16 * rr + 16] = c[:16]
                out[b, t, 1024 + 256 * h + 8 * rr:1024 + 256 * h + 8 * rr + 8] = c[16:]
    return out.reshape(-1)


def unpack_u6(u6, rows: int, K_n: int) -> np.ndarray:
    """Inverse of pack_u6: the INT4 codes [rows, K_n] (U6_DIV times the values of the E2M3 codes)."""
    u6 = np.asarray(u6, np.uint8)
    pitch4 = (K_n + 127) // 128 * 64
    T = pitch4 // 32
    blocks = u6.reshape(-1, T, U6_BLOCK)
    out = np.zeros((rows, 2 * pitch4), np.int8)
    for r in range(rows):
        b, rr = divmod(r, 32)
        for t in range(T):
            for h in range(2):
                blk = blocks[b, t]
                img = bytes(blk[512 * h + 16 * rr:512 * h + 16 * rr + 16]) + \
                    bytes(blk[1024 + 256 * h + 8 * rr:1024 + 256 * h + 8 * rr + 8])
                bits = int.from_bytes(img, "little")
                for i in range(32):
                    out[r, 64 * t + 32 * h + i] = int(U6_DIV * e2m3_value((bits >> (6 * i)) & 63))
    return out[:, :K_n]


def linear_at(qa, qw, group: int, m_idx, n_idx):
    """Integer GEMM + fp64 dequant at output pairs (m_idx[p], n_idx[p]).

    qa / qw are the 4-tuples returned by quantize_rows for X and W.
    Returns (acc4 int32 [P, G], acc8 int32 [P], ystar float64 [P]).
    """
    qa4, sa4, qa8, sa8 = qa
    qw4, sw4, qw8, sw8 = qw
    K_n, n_out = qa4.shape[1], qa8.shape[1]
    G = num_groups(K_n, group)
    m_idx = np.ascontiguousarray(m_idx, np.int32)
    n_idx = np.ascontiguousarray(n_idx, np.int32)
    P = m_idx.size
    acc4 = np.zeros((P, G), np.int32)
    acc8 = np.zeros(P, np.int32)
    y = np.zeros(P, np.float64)
    pad = lambda a, dt: np.ascontiguousarray(a, dt) if a.size else np.zeros(1, dt)  # noqa: E731
    rc = _load().w4o_linear_at(pad(qa4, np.int8), pad(sa4, np.float32), pad(qa8, np.int8),
                               pad(sa8, np.float32), pad(qw4, np.int8), pad(sw4, np.float32),
                               pad(qw8, np.int8), pad(sw8, np.float32), K_n, n_out, group,
                               pad(m_idx, np.int32), pad(n_idx, np.int32), P,
                               pad(acc4, np.int32), pad(acc8, np.int32), pad(y, np.float64))
    if rc != 0:
        raise OverflowError("accumulator outside int32")
    return acc4, acc8, y


def linear_dense(qa, qw, group: int):
    """Integer GEMM + fp64 dequant at every output position (the same steps
    as linear_at, for whole-matrix checks).

    The group sums (step O6) are taken with a library float64 matrix product
    of the codes: every product and partial sum is an integer below 2^53, so
    the product is exact whatever order the library sums in. The dequant
    (O7) evaluates y* = sum_t (sa4 * sw4) * acc4_t + (sa8 * sw8) * acc8 in
    fp64 in the same order and association as linear_at.
    Returns (acc4 int32 [G, M, N], acc8 int32 [M, N], ystar float64 [M, N]).
    """
    qa4, sa4, qa8, sa8 = qa
    qw4, sw4, qw8, sw8 = qw
    M, K_n = qa4.shape
    N, n_out = qw4.shape[0], qa8.shape[1]
    G = num_groups(K_n, group)
    gl = group if group > 0 else K_n

    def exact_sums(a, b):
        s = np.asarray(a, np.float64) @ np.asarray(b, np.float64).T
        if s.size and (s.max() > 2**31 - 1 or s.min() < -2**31):
            raise OverflowError("accumulator outside int32")
        return s.astype(np.int32)

    acc4 = np.zeros((G, M, N), np.int32)
    y = np.zeros((M, N), np.float64)
    for t in range(G):
        acc4[t] = exact_sums(qa4[:, t * gl:(t + 1) * gl], qw4[:, t * gl:(t + 1) * gl])
        y += (np.asarray(sa4[:, t], np.float64)[:, None] * np.asarray(sw4[:, t], np.float64)[None, :]) * acc4[t]
    acc8 = exact_sums(qa8, qw8) if n_out else np.zeros((M, N), np.int32)
    y += (np.asarray(sa8, np.float64)[:, None] * np.asarray(sw8, np.float64)[None, :]) * acc8
    return acc4, acc8, y


def to_fp16(ystar) -> np.ndarray:
    """fp64 -> fp16, round to nearest even (numpy's direct double->half cast)."""
    return np.asarray(ystar, np.float64).astype(np.float16)


def linear(X, W, outlier_idx, group: int):
    """Whole layer on small inputs: every output position.

    Returns a dict with perm, the quantized operands, acc4 [G, M, N],
    acc8 [M, N], ystar [M, N] (fp64) and Y [M, N] (fp16).
    """
    X, W = np.asarray(X), np.asarray(W)
    M, K = X.shape
    N = W.shape[0]
    perm = make_perm(K, outlier_idx)
    n_out = int(np.asarray(outlier_idx).size)
    qa = quantize_rows(X, perm, n_out, group)
    qw = quantize_rows(W, perm, n_out, group)
    mm, nn = np.meshgrid(np.arange(M, dtype=np.int32), np.arange(N, dtype=np.int32),
                         indexing="ij")
    acc4, acc8, y = linear_at(qa, qw, group, mm.reshape(-1), nn.reshape(-1))
    G = acc4.shape[1]
    return {
        "perm": perm, "qa": qa, "qw": qw,
        "acc4": acc4.reshape(M, N, G).transpose(2, 0, 1).copy(),
        "acc8": acc8.reshape(M, N),
        "ystar": y.reshape(M, N),
        "Y": to_fp16(y.reshape(M, N)),
    }


def w4a8_quantize(X, W, group: int):
    """W4A8 operands (the QQQ abstract on the "smoothquant" tag page): per-token INT8 activations over all K
    channels and INT4 weights with one scale per output channel (group 0) or
    per `group` channels, both by the same symmetric quantizer (readings
    R1-R5), in the original channel order. Returns ((q8, s8), (q4, s4))."""
    X, W = np.asarray(X), np.asarray(W)
    K = X.shape[1]
    ident = np.arange(K, dtype=np.int32)
    _, _, qa8, sa8 = quantize_rows(X, ident, K, 0)
    qw4, sw4, _, _ = quantize_rows(W, ident, 0, group)
    return (qa8, sa8), (qw4, sw4)


def w4a8_linear_at(qa, qw, group: int, m_idx, n_idx):
    """W4A8 integer GEMM + fp64 dequant at output pairs (m_idx[p], n_idx[p]):
    acc int32 [P, G] and y* = sa8[m] * sum_t sw4[n, t] * acc[p, t] (fp64 [P])."""
    qa8, sa8 = qa
    qw4, sw4 = qw
    K = qa8.shape[1]
    G = num_groups(K, group)
    m_idx = np.ascontiguousarray(m_idx, np.int32)
    n_idx = np.ascontiguousarray(n_idx, np.int32)
    P = m_idx.size
    acc = np.zeros((P, G), np.int32)
    y = np.zeros(P, np.float64)
    pad = lambda a, dt: np.ascontiguousarray(a, dt) if a.size else np.zeros(1, dt)  # noqa: E731
    rc = _load().w4o_w4a8_linear_at(pad(qa8, np.int8), pad(sa8, np.float32), pad(qw4, np.int8),
                                    pad(sw4, np.float32), K, group, pad(m_idx, np.int32),
                                    pad(n_idx, np.int32), P, pad(acc, np.int32), pad(y, np.float64))
    if rc != 0:
        raise OverflowError("accumulator outside int32")
    return acc, y


def w4a8_linear(X, W, group: int):
    """Whole W4A8 layer on small inputs: acc [G, M, N], ystar [M, N], Y fp16."""
    X, W = np.asarray(X), np.asarray(W)
    M, N = X.shape[0], W.shape[0]
    qa, qw = w4a8_quantize(X, W, group)
    mm, nn = np.meshgrid(np.arange(M, dtype=np.int32), np.arange(N, dtype=np.int32), indexing="ij")
    acc, y = w4a8_linear_at(qa, qw, group, mm.reshape(-1), nn.reshape(-1))
    G = acc.shape[1]
    return {"qa": qa, "qw": qw, "acc": acc.reshape(M, N, G).transpose(2, 0, 1).copy(),
            "ystar": y.reshape(M, N), "Y": to_fp16(y.reshape(M, N))}


def kv_quantize(X, bits: int):
    """Low-bit KV cache (reading V1): every (token, head) vector of X [T, H, D]
    (fp16) is one block of the symmetric quantizer (readings R1-R5), INT4
    (qmax 7) or INT8 (qmax 127). Atom summary page, Summary paragraph 2: the
    KV cache is stored in low bit-width. Returns (codes int8 [T, H, D],
    scales fp32 [T, H])."""
    X = np.asarray(X)
    T, H, D = X.shape
    rows = np.ascontiguousarray(X.reshape(T * H, D))
    ident = np.arange(D, dtype=np.int32)
    if bits == 4:
        q, s, _, _ = quantize_rows(rows, ident, 0, 0)
        return q.reshape(T, H, D), s.reshape(T, H)
    if bits == 8:
        _, _, q, s = quantize_rows(rows, ident, D, 0)
        return q.reshape(T, H, D), s.reshape(T, H)
    raise ValueError("bits must be 4 or 8")


def kv_dequantize(q, s) -> np.ndarray:
    """fp16(fl32(s * q)) for codes q [T, H, D] and scales s [T, H] (reading
    V2): one correctly rounded fp32 product, then round to nearest even."""
    prod = np.asarray(s, np.float32)[..., None] * np.asarray(q, np.int8).astype(np.float32)
    return prod.astype(np.float16)


def kv_pack(q, bits: int) -> np.ndarray:
    """Cache bytes of codes q [T, H, D]: INT4 two per byte, low nibble first
    (the layer's packing); INT8 one per byte. uint8 [T, H, D * bits / 8]."""
    T, H, D = q.shape
    if bits == 8:
        return np.ascontiguousarray(q, np.int8).view(np.uint8)
    return pack_nibbles(q.reshape(T * H, D), D // 2).reshape(T, H, D // 2)
