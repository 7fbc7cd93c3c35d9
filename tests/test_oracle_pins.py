"""Pins for the CPU oracle: facts that do not come from the oracle itself.

Each test checks the oracle against something fixed by the pages or by
mathematics: a hand-worked fixture, a brute-force search on tiny inputs, a
closed-form error bound, a special case that reduces to a textbook matmul, or
an invariance of the definition. Together they are chosen so that a plausible
slip (a dropped tail term, a wrong rounding rule, a wrong qmax, a swapped
index, a transposed operand, a lost sign) fails at least one of them.

Definitions followed: Atom summary page (Summary paragraph 2, Key points item
5, Interesting ideas I1 and I3) and the QUIK abstract.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


# ---------------------------------------------------------------------------
# hand-worked fixture
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_hand_worked_fixture(oracle, case):
    X = np.array(case["X"], np.float16)
    W = np.array(case["W"], np.float16)
    g = case["group"]
    out = oracle.linear(X, W, case["outlier_idx"], g)
    assert out["perm"].tolist() == case["perm"]
    qa4, sa4, qa8, sa8 = out["qa"]
    qw4, sw4, qw8, sw8 = out["qw"]
    assert qa4.tolist() == case["qa4"] and qa8.tolist() == case["qa8"]
    assert sa4.tolist() == case["sa4"] and sa8.tolist() == case["sa8"]
    assert qw4.tolist() == case["qw4"] and qw8.tolist() == case["qw8"]
    assert sw4.tolist() == case["sw4"] and sw8.tolist() == case["sw8"]
    pitch = qa4.shape[1] // 2
    assert oracle.pack_nibbles(qa4, pitch).tolist() == case["qa4_packed"]
    assert out["acc4"].tolist() == case["acc4"]
    assert out["acc8"].tolist() == case["acc8"]
    assert out["ystar"].tolist() == case["ystar"]
    assert out["Y"].astype(np.float64).tolist() == case["Y_fp16"]


# ---------------------------------------------------------------------------
# permutation (Atom, Interesting ideas I1: outliers to a contiguous tail)
# ---------------------------------------------------------------------------
@settings(max_examples=60, deadline=None)
@given(st.integers(1, 70).flatmap(
    lambda K: st.tuples(st.just(K), st.lists(st.integers(0, K - 1), unique=True, max_size=K))))
def test_make_perm_properties(oracle, args):
    K, outl = args
    perm = oracle.make_perm(K, np.array(outl, np.int32))
    n = len(outl)
    assert sorted(perm.tolist()) == list(range(K))               # a permutation
    assert perm[K - n:].tolist() == sorted(outl)                  # tail = outliers
    head = perm[:K - n].tolist()
    assert head == sorted(head) and not set(head) & set(outl)     # stable head


@pytest.mark.parametrize("bad", [[3, 3], [-1], [8]])
def test_make_perm_rejects(oracle, bad):
    with pytest.raises(ValueError):
        oracle.make_perm(8, np.array(bad, np.int32))


# ---------------------------------------------------------------------------
# one quantized block: brute force over all candidate codes
# ---------------------------------------------------------------------------
def _brute_block(v, qmax):
    """Absmax by enumeration; code = candidate nearest to fl32(x/s), ties even."""
    v = [np.float32(x) for x in v]
    a = max([abs(float(x)) for x in v] + [0.0])
    s = np.float32(Fraction(a) / qmax)  # nearest fp32 to the exact quotient
    # np.float32(Fraction) goes through float(): a / qmax in fp64 is exact or
    # correctly rounded, and double rounding to fp32 is innocuous (53 >= 2*24+2)
    if s == 0:
        return [0] * len(v), s
    codes = []
    for x in v:
        d = Fraction(float(np.float32(float(x) / float(s))))  # fl32(x/s), same argument
        best = None
        for c in range(-qmax - 1, qmax + 1):
            key = (abs(d - c), c % 2)
            if best is None or key < best[0]:
                best = (key, c)
        # clamp: the best in-range candidate is the clamped rint when |d| is large
        codes.append(best[1])
    return codes, s


fp16_values = st.floats(-65504, 65504, allow_nan=False, width=16)


@settings(max_examples=300, deadline=None)
@given(st.lists(fp16_values, min_size=1, max_size=12), st.sampled_from([7, 127]))
def test_quantize_block_brute_force(oracle, vals, qmax):
    q, s = oracle.quantize_block(np.array(vals, np.float16), qmax)
    bq, bs = _brute_block(np.array(vals, np.float16), qmax)
    assert s == bs
    assert q.tolist() == bq


def test_quantize_block_ties_and_zero(oracle):
    # scale 1 (absmax 7): exact halves must go to the even neighbour
    q, s = oracle.quantize_block(np.array([7, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5], np.float32), 7)
    assert s == 1.0 and q.tolist() == [7, 0, 2, 2, 0, -2, -2, 4]
    q, s = oracle.quantize_block(np.zeros(5, np.float32), 7)
    assert s == 0.0 and q.tolist() == [0] * 5


# ---------------------------------------------------------------------------
# whole-row quantization: bounds and the absmax element
# ---------------------------------------------------------------------------
def _check_bound(x, q, s, qmax):
    s64 = np.float64(s)
    err = np.abs(x.astype(np.float64) - s64 * q.astype(np.float64))
    # |x - s q| <= s/2 plus the fp32 division error of x/s (|x/s| <= qmax+1)
    assert np.all(err <= s64 * (0.5 + (qmax + 1) * 2.0 ** -23) + 1e-300)


@pytest.mark.parametrize("group", [0, 16, 32])
def test_quantize_rows_error_bound_and_absmax(oracle, group):
    rng = np.random.default_rng(11)
    K, n_out, rows = 96, 32 if group != 16 else 16, 40
    X = rng.standard_normal((rows, K)).astype(np.float16)
    O = rng.choice(K, n_out, replace=False)
    X[:, O] *= np.float16(40)
    perm = oracle.make_perm(K, O)
    q4, s4, q8, s8 = oracle.quantize_rows(X, perm, n_out, group)
    Xr = X[:, perm].astype(np.float32)
    K_n = K - n_out
    gl = group or K_n
    for r in range(rows):
        for t in range(K_n // gl):
            blk = Xr[r, t * gl:(t + 1) * gl]
            qb = q4[r, t * gl:(t + 1) * gl]
            _check_bound(blk, qb, s4[r, t], 7)
            i = int(np.argmax(np.abs(blk)))
            assert abs(int(qb[i])) == 7 and np.sign(qb[i]) == np.sign(blk[i])
            assert qb.min() >= -7 and qb.max() <= 7
        _check_bound(Xr[r, K_n:], q8[r], s8[r], 127)
        assert abs(int(q8[r][np.argmax(np.abs(Xr[r, K_n:]))])) == 127


# ---------------------------------------------------------------------------
# lossless grid: the quantized layer reduces to a textbook matmul
# ---------------------------------------------------------------------------
def _grid_operand(rng, rows, K, perm, n_out, group, e):
    """Values c * 2^e with integer c; each block (in reordered order) holds +-7
    (INT4) or +-127 (tail), so s = 2^e exactly and the codes equal c."""
    K_n = K - n_out
    gl = group or K_n
    R = np.zeros((rows, K), np.float64)
    R[:, :K_n] = rng.integers(-7, 8, (rows, K_n))
    R[:, K_n:] = rng.integers(-127, 128, (rows, n_out))
    for r in range(rows):
        for t in range(K_n // gl if K_n else 0):
            R[r, t * gl + rng.integers(gl)] = rng.choice([-7, 7])
        if n_out:
            R[r, K_n + rng.integers(n_out)] = rng.choice([-127, 127])
    X = np.zeros_like(R)
    X[:, perm] = R
    return X * 2.0 ** e, R


@pytest.mark.parametrize("M,N,K,n_out,group", [(5, 7, 48, 8, 0), (3, 9, 72, 8, 16),
                                               (4, 6, 40, 0, 0), (6, 5, 64, 64, 0)])
def test_lossless_grid_reduces_to_matmul(oracle, M, N, K, n_out, group):
    rng = np.random.default_rng(M * 100 + K)
    O = rng.choice(K, n_out, replace=False)
    perm = oracle.make_perm(K, O)
    X, RX = _grid_operand(rng, M, K, perm, n_out, group, -3)
    W, RW = _grid_operand(rng, N, K, perm, n_out, group, -6)
    out = oracle.linear(X.astype(np.float16), W.astype(np.float16), O, group)
    K_n = K - n_out
    assert np.array_equal(out["qa"][0], RX[:, :K_n]) and np.array_equal(out["qa"][2], RX[:, K_n:])
    assert np.all(out["qa"][1] == 2.0 ** -3) and np.all(out["qw"][1] == 2.0 ** -6)
    exact = X @ W.T                                  # textbook matmul, exact here
    assert np.array_equal(out["ystar"], exact)
    assert np.array_equal(out["Y"], exact.astype(np.float16))


# ---------------------------------------------------------------------------
# integer GEMM: equals a float64 library matmul of the codes (exact here)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("group", [0, 8, 24])
def test_int_gemm_equals_library_matmul(oracle, group):
    rng = np.random.default_rng(5 + group)
    M, N, K, n_out = 7, 11, 72, 24
    X = rng.standard_normal((M, K)).astype(np.float16)
    W = rng.standard_normal((N, K)).astype(np.float16)
    O = rng.choice(K, n_out, replace=False)
    out = oracle.linear(X, W, O, group)
    qa4, _, qa8, _ = out["qa"]
    qw4, _, qw8, _ = out["qw"]
    gl = group or (K - n_out)
    for t in range(out["acc4"].shape[0]):
        ref = qa4[:, t * gl:(t + 1) * gl].astype(np.float64) @ qw4[:, t * gl:(t + 1) * gl].T.astype(np.float64)
        assert np.array_equal(out["acc4"][t], ref.astype(np.int64))
    assert np.array_equal(out["acc8"], (qa8.astype(np.float64) @ qw8.T.astype(np.float64)).astype(np.int64))


@pytest.mark.parametrize("M,N,K,n_out,group", [(9, 13, 96, 16, 16), (7, 5, 64, 0, 0), (6, 10, 40, 40, 0),
                                               (12, 8, 200, 8, 48), (3, 4, 130, 2, 0)])
def test_linear_dense_equals_linear_at(oracle, M, N, K, n_out, group):
    """The whole-matrix form of the GEMM and dequant agrees with the C oracle's
    per-position loops bit for bit: accumulators and fp64 y*."""
    rng = np.random.default_rng(M * N + K + group)
    X = (rng.standard_normal((M, K)) * rng.choice([1.0, 30.0], K)).astype(np.float16)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    O = rng.choice(K, n_out, replace=False)
    ref = oracle.linear(X, W, O, group)
    acc4, acc8, ystar = oracle.linear_dense(ref["qa"], ref["qw"], group)
    assert np.array_equal(acc4, ref["acc4"])
    assert np.array_equal(acc8, ref["acc8"])
    assert np.array_equal(ystar, ref["ystar"])


def test_all_outliers_is_w8a8(oracle):
    rng = np.random.default_rng(3)
    M, N, K = 4, 5, 32
    X = rng.standard_normal((M, K)).astype(np.float16)
    W = rng.standard_normal((N, K)).astype(np.float16)
    out = oracle.linear(X, W, np.arange(K), 0)
    assert out["acc4"].shape[0] == 0
    qa8, sa8, qw8, sw8 = out["qa"][2], out["qa"][3], out["qw"][2], out["qw"][3]
    ref = (qa8.astype(np.float64) @ qw8.T.astype(np.float64))
    assert np.array_equal(out["acc8"], ref.astype(np.int64))
    assert np.allclose(out["ystar"], sa8[:, None].astype(np.float64) * sw8[None, :] * ref, rtol=1e-15)


# ---------------------------------------------------------------------------
# closed-form error bound against the exact product X W^T
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("group", [0, 32])
def test_output_error_bound(oracle, group):
    rng = np.random.default_rng(21)
    M, N, K, n_out = 6, 8, 160, 32
    X = rng.standard_normal((M, K)).astype(np.float16)
    O = rng.choice(K, n_out, replace=False)
    X[:, O] *= np.float16(50)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    out = oracle.linear(X, W, O, group)
    perm = out["perm"]
    K_n = K - n_out
    gl = group or K_n
    slack = 0.5 + 128 * 2.0 ** -23

    def eps(q):  # per element half-step bound in reordered order
        s4, s8 = q[1], q[3]
        e = np.zeros((s4.shape[0], K))
        for t in range(s4.shape[1]):
            e[:, t * gl:(t + 1) * gl] = s4[:, t:t + 1] * slack
        e[:, K_n:] = s8[:, None] * slack
        return e

    ex, ew = eps(out["qa"]), eps(out["qw"])
    Xr = np.abs(X[:, perm].astype(np.float64))
    Wr = np.abs(W[:, perm].astype(np.float64))
    bound = Xr @ ew.T + ex @ Wr.T + ex @ ew.T
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    assert np.all(np.abs(out["ystar"] - exact) <= bound * (1 + 1e-12))


# ---------------------------------------------------------------------------
# invariances of the definition
# ---------------------------------------------------------------------------
def _case(seed, M=5, N=6, K=64, n_out=16):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K)).astype(np.float16)
    O = rng.choice(K, n_out, replace=False)
    X[:, O] *= np.float16(30)
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float16)
    return rng, X, W, O


def test_joint_channel_relabel_invariance_per_row(oracle):
    rng, X, W, O = _case(1)
    K = X.shape[1]
    base = oracle.linear(X, W, O, 0)
    sigma = rng.permutation(K)                 # new channel c holds old channel sigma[c]
    inv = np.argsort(sigma)
    moved = oracle.linear(X[:, sigma], W[:, sigma], inv[O], 0)
    assert np.array_equal(base["ystar"], moved["ystar"])
    assert np.array_equal(base["acc8"], moved["acc8"])


def test_within_group_permutation_invariance(oracle):
    rng, X, W, O = _case(2)
    g = 16
    base = oracle.linear(X, W, O, g)
    perm = base["perm"]
    K, n_out = X.shape[1], len(O)
    # shuffle inside each reordered group and inside the tail, then express the
    # new order as a relabelling of the original channels
    newr = []
    for t in range((K - n_out) // g):
        newr += list(rng.permutation(perm[t * g:(t + 1) * g]))
    newr += list(rng.permutation(perm[K - n_out:]))
    newr = np.array(newr)
    # channel c of the relabelled problem is old channel newr-order: build X' so
    # that the stable reorder of X' reproduces the shuffled order
    sigma = np.empty(K, np.int64)
    head, tail = sorted(range(K - n_out)), list(range(K - n_out, K))
    sigma[head] = newr[:K - n_out]
    sigma[tail] = newr[K - n_out:]
    moved = oracle.linear(X[:, sigma], W[:, sigma], np.arange(K - n_out, K), g)
    assert np.array_equal(base["acc4"], moved["acc4"])
    assert np.allclose(base["ystar"], moved["ystar"], rtol=1e-15, atol=0)


@pytest.mark.parametrize("group", [0, 16])
def test_sign_symmetry(oracle, group):
    _, X, W, O = _case(3)
    a = oracle.linear(X, W, O, group)
    b = oracle.linear(-X, W, O, group)
    assert np.array_equal(a["ystar"], -b["ystar"])
    assert np.array_equal(a["Y"], -b["Y"])


@pytest.mark.parametrize("group", [0, 16])
def test_power_of_two_scaling(oracle, group):
    _, X, W, O = _case(4)
    a = oracle.linear(X, W, O, group)
    b = oracle.linear((X.astype(np.float32) * 4).astype(np.float16), W, O, group)
    assert np.array_equal(a["qa"][0], b["qa"][0]) and np.array_equal(a["qa"][2], b["qa"][2])
    assert np.array_equal(a["qa"][1] * 4, b["qa"][1])
    assert np.array_equal(a["ystar"] * 4, b["ystar"])


# ---------------------------------------------------------------------------
# packing and the final fp16 rounding
# ---------------------------------------------------------------------------
@settings(max_examples=50, deadline=None)
@given(st.lists(st.integers(-8, 7), min_size=1, max_size=40), st.integers(0, 3))
def test_pack_round_trip(oracle, codes, extra):
    q = np.array([codes], np.int8)
    pitch = (len(codes) + 1) // 2 + extra
    p = oracle.pack_nibbles(q, pitch)
    lo = (p[0].astype(np.int16) & 15)
    hi = (p[0].astype(np.int16) >> 4) & 15
    un = np.stack([lo, hi], 1).reshape(-1)
    un = np.where(un >= 8, un - 16, un)
    assert un[:len(codes)].tolist() == codes
    assert not un[len(codes):].any()             # zero padding


def test_pack_known_bytes(oracle):
    p = oracle.pack_nibbles(np.array([[-8, 7, 1, -1, 0, -8]], np.int8), 4)
    assert p.tolist() == [[0x78, 0xF1, 0x80, 0x00]]


def test_fp64_to_fp16_rounding_is_nearest_even(oracle):
    rng = np.random.default_rng(0)
    h = rng.integers(0, 0x7BFF, 4000, dtype=np.uint16).view(np.float16)
    lo = h.astype(np.float64)
    hi = np.nextafter(h, np.float16(np.inf)).astype(np.float64)
    mid = (lo + hi) / 2                               # exact in fp64
    got = oracle.to_fp16(mid)
    even = np.where((h.view(np.uint16) & 1) == 0, h, np.nextafter(h, np.float16(np.inf)))
    assert np.array_equal(got, even)
    # just above / below the midpoint
    assert np.array_equal(oracle.to_fp16(np.nextafter(mid, np.inf)),
                          np.nextafter(h, np.float16(np.inf)))
    assert np.array_equal(oracle.to_fp16(np.nextafter(mid, -np.inf)), h)


# ---------------------------------------------------------------------------
# FP6 (E2M3) packing of INT4 codes for the prefill GEMM
# ---------------------------------------------------------------------------
E2M3 = os.path.join(os.path.dirname(__file__), "golden", "e2m3_int4.json")


def test_e2m3_codes_match_hand_derived(oracle):
    want = json.load(open(E2M3))["codes"]
    for q, code in want.items():
        assert oracle.e2m3_code(int(q)) == code, q
        assert oracle.e2m3_value(code) == int(q) / 8


def test_e2m3_value_closed_forms(oracle):
    assert oracle.e2m3_value(0b011111) == 7.5           # the largest finite value: 2^2 * 1.875
    assert oracle.e2m3_value(0b011000) == 4.0           # 2^2
    assert oracle.e2m3_value(0b000001) == 1 / 8         # the smallest subnormal
    assert oracle.e2m3_value(0b000111) == 7 / 8         # the largest subnormal
    assert oracle.e2m3_value(0b001000) == 1.0           # the smallest normal: -8 / 8 in magnitude
    assert oracle.e2m3_value(0b100000) == 0.0           # -0
    assert oracle.e2m3_value(0b110100) == -3.0          # -2^1 * 1.5
    vals = sorted(oracle.e2m3_value(c) for c in range(32))
    assert len(set(vals)) == 32 and vals[0] == 0.0      # 32 distinct non-negative values
    # the values are the multiples of 1/8 up to 1, of 1/4 up to 4 and of 1/2 up to 7.5
    assert vals == [i / 8 for i in range(8)] + [1 + i / 8 for i in range(8)] + \
        [2 + i / 4 for i in range(8)] + [4 + i / 2 for i in range(8)]


def test_pack_u6_bit_positions(oracle):
    """Code i of a row's chunk (32 channels) sits at bits 6i of the chunk's
    192-bit image; image bytes 0..15 and 16..23 sit where the block layout
    puts them; channels past K_n and rows past the last are code 0."""
    rng = np.random.default_rng(7)
    rows, K_n, pitch4 = 40, 200, 128                   # 2 row blocks, 4 tiles of 64 channels
    q = rng.integers(-8, 8, (rows, K_n), dtype=np.int8)
    u6 = oracle.pack_u6(q, pitch4)
    assert u6.shape == (2 * 4 * 1536,)
    blk = u6.reshape(2, 4, 1536)
    for r in range(64):
        b, rr = divmod(r, 32)
        for c in range(8):
            t, h = divmod(c, 2)
            img = bytes(blk[b, t, 512 * h + 16 * rr:512 * h + 16 * rr + 16]) + \
                bytes(blk[b, t, 1024 + 256 * h + 8 * rr:1024 + 256 * h + 8 * rr + 8])
            bits = int.from_bytes(img, "little")
            for i in range(32):
                j = 32 * c + i
                want = oracle.e2m3_code(int(q[r, j])) if r < rows and j < K_n else 0
                assert (bits >> (6 * i)) & 63 == want


def test_pack_u6_round_trip(oracle):
    rng = np.random.default_rng(8)
    q = rng.integers(-8, 8, (37, 100), dtype=np.int8)
    u6 = oracle.pack_u6(q, 64)
    assert np.array_equal(oracle.unpack_u6(u6, 37, 100), q)


def test_pack_u6_known_bytes(oracle):
    """One chunk by hand: q = [1, -1, 7, -8, 0, ...] in row 0: the E2M3 codes
    of 1/8, -1/8, 7/8, -1 are 1, 33, 7, 40, at bits 0, 6, 12, 18 ->
    1 | 33 << 6 | 7 << 12 | 40 << 18 = 0xA07841, the first bytes of block (0, 0)."""
    q = np.zeros((1, 32), np.int8)
    q[0, :4] = [1, -1, 7, -8]
    u6 = oracle.pack_u6(q, 64)
    assert u6.size == 2 * 1536
    assert u6[:4].tolist() == [0x41, 0x78, 0xA0, 0x00]
    assert not u6[4:].any()
