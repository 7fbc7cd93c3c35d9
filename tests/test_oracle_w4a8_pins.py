"""Pins for the oracle's W4A8 layer (the QQQ abstract on the "smoothquant" tag page: 4-bit weights with 8-bit
activations, per-channel and per-group GEMMs).

Definition: activations get one INT8 scale per token over all K channels,
weights INT4 scales per output channel (group 0) or per `group` channels, by
the same symmetric round-to-nearest quantizer as the W4A4 layer (readings
R1-R5); acc_t = sum over group t of qa8 * qw4 (exact), y* = sa8[m] *
sum_t sw4[n, t] * acc_t in fp64, Y = fp16(y*).

Pins: a float64 matmul of the codes (exact below 2^53), a lossless grid that
reduces the layer to numpy's X W^T, the closed-form error bound against the
real product, sign / power-of-two / in-group permutation invariances and a
Fraction brute force on tiny shapes.
"""
from fractions import Fraction

import numpy as np
import pytest


def _data(seed, M, N, K, w_std=0.02):
    rng = np.random.default_rng(seed)
    X = (rng.standard_normal((M, K)) * rng.choice([1, 1, 30], K)).astype(np.float16)
    W = (rng.standard_normal((N, K)) * w_std).astype(np.float16)
    return X, W


@pytest.mark.parametrize("group", [0, 64, 128])
def test_integer_sums_equal_a_library_matmul(oracle, group):
    X, W = _data(1, 9, 11, 256)
    r = oracle.w4a8_linear(X, W, group)
    (qa8, _), (qw4, _) = r["qa"], r["qw"]
    G = r["acc"].shape[0]
    gl = group or 256
    for t in range(G):
        ref = qa8[:, t * gl:(t + 1) * gl].astype(np.float64) @ qw4[:, t * gl:(t + 1) * gl].astype(np.float64).T
        assert np.array_equal(r["acc"][t].astype(np.float64), ref)


@pytest.mark.parametrize("group", [0, 32])
def test_lossless_grid_reduces_to_matmul(oracle, group):
    """X rows c * 2^e (c in [-127, 127], +-127 present) and W groups c' * 2^e'
    (c' in [-7, 7], +-7 in each group): every scale is a power of two, the
    codes are c and c', and Y = fp16(X W^T) exactly."""
    rng = np.random.default_rng(2)
    M, N, K = 6, 7, 128
    ex = rng.integers(-6, 0, M)
    cx = rng.integers(-127, 128, (M, K))
    cx[:, 0] = 127
    X = (cx * 2.0 ** ex[:, None]).astype(np.float16)
    gl = group or K
    cw = rng.integers(-7, 8, (N, K))
    cw[:, ::gl] = -7
    ew = rng.integers(-9, -4, (N, K // gl))
    W = (cw * np.repeat(2.0 ** ew, gl, axis=1)).astype(np.float16)
    assert np.array_equal(X.astype(np.float64), cx * 2.0 ** ex[:, None])
    r = oracle.w4a8_linear(X, W, group)
    assert np.array_equal(r["qa"][0], cx.astype(np.int8))
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    assert np.array_equal(r["Y"], exact.astype(np.float16))


@pytest.mark.parametrize("group", [0, 128])
def test_error_bound_against_the_real_product(oracle, group):
    X, W = _data(3, 8, 10, 512)
    r = oracle.w4a8_linear(X, W, group)
    (_, sa8), (_, sw4) = r["qa"], r["qw"]
    gl = group or 512
    ex = sa8.astype(np.float64) * (0.5 + 127 * 2.0 ** -24)
    ew = np.repeat(sw4.astype(np.float64), gl, axis=1) * (0.5 + 7 * 2.0 ** -24)
    Xd, Wd = X.astype(np.float64), W.astype(np.float64)
    bound = (np.abs(Xd) @ ew.T + ex[:, None] * np.abs(Wd).sum(axis=1)[None, :] + ex[:, None] * ew.sum(axis=1)[None, :])
    assert np.all(np.abs(r["ystar"] - Xd @ Wd.T) <= bound * (1 + 1e-12) + 1e-300)


def test_sign_and_power_of_two(oracle):
    X, W = _data(4, 5, 6, 256)
    X = np.where(np.abs(X) < 2.0 ** -8, np.float16(2.0 ** -8), X)
    r = oracle.w4a8_linear(X, W, 128)
    assert np.array_equal(oracle.w4a8_linear(-X, W, 128)["ystar"], -r["ystar"])
    Xs = (X.astype(np.float32) * 4).astype(np.float16)
    r2 = oracle.w4a8_linear(Xs, W, 128)
    assert np.array_equal(r2["acc"], r["acc"])
    assert np.array_equal(r2["ystar"], r["ystar"] * 4)


@pytest.mark.parametrize("group", [0, 64])
def test_permutation_inside_groups(oracle, group):
    """The same permutation of channels inside every group (any permutation of
    all channels with per-channel scales), on X and W together."""
    X, W = _data(5, 4, 5, 256)
    gl = group or 256
    rng = np.random.default_rng(6)
    p = np.concatenate([t * gl + rng.permutation(gl) for t in range(256 // gl)])
    a, b = oracle.w4a8_linear(X, W, group), oracle.w4a8_linear(X[:, p], W[:, p], group)
    assert np.array_equal(a["acc"], b["acc"]) and np.array_equal(a["ystar"], b["ystar"])


def test_fraction_brute_force(oracle):
    X, W = _data(7, 3, 4, 32)
    r = oracle.w4a8_linear(X, W, 16)
    (qa8, sa8), (qw4, sw4) = r["qa"], r["qw"]
    for m in range(3):
        for n in range(4):
            tot = Fraction(0)
            for t in range(2):
                acc = sum(int(qa8[m, j]) * int(qw4[n, j]) for j in range(16 * t, 16 * t + 16))
                assert acc == r["acc"][t, m, n]
                tot += Fraction(float(sw4[n, t])) * acc
            want = Fraction(float(sa8[m])) * tot
            assert abs(Fraction(r["ystar"][m, n]) - want) <= abs(want) * Fraction(1, 2 ** 50)
