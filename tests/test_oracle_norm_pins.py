"""Pins for the oracle's RMSNorm in front of the quantizer (readings N1-N3).

The fused producer normalizes each token row before it quantizes it:
rstd = fl32(1 / sqrt(fl64(fl64(S) / K) + eps)) with S the exact sum of
squares, then y = fl16(gamma * fl16(fl32(x * rstd))). Nothing here trusts
the oracle: the tests check closed forms where every step is exact, a
high-precision value of 1 / sqrt(mean + eps), rows built so that a rounded
running sum would give another rstd, invariances of the definition, and
torch's own fp16 arithmetic for the two roundings of the output.

Sources: the Atom summary page (Summary paragraph 2: quantization fused into
the operators around the GEMM; Interesting ideas I2) and the standard RMSNorm
of the Llama models the pages evaluate.
"""
import decimal
import math
from fractions import Fraction

import numpy as np
import pytest


def _ulp32(v: float) -> float:
    v = abs(float(v))
    return float(np.spacing(np.float32(v)))


def _true_rstd(row16, eps: float) -> Fraction:
    """1 / sqrt(mean(x^2) + eps) to 40 significant digits (decimal module)."""
    S = sum(Fraction(float(x)) ** 2 for x in row16)
    v = S / len(row16) + Fraction(float(np.float32(eps)))
    with decimal.localcontext() as ctx:
        ctx.prec = 40
        d = decimal.Decimal(v.numerator) / decimal.Decimal(v.denominator)
        r = decimal.Decimal(1) / d.sqrt()
        return Fraction(r)


# ---------------------------------------------------------------------------
# closed forms: every step exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("K", [1, 3, 7, 64, 4096])
@pytest.mark.parametrize("e", [-10, -3, 0, 4, 7])
def test_constant_magnitude_row(oracle, K, e):
    """|x| = 2^e everywhere, eps = 0: mean square 4^e, rstd = 2^-e exactly."""
    rng = np.random.default_rng(K * 31 + e)
    x = (rng.choice([-1.0, 1.0], size=(2, K)) * 2.0 ** e).astype(np.float16)
    r = oracle.rms_rstd(x, 0.0)
    assert np.all(r == np.float32(2.0 ** -e))


def test_eps_enters_under_the_root(oracle):
    """All ones with eps = 3: mean 1, 1 + 3 = 4, rstd = 1/2. A missing eps,
    square root, reciprocal or mean gives 1, 1/4, 2 or 1/(2 sqrt K)."""
    x = np.ones((3, 40), np.float16)
    assert np.all(oracle.rms_rstd(x, 3.0) == np.float32(0.5))
    assert np.all(oracle.rms_rstd(np.zeros((1, 8), np.float16), 0.25) == np.float32(2.0))


def test_zero_row_without_eps_is_zero(oracle):
    """Reading N3: mean square + eps == 0 gives rstd = 0 (and zero outputs)."""
    x = np.zeros((2, 16), np.float16)
    assert np.all(oracle.rms_rstd(x, 0.0) == 0)
    y = oracle.rmsnorm(x, np.ones(16, np.float16), 0.0)
    assert np.all(y == 0) and not np.any(np.isnan(y))


@pytest.mark.parametrize("j", [0, 2, 6])
def test_single_nonzero_at_every_position(oracle, j):
    """K = 4^j, one entry 2^e, the rest 0, eps = 0: rstd = 2^(j - e) exactly,
    wherever the entry sits (a skipped first, last or middle term fails)."""
    K = 4 ** j
    e = 3
    for p in sorted({0, K // 2, K - 1}):
        x = np.zeros((1, K), np.float16)
        x[0, p] = -(2.0 ** e)
        assert oracle.rms_rstd(x, 0.0)[0] == np.float32(2.0 ** (j - e)), p


# ---------------------------------------------------------------------------
# high precision and exact summation
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("K,eps", [(16, 1e-6), (300, 1e-5), (4096, 1e-6), (4096, 0.0)])
def test_rstd_is_within_half_ulp_plus_rounding(oracle, K, eps):
    """rstd is the fp32 value nearest to 1/sqrt(mean + eps) up to the binary64
    steps: |rstd - true| <= ulp32 * (1/2 + 2^-20)."""
    rng = np.random.default_rng(K)
    x = rng.standard_normal((6, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 32), replace=False)] *= 30
    x = x.astype(np.float16)
    r = oracle.rms_rstd(x, eps)
    for i in range(x.shape[0]):
        t = _true_rstd(x[i], eps)
        assert abs(Fraction(float(r[i])) - t) <= Fraction(_ulp32(float(t))) * (Fraction(1, 2) + Fraction(1, 2 ** 20))


def test_sum_is_exact_not_a_running_fp32_sum(oracle):
    """One 2^10 entry (square 2^20) and 4095 entries 2^-6 (square 2^-12): an
    fp32 running sum loses the small squares (ulp of 2^20 is 2^-3) and its
    rstd is several ulps off; the exact sum is 2^20 + 4095 * 2^-12."""
    K = 4096
    x = np.full((2, K), 2.0 ** -6, np.float16)
    x[0, 0] = 2.0 ** 10
    x[1, K - 1] = -(2.0 ** 10)
    r = oracle.rms_rstd(x, 0.0)
    for i in range(2):
        t = _true_rstd(x[i], 0.0)
        assert abs(Fraction(float(r[i])) - t) <= Fraction(_ulp32(float(t))) / 2 * (1 + Fraction(1, 2 ** 20))
    # the test can tell: a running fp32 sum (cumsum is sequential) of row 0
    # gives an rstd more than an ulp away
    run = np.cumsum((x[0].astype(np.float32)) ** 2, dtype=np.float32)[-1]
    naive = np.float32(1.0 / math.sqrt(float(run) / K))
    assert abs(float(naive) - float(r[0])) > _ulp32(float(r[0]))


def test_order_of_channels_does_not_matter(oracle):
    """Exact S: any permutation of a row's entries gives the same rstd bits."""
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((8, 1000)) * rng.choice([1, 30, 300], size=(8, 1000))).astype(np.float16)
    r0 = oracle.rms_rstd(x, 1e-6)
    for s in range(3):
        p = np.random.default_rng(s).permutation(1000)
        assert np.array_equal(oracle.rms_rstd(np.ascontiguousarray(x[:, p]), 1e-6), r0)


def test_brute_force_tiny_rows(oracle):
    """Tiny rows by the definition in Python: exact Fraction sum, Python's
    correctly rounded float(), /, + and math.sqrt, then the fp32 cast."""
    rng = np.random.default_rng(5)
    for K in (1, 2, 5, 9, 16):
        x = (rng.standard_normal((20, K)) * rng.choice([2.0 ** -12, 1.0, 200.0], size=(20, K))).astype(np.float16)
        for eps in (0.0, 1e-6, 0.5):
            r = oracle.rms_rstd(x, eps)
            for i in range(x.shape[0]):
                S = sum(Fraction(float(v)) ** 2 for v in x[i])
                v = float(S) / K + float(np.float32(eps))
                want = np.float32(0.0) if v == 0.0 else np.float32(1.0 / math.sqrt(v))
                assert r[i] == want, (K, eps, i)


def test_power_of_two_scaling_leaves_the_norm_unchanged(oracle):
    """eps = 0: x * 2^k scales S by 4^k exactly, so rstd by 2^-k exactly and
    the normalized row is bit-identical."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((5, 256))
    x = np.where(np.abs(x) < 2.0 ** -6, 2.0 ** -6, x).astype(np.float16)   # no fp16 subnormals at 2^-4 x
    g = (1 + 0.1 * rng.standard_normal(256)).astype(np.float16)
    y0 = oracle.rmsnorm(x, g, 0.0)
    for k in (-4, 3):
        xs = (x.astype(np.float32) * 2.0 ** k).astype(np.float16)
        assert np.array_equal(xs.astype(np.float32), x.astype(np.float32) * 2.0 ** k)
        assert np.array_equal(oracle.rms_rstd(xs, 0.0), oracle.rms_rstd(x, 0.0) * np.float32(2.0 ** -k))
        assert np.array_equal(oracle.rmsnorm(xs, g, 0.0), y0)


def test_validation(oracle):
    with pytest.raises(ValueError):
        oracle.rms_rstd(np.ones((1, 4), np.float16), -1.0)
    with pytest.raises(ValueError):
        oracle.rms_rstd(np.ones((1, 4), np.float16), float("inf"))
    with pytest.raises(TypeError):
        oracle.rms_rstd(np.ones((1, 4), np.float32), 0.0)


# ---------------------------------------------------------------------------
# the normalized row
# ---------------------------------------------------------------------------
def test_output_roundings_match_torch_fp16_arithmetic(oracle):
    """Given rstd, y = gamma * fp16(x * rstd) as torch computes it on the CPU
    (fp32 product rounded to fp16, then an fp16 product)."""
    import torch
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((16, 512)) * rng.choice([1, 40], size=512)).astype(np.float16)
    g = (1 + 0.2 * rng.standard_normal(512)).astype(np.float16)
    r = oracle.rms_rstd(x, 1e-5)
    xt = torch.from_numpy(x)
    ref = (xt.float() * torch.from_numpy(r)[:, None]).half() * torch.from_numpy(g)
    assert ref.dtype == torch.float16
    assert np.array_equal(oracle.rmsnorm(x, g, 1e-5).view(np.uint16), ref.numpy().view(np.uint16))


def test_output_is_within_two_half_ulps_of_the_real_norm(oracle):
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((4, 2048)) * rng.choice([1, 30], size=2048)).astype(np.float16)
    g = (1 + 0.5 * rng.standard_normal(2048)).astype(np.float16)
    y = oracle.rmsnorm(x, g, 1e-6).astype(np.float64)
    xd = x.astype(np.float64)
    true = g.astype(np.float64) * xd / np.sqrt((xd ** 2).mean(axis=1, keepdims=True) + 1e-6)
    bound = 1.01 * 2.0 ** -10 * np.abs(true) + 2.0 ** -24 * (np.abs(g.astype(np.float64)) + 1)
    assert np.all(np.abs(y - true) <= bound)


@pytest.mark.parametrize("group", [0, 16])
def test_quantized_norm_follows_a_joint_channel_relabel(oracle, group):
    """Relabeling the K channels of X, gamma and the outlier set together gives
    the same codes and scales (per-row mode; in group mode the relabel keeps
    every channel's reordered position). A gamma read at the reordered
    position instead of the original channel fails this."""
    rng = np.random.default_rng(21 + group)
    K, n_out = 64, 16
    x = (rng.standard_normal((5, K)) * 3).astype(np.float16)
    g = (1 + 0.3 * rng.standard_normal(K)).astype(np.float16)
    out = np.sort(rng.choice(K, n_out, replace=False))
    perm = oracle.make_perm(K, out)
    q = oracle.rmsnorm_quantize_rows(x, g, 1e-6, perm, n_out, group)
    sigma = rng.permutation(K)                 # new label of old channel c is sigma[c]
    inv = np.argsort(sigma)
    x2, g2 = np.ascontiguousarray(x[:, inv]), np.ascontiguousarray(g[inv])
    perm2 = sigma[perm].astype(np.int32)       # the same reordered sequence of channels
    q2 = oracle.quantize_rows(oracle.rmsnorm(x2, g2, 1e-6), perm2, n_out, group)
    for a, b in zip(q, q2):
        assert np.array_equal(a, b)
