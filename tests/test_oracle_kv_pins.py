"""Pins for the oracle's low-bit KV cache (readings V1-V2).

Atom summary page (Summary paragraph 2): the KV cache is kept in low bit-width.
The NQKV abstract on the "smoothquant" tag page quantizes the cache per block.
Reading V1: every (token, head) vector is one block of the layer's symmetric
quantizer (R1-R5), INT4 or INT8. V2: dequantization is fp16(fl32(s * q)).

The block quantizer itself is pinned in test_oracle_pins.py; here: the
per-(token, head) blocking against a literal loop, the dequantization error
bound, a lossless grid, and the byte layout.
"""
import numpy as np
import pytest


@pytest.mark.parametrize("bits", [4, 8])
def test_blocks_are_token_head_vectors(oracle, bits):
    rng = np.random.default_rng(bits)
    T, H, D = 5, 3, 64
    X = (rng.standard_normal((T, H, D)) * rng.choice([0.1, 1, 20], (T, H, 1))).astype(np.float16)
    q, s = oracle.kv_quantize(X, bits)
    qmax = 7 if bits == 4 else 127
    for t in range(T):
        for h in range(H):
            qb, sb = oracle.quantize_block(X[t, h].astype(np.float32), qmax)
            assert np.array_equal(q[t, h], qb) and s[t, h] == sb


@pytest.mark.parametrize("bits", [4, 8])
def test_dequantization_error_bound(oracle, bits):
    rng = np.random.default_rng(10 + bits)
    X = (rng.standard_normal((64, 8, 128)) * 3).astype(np.float16)
    q, s = oracle.kv_quantize(X, bits)
    qmax = 7 if bits == 4 else 127
    y = oracle.kv_dequantize(q, s).astype(np.float64)
    sd = s.astype(np.float64)[..., None]
    bound = sd * (0.5 + qmax * 2.0 ** -24) + np.abs(y) * 2.0 ** -11 + 2.0 ** -25
    assert np.all(np.abs(y - X.astype(np.float64)) <= bound)


def test_dequantization_rounding_by_hand(oracle):
    """s = fl32(0.1) times q = 3: the fp32 product is 0.30000001192...; fp16
    spacing at 0.3 is 2^-12 and 0.30000001192 / 2^-12 = 1228.80005, so the
    fp16 result is 1229 * 2^-12 = 0.300048828125."""
    s = np.array([[np.float32(0.1)]])
    q = np.array([[[3, -7, 0, 1]]], np.int8)
    y = oracle.kv_dequantize(q, s)
    want = [np.float16(np.float32(0.1) * np.float32(v)) for v in (3, -7, 0, 1)]
    assert np.array_equal(y[0, 0], np.array(want, np.float16))
    assert float(y[0, 0, 0]) == 1229 * 2.0 ** -12


@pytest.mark.parametrize("bits", [4, 8])
def test_lossless_grid(oracle, bits):
    """Heads c * 2^e with integer c in [-qmax, qmax] and +-qmax present: the
    scale is 2^e, the codes are c and the dequantized cache equals X."""
    qmax = 7 if bits == 4 else 127
    rng = np.random.default_rng(20 + bits)
    T, H, D = 6, 4, 128
    c = rng.integers(-qmax, qmax + 1, (T, H, D))
    c[:, :, 5] = qmax
    e = rng.integers(-12, 2, (T, H, 1))
    X = (c * 2.0 ** e).astype(np.float16)
    assert np.array_equal(X.astype(np.float64), c * 2.0 ** e)
    q, s = oracle.kv_quantize(X, bits)
    assert np.array_equal(q, c.astype(np.int8))
    assert np.array_equal(oracle.kv_dequantize(q, s), X)


def test_pack_layout(oracle):
    q = np.array([[[1, -1, -8, 7]]], np.int8)
    assert list(oracle.kv_pack(q, 4)[0, 0]) == [0xF1, 0x78]
    assert list(oracle.kv_pack(q, 8)[0, 0]) == [1, 255, 248, 7]
