"""GPU parity of the offline outlier-channel selection (w4a4_select_outliers,
through the C ABI) against the oracle's select_outliers: selected indices,
permutation and per-channel absmax bit-exact. The pages keep a small set of
outlier channels in 8 bits after reordering (Atom summary page, Summary
paragraph 2, Interesting ideas I1 and I3) without a rule for choosing them;
the rule here is the top-n_out calibration absmax, ties to the lower index.
"""
import sys

import numpy as np
import pytest

import mixed_precision_integer_amd as w4
from mixed_precision_integer_amd import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    sys.stderr.write(f"\n[gpu case] {msg}\n")
    sys.stderr.flush()


def check(oracle, X, n_out, ld=None):
    R, K = X.shape
    ld = ld or (K + 7) // 8 * 8
    buf = torch.zeros((max(R, 1), ld), dtype=torch.float16, device=DEV)
    if R:
        buf[:R, :K] = torch.from_numpy(X).to(DEV)
    Xd = buf[:R, :K]
    idx, perm, amax = w4.select_outliers(Xd, n_out, want_absmax=True)
    want = oracle.select_outliers(X, n_out)
    torch.cuda.synchronize()
    assert np.array_equal(amax.cpu().numpy().view(np.uint16), oracle.channel_absmax(X).view(np.uint16)), "absmax"
    assert np.array_equal(idx.cpu().numpy(), want), "selected channels"
    assert np.array_equal(perm.cpu().numpy(), oracle.make_perm(K, want)), "permutation"
    return want


SELECT = [
    # rows, K, n_out
    (32768, 4096, 128),     # a calibration batch of 16 x 2048 tokens for a 4096-channel input
    (8192, 22016, 256),     # the 65B down_proj input channels
    (300, 11008, 1000),     # many selected, ragged row chunks
    (17, 4096, 4095),       # all but one
    (5, 300, 0),            # nothing selected
    (5, 300, 300),          # everything selected
    (3, 32768, 700),        # the widest row the selection takes
    (1, 8, 1),
    (4, 1, 1),              # one channel (a partial 8-channel group)
    (9, 7, 3),              # fewer channels than one 16-byte load
]


@pytest.mark.parametrize("rows,K,n_out", SELECT)
def test_select_parity(oracle, rows, K, n_out):
    _say(f"select rows={rows} K={K} n_out={n_out}")
    X, _, o = wl.draw(rows, 1, K, min(n_out, K // 2), seed=rows + K + n_out, outlier_factor=30.0)
    got = check(oracle, X, n_out)
    if rows >= 256 and 0 < n_out <= K // 2:
        assert set(o.tolist()) <= set(got.tolist()), "the planted heavy columns are found"


def test_select_ties(oracle):
    """Scores drawn from four values: the threshold falls inside a tie and the
    lower-index rule decides."""
    _say("select ties")
    rng = np.random.default_rng(7)
    vals = np.array([0.5, -1.0, 2.0, -2.0], np.float16)
    X = vals[rng.integers(0, 4, (37, 2048))]
    for n_out in (1, 100, 555, 1024, 2047):
        check(oracle, X, n_out)


def test_select_ragged_columns_and_pitch(oracle):
    _say("select ragged K=1003 ld=1016")
    X, _, _ = wl.draw(700, 1, 1003, 60, seed=11, outlier_factor=30.0)
    check(oracle, X, 60, ld=1016)


def test_select_empty_batch(oracle):
    _say("select empty batch")
    check(oracle, np.zeros((0, 96), np.float16), 10)


def test_select_feeds_the_layer(oracle):
    """The device permutation drives the producer: the same codes as the host
    make_perm of the oracle's selection."""
    _say("select then produce")
    X, _, _ = wl.draw(512, 1, 4096, 128, seed=5, outlier_factor=30.0)
    Xd = torch.from_numpy(X).to(DEV)
    idx, perm = w4.select_outliers(Xd, 128)
    a = w4.quant_reorder_act(Xd[:64].contiguous(), perm, 128, 128)
    p_h = oracle.make_perm(4096, oracle.select_outliers(X, 128))
    q4, s4, q8, s8 = oracle.quantize_rows(X[:64], p_h, 128, 128)
    torch.cuda.synchronize()
    assert np.array_equal(a.q4.cpu().numpy(), oracle.pack_nibbles(q4, 3968 // 2))
    assert np.array_equal(a.s4.cpu().numpy().view(np.uint32), s4.view(np.uint32))
