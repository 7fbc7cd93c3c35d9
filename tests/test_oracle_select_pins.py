"""Pins for the oracle's offline outlier-channel selection (reading S1).

Definition: score[c] = max over calibration rows of |x[r, c]| (fp16, exact);
channel c is selected iff fewer than n_out channels beat it, where j beats c
when score[j] > score[c], or score[j] == score[c] and j < c. The selected
channels are returned ascending. The pages keep a small set of outlier
channels in 8 bits after reordering (Atom summary page, Summary paragraph 2;
Interesting ideas I1 and I3) but give no rule for choosing them; the QUIK
abstract keeps "some outlier" activations in higher precision.

Pins: a literal-loop brute force of the rank rule, planted outlier columns,
closed cases (all ties, n_out = 0 or K, an empty batch) and invariances of the
definition (row order, signs, powers of two, channel relabeling).
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st


def _brute(X, n_out):
    R, K = X.shape
    score = [max([abs(float(X[r, c])) for r in range(R)] + [0.0]) for c in range(K)]
    sel = []
    for c in range(K):
        beaten_by = sum(1 for j in range(K) if score[j] > score[c] or (score[j] == score[c] and j < c))
        if beaten_by < n_out:
            sel.append(c)
    return score, sel


@settings(max_examples=80, deadline=None)
@given(st.integers(0, 6), st.integers(1, 24), st.integers(0, 10 ** 6), st.data())
def test_brute_force_rank_rule(oracle, R, K, seed, data):
    """Scores from a small value set so that ties are common."""
    n_out = data.draw(st.integers(0, K))
    rng = np.random.default_rng(seed)
    vals = np.array([0.0, 0.5, -0.5, 1.0, -1.0, 2.0, 3.0, -3.0, 65504.0, 2.0 ** -24], np.float16)
    X = vals[rng.integers(0, vals.size, (R, K))]
    score, sel = _brute(X, n_out)
    assert list(oracle.select_outliers(X, n_out)) == sel
    assert np.array_equal(oracle.channel_absmax(X).astype(np.float64), np.array(score))


def test_planted_outlier_columns(oracle):
    rng = np.random.default_rng(1)
    R, K, n_out = 64, 512, 24
    X = rng.standard_normal((R, K)).astype(np.float32)
    S = rng.choice(K, n_out, replace=False)
    X[:, S] *= 100
    assert np.array_equal(oracle.select_outliers(X.astype(np.float16), n_out), np.sort(S))


def test_closed_cases(oracle):
    X = np.full((3, 10), -1.5, np.float16)
    assert list(oracle.select_outliers(X, 4)) == [0, 1, 2, 3]          # all tied: lowest indices
    assert oracle.select_outliers(X, 0).size == 0
    assert list(oracle.select_outliers(X, 10)) == list(range(10))
    E = np.zeros((0, 7), np.float16)                                      # empty batch: all scores 0
    assert list(oracle.select_outliers(E, 3)) == [0, 1, 2]
    with pytest.raises(ValueError):
        oracle.select_outliers(X, 11)


def test_invariances(oracle):
    rng = np.random.default_rng(2)
    R, K, n_out = 40, 300, 17
    X = (rng.standard_normal((R, K)) * rng.choice([1, 10, 50], K)).astype(np.float16)
    X = np.where(np.abs(X) < 2.0 ** -10, np.float16(2.0 ** -10), X)      # no subnormals at 2^-3 X
    base = oracle.select_outliers(X, n_out)
    assert np.array_equal(oracle.select_outliers(X[rng.permutation(R)], n_out), base)
    flips = rng.choice([-1.0, 1.0], (R, K)).astype(np.float16)
    assert np.array_equal(oracle.select_outliers(X * flips, n_out), base)
    for k in (-3, 2):
        Xs = (X.astype(np.float32) * 2.0 ** k).astype(np.float16)
        assert np.array_equal(Xs.astype(np.float32), X.astype(np.float32) * 2.0 ** k)
        assert np.array_equal(oracle.select_outliers(Xs, n_out), base)
    # relabeling the channels maps the selection (distinct scores: no tie rule involved)
    X[0] = (1024 + rng.permutation(K)).astype(np.float16)               # distinct column maxima
    base = oracle.select_outliers(X, n_out)
    assert np.unique(oracle.channel_absmax(X)).size == K
    sigma = rng.permutation(K)                  # old channel c becomes sigma[c]
    X2 = np.empty_like(X)
    X2[:, sigma] = X
    assert np.array_equal(oracle.select_outliers(X2, n_out), np.sort(sigma[base]))


def test_selection_feeds_the_permutation(oracle):
    """make_perm of the selection puts exactly the n_out largest-score channels
    in the tail."""
    rng = np.random.default_rng(3)
    X = (rng.standard_normal((32, 128)) * rng.choice([1, 30], 128)).astype(np.float16)
    sel = oracle.select_outliers(X, 16)
    perm = oracle.make_perm(128, sel)
    a = oracle.channel_absmax(X).astype(np.float32)
    assert a[perm[112:]].min() >= a[perm[:112]].max()
