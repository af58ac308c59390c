"""Pins of the oracle's draft-token sampler (no GPU).

The sampler draws one token per row from p = softmax(l/T) [Edge, scheduler
section: the temperature softmax] with the inverse-CDF rule of the verify draw,
y = min{ j : C_j > u*S } in ascending token order; the draft model proposes
its tokens this way [Primer 考点1]. T == 0 is the lowest-index argmax.

Pinned by:
* hand-computed CDF intervals of a four-token distribution;
* zero-mass tokens are never drawn, and the top of the CDF gives the last
  token of positive mass;
* greedy rows equal numpy.argmax (first occurrence), ties included;
* temperature: drawing from l at T = 2 equals drawing from l/2 at T = 1;
* the histogram of 10^6 draws matches softmax(l/T) (Pearson chi-square), and
  draws made at the wrong temperature fail that test;
* a verify request with gamma = 0 (bonus token only) draws the same token;
* unusable rows give -1.
"""
import numpy as np
import scipy.special
import scipy.stats

import inputgen
import oracle


def _rows(l, n):
    return np.ascontiguousarray(np.broadcast_to(np.asarray(l, np.float32), (n, len(l))))


def test_cdf_intervals_by_hand():
    # p = (0.1, 0.2, 0.3, 0.4): the CDF steps at 0.1, 0.3 and 0.6
    logits = _rows(np.log([0.1, 0.2, 0.3, 0.4]), 8)
    u = np.array([0.0, 0.0999, 0.1001, 0.2999, 0.3001, 0.5999, 0.6001, 1.0 - 2.0 ** -24], np.float32)
    r = oracle.sample_rows(logits, 1.0, u)
    assert r["tokens"].tolist() == [0, 0, 1, 1, 2, 2, 3, 3]
    assert np.all(r["margin"] >= 0.0)


def test_zero_mass_never_drawn():
    ninf = -np.inf
    logits = _rows([ninf, 0.0, ninf, 0.0, ninf], 6)
    u = np.array([0.0, 0.25, 0.4999, 0.5001, 0.75, 1.0 - 2.0 ** -24], np.float32)
    r = oracle.sample_rows(logits, 1.0, u)
    assert r["tokens"].tolist() == [1, 1, 1, 3, 3, 3]


def test_greedy_is_first_argmax():
    rng = np.random.default_rng(7)
    l = rng.integers(-4, 5, size=(200, 37)).astype(np.float32)  # many tied maxima
    r = oracle.sample_rows(l, 0.0, 0.5)
    assert np.array_equal(r["tokens"], np.argmax(l, axis=1))
    assert np.all(np.isnan(r["margin"]))
    # greedy rows ignore the uniform, even an unusable one
    assert np.array_equal(oracle.sample_rows(l, 0.0, 2.0)["tokens"], np.argmax(l, axis=1))


def test_temperature_scaling_is_exact():
    rng = np.random.default_rng(8)
    l = (rng.integers(-64, 64, size=(1000, 50)) / 8.0).astype(np.float32)  # halving is exact
    u = inputgen.uniform24(8, inputgen.S_USAMP, 1000)
    a = oracle.sample_rows(l, 2.0, u)["tokens"]
    b = oracle.sample_rows(l / np.float32(2.0), 1.0, u)["tokens"]
    assert np.array_equal(a, b)


def test_histogram_matches_softmax():
    rng = np.random.default_rng(9)
    l = rng.normal(0.0, 1.0, size=16).astype(np.float32)
    T = 0.8
    n = 1_000_000
    u = inputgen.uniform24(9, inputgen.S_USAMP, n)
    tok = oracle.sample_rows(_rows(l, n), T, u)["tokens"]
    counts = np.bincount(tok, minlength=16)

    def chi2_p(p):
        e = n * p
        return scipy.stats.chi2.sf(((counts - e) ** 2 / e).sum(), len(p) - 1)

    p = scipy.special.softmax(l.astype(np.float64) / T)
    assert p.min() > 1e-3
    assert chi2_p(p) > 1e-3
    # the same draws tested against the wrong temperature fail
    assert chi2_p(scipy.special.softmax(l.astype(np.float64) / 1.0)) < 1e-6


def test_matches_the_verify_bonus_draw():
    d = inputgen.make("tiny")
    rows = d["target"][:, 0, :]  # [B, V] fp32
    B = rows.shape[0]
    u = inputgen.uniform24(11, inputgen.S_USAMP, B)
    T = d["temperature"]
    ref = oracle.verify_chain(rows[:, None, :], np.zeros((B, 0, rows.shape[1]), np.float32),
                              np.zeros((B, 0), np.int32), np.zeros((B, 0), np.float32), u[:, None], T)
    assert np.array_equal(ref["num_accepted"], np.zeros(B, np.int32))
    assert np.array_equal(oracle.sample_rows(rows, T, u)["tokens"], ref["out_tokens"][:, 0])


def test_unusable_rows():
    l = np.zeros((9, 4), np.float32)
    l[6, 2] = np.nan
    l[7, :] = -np.inf
    l[8, 1] = np.inf
    T = np.array([np.nan, -1.0, 1e-40, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0], np.float32)
    u = np.array([0.5, 0.5, 0.5, 1.0, np.nan, -0.25, 0.5, 0.5, 0.5], np.float32)
    r = oracle.sample_rows(l, T, u)
    assert r["tokens"].tolist() == [-1] * 9
