"""Statistical pins of the oracle (no GPU).

* Losslessness [Primer 考点2, the total-probability identity]: the token emitted
  at position i is distributed as p_target of that position. Pearson chi-square
  over 10^6 requests at V = 16; planted mistakes in the oracle must fail it.
* Expected tokens per step [Primer 考点4]: (1 - a^(g+1)) / (1 - a) under a
  constructed constant acceptance rate a; the page's printed 3.36 equals the
  mean of min(n+1, g).
* Lower bound [Primer 考点4]: with a = 0 every step still yields one token.
"""
import json
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats

import inputgen
import oracle

V16 = 16


def _tiled_requests(t_rows, d_rows, B, seed):
    """B requests sharing the same logits; draft tokens drawn per request from p_draft."""
    g = d_rows.shape[0]
    target = np.ascontiguousarray(np.broadcast_to(t_rows, (B,) + t_rows.shape))
    draft = np.ascontiguousarray(np.broadcast_to(d_rows, (B,) + d_rows.shape))
    T = np.ones(B, np.float32)
    tok = inputgen.sample_tokens(seed, draft.reshape(-1, t_rows.shape[-1]), np.ones(B * g, np.float32),
                                 np.arange(B * g, dtype=np.int64)).reshape(B, g)
    ua = inputgen.uniform24(seed, inputgen.S_UACC, B * g).reshape(B, g)
    us = inputgen.uniform24(seed, inputgen.S_USAMP, B * (g + 1)).reshape(B, g + 1)
    return target, draft, tok, ua, us, T


def _chi2_p(counts, p):
    n = counts.sum()
    exp = n * p
    stat = ((counts - exp) ** 2 / exp).sum()
    return scipy.stats.chi2.sf(stat, len(p) - 1)


def _rows(gamma, seed):
    rng = np.random.default_rng(seed)
    t = rng.normal(0, 1.0, size=(gamma + 1, V16)).astype(np.float32)
    d = (t[:gamma] + rng.normal(0, 1.0, size=(gamma, V16))).astype(np.float32)
    return t, d


def _position_hist(res, i, B):
    na = res["num_accepted"]
    sel = na >= i
    return np.bincount(res["out_tokens"][sel, i], minlength=V16), sel.sum()


@pytest.fixture(scope="module")
def gamma1():
    t, d = _rows(1, 100)
    B = 1_000_000
    return t, d, _tiled_requests(t, d, B, seed=101)


def test_lossless_chi_square_gamma1(gamma1):
    t, d, (target, draft, tok, ua, us, T) = gamma1
    r = oracle.verify_chain(target, draft, tok, ua, us, T)
    pt0 = scipy.special.softmax(t[0].astype(np.float64))
    assert pt0.min() > 1e-3
    counts, n = _position_hist(r, 0, len(T))
    assert n == len(T)
    p = _chi2_p(counts, pt0)
    assert p > 1e-3, p
    # the rejection path is exercised
    assert 0.05 < (r["num_accepted"] == 0).mean() < 0.95


@pytest.mark.parametrize("mutant", [oracle.MUT_LOGIT_RESIDUAL, oracle.MUT_RESAMPLE_TARGET,
                                    oracle.MUT_ALWAYS_ACCEPT])
def test_lossless_negative_controls_fail(gamma1, mutant):
    """Planted mistakes (residual over raw logits, resampling from p_t, no rejection) must fail."""
    t, d, (target, draft, tok, ua, us, T) = gamma1
    r = oracle.verify_chain(target, draft, tok, ua, us, T, mutant=mutant)
    counts, _ = _position_hist(r, 0, len(T))
    pt0 = scipy.special.softmax(t[0].astype(np.float64))
    assert _chi2_p(counts, pt0) < 1e-6


def test_lossless_per_position_gamma3():
    """gamma = 3: at every position i (requests that reach i) the emitted token ~ p_t,i;
    dropping the bonus row fails at position gamma."""
    t, d = _rows(3, 200)
    B = 400_000
    target, draft, tok, ua, us, T = _tiled_requests(t, d, B, seed=201)
    r = oracle.verify_chain(target, draft, tok, ua, us, T)
    for i in range(4):
        counts, n = _position_hist(r, i, B)
        assert n > 20_000
        assert _chi2_p(counts, scipy.special.softmax(t[i].astype(np.float64))) > 1e-3, i
    rm = oracle.verify_chain(target, draft, tok, ua, us, T, mutant=oracle.MUT_NO_BONUS)
    counts, _ = _position_hist(rm, 3, B)
    assert _chi2_p(counts, scipy.special.softmax(t[3].astype(np.float64))) < 1e-6


def _constant_alpha(alpha, gamma, B, seed):
    """p_draft = 1/8 on tokens 0..7 (exactly 0 elsewhere); p_target = alpha/8 on 0..7 and
    (1-alpha)/8 on 8..15, so every drafted token has acceptance ratio alpha."""
    d = np.full(V16, -1e4, np.float32)
    d[:8] = 0.0
    t = np.empty(V16, np.float32)
    t[:8] = np.log(alpha / 8) if alpha > 0 else -1e4
    t[8:] = np.log((1 - alpha) / 8)
    t_rows = np.tile(t, (gamma + 1, 1))
    d_rows = np.tile(d, (gamma, 1))
    return _tiled_requests(t_rows, d_rows, B, seed)


def test_expected_tokens_closed_form(golden_dir):
    with open(os.path.join(golden_dir, "primer_worked_examples.json")) as f:
        cases = json.load(f)["expected_tokens"]
    for case in cases:
        g, a = case["gamma"], case["alpha"]
        B = 200_000
        target, draft, tok, ua, us, T = _constant_alpha(a, g, B, seed=300 + int(a * 10))
        r = oracle.verify_chain(target, draft, tok, ua, us, T)
        n = r["num_accepted"].astype(np.float64)
        k = np.arange(g + 1)
        pk = np.where(k < g, a ** k * (1 - a), a ** g)
        mean = ((k + 1) * pk).sum()
        assert mean == pytest.approx(case["formula_value"], rel=1e-4)
        sd = np.sqrt((((k + 1) - mean) ** 2 * pk).sum())
        assert abs((n + 1).mean() - case["formula_value"]) < 5 * sd / np.sqrt(B)
        # geometric law of the accepted count
        counts = np.bincount(r["num_accepted"], minlength=g + 1)
        assert _chi2_p(counts, pk) > 1e-3
        # the page's printed value is the count without the extra token
        no_bonus = np.minimum(n + 1, g).mean()
        ref = (1 - a ** g) / (1 - a)
        assert abs(no_bonus - ref) < 5 * sd / np.sqrt(B)
        if a == 0.8:
            assert ref == pytest.approx(case["page_printed_value"], abs=0.005)
        # residual tokens land uniformly on 8..15
        rej = r["num_accepted"] < g
        ys = r["out_tokens"][np.nonzero(rej)[0], r["num_accepted"][rej]]
        assert ys.min() >= 8
        assert _chi2_p(np.bincount(ys - 8, minlength=8), np.full(8, 1 / 8)) > 1e-3


def test_lower_bound_alpha_zero(golden_dir):
    with open(os.path.join(golden_dir, "primer_worked_examples.json")) as f:
        assert json.load(f)["lower_bound"]["min_tokens_per_step"] == 1
    target, draft, tok, ua, us, T = _constant_alpha(0.0, 5, 50_000, seed=400)
    r = oracle.verify_chain(target, draft, tok, ua, us, T)
    assert (r["num_accepted"] == 0).all()
    y = r["out_tokens"][:, 0]
    assert (y >= 8).all()
    assert _chi2_p(np.bincount(y - 8, minlength=8), np.full(8, 1 / 8)) > 1e-3
