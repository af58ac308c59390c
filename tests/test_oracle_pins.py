"""Pins of the CPU oracle against what the pages and mathematics fix (no GPU).

Each test names the passage or the independent routine it checks against.
"""
import json
import os

import numpy as np
import pytest
import scipy.special

import inputgen
import oracle


def _single(p_target, p_draft, token, u_accept, u_sample, T=1.0, bonus_row=None):
    """One request, gamma = 1, logits = log(p) so that softmax recovers p."""
    pt = np.log(np.asarray(p_target, np.float64)).astype(np.float32)
    pd = np.log(np.asarray(p_draft, np.float64)).astype(np.float32)
    bonus = pt if bonus_row is None else np.log(np.asarray(bonus_row)).astype(np.float32)
    target = np.stack([pt, bonus])[None]
    draft = pd[None, None]
    return oracle.verify_chain(target, draft, np.array([[token]]), np.array([[u_accept]], np.float32),
                               np.array([[u_sample, u_sample]], np.float32), np.array([T], np.float32))


def _cases(golden_dir):
    with open(os.path.join(golden_dir, "primer_worked_examples.json")) as f:
        return json.load(f)


def test_worked_acceptance_examples(golden_dir):
    """[Primer 考点2 / 第二章 / 第三章] printed probabilities: accept iff u < printed ratio;
    on rejection the residual is a single token, drawn for every u_sample."""
    for case in _cases(golden_dir)["acceptance_cases"]:
        a = case["accept_probability"]
        for u in (0.0, a - 1e-4, a + 1e-4, 1.0 - 2.0 ** -24):
            if not (0.0 <= u < 1.0):
                continue
            for us in (0.0, 0.37, 1.0 - 2.0 ** -24):
                r = _single(case["p_target"], case["p_draft"], case["token"], u, us)
                n = int(r["num_accepted"][0])
                expect_accept = u < a
                assert n == (1 if expect_accept else 0), (case["cite"], u)
                if expect_accept:
                    assert r["out_tokens"][0, 0] == case["token"]
                else:
                    assert r["out_tokens"][0, 0] == case["derived_residual_token_always"], (case["cite"], u, us)
                    assert r["out_tokens"][0, 1] == -1
                pt, pd = r["p_t"][0], r["p_d"][0]
                assert pt == pytest.approx(case["p_target"][case["token"]], rel=1e-6)
                assert pd == pytest.approx(case["p_draft"][case["token"]], rel=1e-6)


def test_zero_draft_probability_semantics():
    """Division-free test u*P_d < P_t: P_d = 0 accepts iff P_t > 0."""
    V = 4
    t = np.array([0.0, 0.0, -1e4, 0.0], np.float32)
    d = np.array([0.0, -1e4, -1e4, 0.0], np.float32)
    target = np.stack([t, t])[None]
    draft = d[None, None]
    for tok, expect in ((1, 1), (2, 0)):
        r = oracle.verify_chain(target, draft, np.array([[tok]]), np.array([[0.999]], np.float32),
                                np.array([[0.5, 0.5]], np.float32), np.array([1.0], np.float32))
        assert r["num_accepted"][0] == expect


def test_row_stats_against_scipy():
    """log Z = logsumexp(l/T) - max(l)/T (scipy), max and first-occurrence argmax (numpy)."""
    rng = np.random.default_rng(0)
    rows = rng.normal(0, 3, size=(40, 1000)).astype(np.float32)
    rows[3, 17] = rows[3, 500] = rows[3].max() + 1  # tie: first index must win
    rows[5, :] = -np.inf
    rows[5, 999] = 2.0
    T = np.where(np.arange(40) % 3 == 0, 0.0, 0.3 + 0.1 * np.arange(40)).astype(np.float32)
    s = oracle.row_stats(rows, T)
    for r in range(40):
        l = rows[r].astype(np.float64)
        assert s["valid"][r]
        assert s["max"][r] == l.max()
        if T[r] == 0:
            assert s["argmax"][r] == int(np.argmax(l))
        else:
            ref = scipy.special.logsumexp(l / T[r]) - l.max() / T[r]
            assert s["logz"][r] == pytest.approx(ref, rel=1e-12, abs=1e-12)
    assert s["argmax"][3] == 17


def test_greedy_reduces_to_argmax_prefix_match():
    """T = 0: n = first position where the draft token differs from numpy.argmax of the target row."""
    B, g, V = 64, 6, 50
    rng = np.random.default_rng(1)
    target = rng.integers(-3, 3, size=(B, g + 1, V)).astype(np.float32)  # many ties
    draft = rng.normal(size=(B, g, V)).astype(np.float32)
    amax = target.argmax(-1)
    tok = amax[:, :g].copy()
    cut = rng.integers(0, g + 1, size=B)
    for b in range(B):
        if cut[b] < g:
            tok[b, cut[b]] = (tok[b, cut[b]] + 1 + rng.integers(0, V - 1)) % V
    ua = np.full((B, g), np.nan, np.float32)  # unused when greedy
    us = np.full((B, g + 1), np.nan, np.float32)
    r = oracle.verify_chain(target, draft, tok, ua, us, np.zeros(B, np.float32))
    for b in range(B):
        n = int(np.argmax(np.append(tok[b] != amax[b, :g], True)))
        assert r["num_accepted"][b] == n
        assert list(r["out_tokens"][b, :n]) == list(tok[b, :n])
        assert r["out_tokens"][b, n] == amax[b, n]
        assert (r["out_tokens"][b, n + 1:] == -1).all()


def test_bonus_matches_numpy_searchsorted():
    """All drafts accepted (draft == target, ratio 1): the bonus token is
    numpy.searchsorted(cumsum(p), u*sum(p), 'right') of scipy's softmax of the last row."""
    d = inputgen.chain_inputs(256, 3, 300, seed=11, scale=2.0, noise_sd=0.0, temperature=0.7)
    T = float(np.float32(0.7))
    r = oracle.verify_chain(d["target"], d["draft"], d["draft_tokens"], d["u_accept"], d["u_sample"],
                            d["temperature"])
    assert (r["num_accepted"] == 3).all()
    checked = 0
    for b in range(256):
        p = scipy.special.softmax(d["target"][b, 3].astype(np.float64) / T)
        c = np.cumsum(p)
        y = int(np.searchsorted(c, float(d["u_sample"][b, 3]) * c[-1], side="right"))
        if r["cdf_margin"][b] > 1e-9:
            assert r["out_tokens"][b, 3] == y
            checked += 1
    assert checked > 250


def test_residual_support_invariant():
    """On rejection the emitted token has p_t > p_d and differs from the rejected draft token."""
    d = inputgen.make("tiny", seed=123, B=400)
    r = oracle.verify_chain(d["target"], d["draft"], d["draft_tokens"], d["u_accept"], d["u_sample"],
                            d["temperature"])
    rejected = 0
    for b in range(400):
        n = int(r["num_accepted"][b])
        if n < 4:
            rejected += 1
            y = int(r["out_tokens"][b, n])
            pt = scipy.special.softmax(d["target"][b, n].astype(np.float64))
            pd = scipy.special.softmax(d["draft"][b, n].astype(np.float64))
            assert pt[y] > pd[y]
            assert y != d["draft_tokens"][b, n]
    assert rejected > 50


def test_request_validation_sentinels():
    """Unusable inputs give num_accepted = -1 and -1 tokens, for that request only."""
    base = inputgen.make("tiny", seed=7)

    def run(mod):
        d = {k: (v.copy() if hasattr(v, "copy") else v) for k, v in base.items()}
        mod(d)
        return oracle.verify_chain(d["target"], d["draft"], d["draft_tokens"], d["u_accept"], d["u_sample"],
                                   d["temperature"])

    good = run(lambda d: None)
    assert (good["num_accepted"] >= 0).all()
    mods = {
        "T nan": lambda d: d["temperature"].__setitem__(2, np.nan),
        "T neg": lambda d: d["temperature"].__setitem__(2, -1.0),
        "T inf": lambda d: d["temperature"].__setitem__(2, np.inf),
        "T subnormal": lambda d: d["temperature"].__setitem__(2, 1e-40),
        "token high": lambda d: d["draft_tokens"].__setitem__((2, 3), 256),
        "token neg": lambda d: d["draft_tokens"].__setitem__((2, 0), -1),
        "u_accept 1": lambda d: d["u_accept"].__setitem__((2, 3), 1.0),
        "u_sample nan": lambda d: d["u_sample"].__setitem__((2, 4), np.nan),
        "nan target": lambda d: d["target"].__setitem__((2, 4, 17), np.nan),
        "inf target": lambda d: d["target"].__setitem__((2, 1, 0), np.inf),
        "nan draft": lambda d: d["draft"].__setitem__((2, 3, 255), np.nan),
        "all -inf": lambda d: d["draft"].__setitem__((2, 0), -np.inf),
    }
    for name, mod in mods.items():
        r = run(mod)
        assert r["num_accepted"][2] == -1, name
        assert (r["out_tokens"][2] == -1).all(), name
        keep = np.arange(8) != 2
        assert (r["num_accepted"][keep] == good["num_accepted"][keep]).all(), name
        assert (r["out_tokens"][keep] == good["out_tokens"][keep]).all(), name
    # -inf entries are allowed as long as a finite value remains
    r = run(lambda d: d["target"].__setitem__((2, 0, slice(0, 200)), -np.inf))
    assert r["num_accepted"][2] >= 0
    # greedy requests read neither the draft rows nor the uniforms
    def greedy_bad_draft(d):
        d["temperature"][2] = 0.0
        d["draft"][2, :, :] = np.nan
        d["u_accept"][2] = np.nan
    assert run(greedy_bad_draft)["num_accepted"][2] >= 0


def test_monotone_in_u_accept():
    """Lowering every u_accept can only lengthen the accepted prefix."""
    d = inputgen.make("tiny", seed=5, B=200)
    r1 = oracle.verify_chain(d["target"], d["draft"], d["draft_tokens"], d["u_accept"], d["u_sample"],
                             d["temperature"])
    r2 = oracle.verify_chain(d["target"], d["draft"], d["draft_tokens"], d["u_accept"] * 0.5, d["u_sample"],
                             d["temperature"])
    assert (r2["num_accepted"] >= r1["num_accepted"]).all()
    assert (r1["num_accepted"] >= 0).all() and (r1["out_tokens"][np.arange(200), r1["num_accepted"]] >= 0).all()


def test_temperature_scales_softmax():
    """Softmax at T equals scipy's softmax of l/T at the drafted token (per-position diagnostics)."""
    d = inputgen.make("tiny", seed=9)
    d["temperature"][:] = 0.45
    r = oracle.verify_chain(d["target"], d["draft"], d["draft_tokens"], d["u_accept"], d["u_sample"],
                            d["temperature"])
    for b in range(8):
        for i in range(4):
            x = d["draft_tokens"][b, i]
            T = float(np.float32(0.45))  # the temperature input is float32
            pt = scipy.special.softmax(d["target"][b, i].astype(np.float64) / T)[x]
            pd = scipy.special.softmax(d["draft"][b, i].astype(np.float64) / T)[x]
            assert r["p_t"][b * 4 + i] == pytest.approx(pt, rel=1e-12)
            assert r["p_d"][b * 4 + i] == pytest.approx(pd, rel=1e-12)


def test_bf16_decoding_is_exact():
    """bf16 bits decode to the float32 with those high 16 bits (checked through row maxima)."""
    bits = np.array([[0x3F80, 0x4049, 0xC2F7, 0x0001, 0x7F7F, 0xFF7F]], np.uint16)
    s = oracle.row_stats(bits, np.array([0.0], np.float32))
    expect = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert s["max"][0] == expect.max()
    assert s["argmax"][0] == 4
