"""Property tests of the oracle's chain verification (no GPU), on random small
batches drawn by hypothesis. Each property follows from the method as the
pages define it [Primer 考点2, 考点4]:

* every request emits at least one token and at most gamma + 1; the accepted
  prefix is the drafted prefix; the row is padded with -1 after the last
  token; tokens lie in [0, V);
* after a rejection at position n the drawn token has more target than draft
  mass, and it is not the rejected draft token (the residual's support);
* the draw is monotone in its uniform (inverse CDF): a larger u_sample at the
  final position never gives a smaller token index;
* acceptance is monotone in its uniforms: lowering one u_accept never lowers
  the number of accepted drafts.
"""
import numpy as np
import scipy.special
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle

SETTINGS = settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])


@st.composite
def chain_batch(draw):
    B = draw(st.integers(1, 4))
    g = draw(st.integers(0, 4))
    V = draw(st.integers(2, 24))
    T = draw(st.sampled_from([0.0, 0.5, 1.0, 2.0]))
    seed = draw(st.integers(0, 2 ** 32 - 1))
    rng = np.random.default_rng(seed)
    # small-integer logits give ties; a few -inf entries give zero mass
    tgt = rng.integers(-4, 5, size=(B, g + 1, V)).astype(np.float32) * np.float32(0.75)
    dft = (tgt[:, :g] + rng.normal(0.0, 1.5, size=(B, g, V))).astype(np.float32)
    for a in (tgt, dft):
        m = rng.random(a.shape) < 0.1
        m[..., 0] = False  # every row keeps a finite value
        a[m] = -np.inf
    tok = rng.integers(0, V, size=(B, g)).astype(np.int32)
    ua = (rng.random((B, g)) * (1 - 2 ** -24)).astype(np.float32)
    us = (rng.random((B, g + 1)) * (1 - 2 ** -24)).astype(np.float32)
    return dict(target=tgt, draft=dft, draft_tokens=tok, u_accept=ua, u_sample=us,
                temperature=np.full(B, T, np.float32))


def run(d):
    return oracle.verify_chain(d["target"], d["draft"], d["draft_tokens"], d["u_accept"], d["u_sample"],
                               d["temperature"])


@SETTINGS
@given(chain_batch())
def test_output_shape_and_padding(d):
    r = run(d)
    B, g = d["draft_tokens"].shape
    V = d["target"].shape[-1]
    for b in range(B):
        n = int(r["num_accepted"][b])
        assert 0 <= n <= g
        row = r["out_tokens"][b]
        assert (row[:n] == d["draft_tokens"][b, :n]).all()
        assert 0 <= row[n] < V
        assert (row[n + 1:] == -1).all()


@SETTINGS
@given(chain_batch())
def test_residual_support(d):
    r = run(d)
    B, g = d["draft_tokens"].shape
    T = float(d["temperature"][0])
    if T == 0.0:
        return
    for b in range(B):
        n = int(r["num_accepted"][b])
        if n == g:
            continue
        pt = scipy.special.softmax(d["target"][b, n].astype(np.float64) / T)
        pd = scipy.special.softmax(d["draft"][b, n].astype(np.float64) / T)
        y = int(r["out_tokens"][b, n])
        if (pt - pd).clip(min=0).sum() > 1e-12:  # a residual with mass (else the target row is used)
            assert pt[y] > pd[y]
            assert y != d["draft_tokens"][b, n]


@SETTINGS
@given(chain_batch(), st.floats(0.0, 1.0 - 2 ** -24, width=32), st.floats(0.0, 1.0 - 2 ** -24, width=32))
def test_draw_monotone_in_its_uniform(d, u1, u2):
    lo, hi = sorted((np.float32(u1), np.float32(u2)))
    r = run(d)
    B = d["draft_tokens"].shape[0]
    a = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in d.items()}
    b_ = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in d.items()}
    for b in range(B):
        n = int(r["num_accepted"][b])
        a["u_sample"][b, n] = lo
        b_["u_sample"][b, n] = hi
    ra, rb = run(a), run(b_)
    assert np.array_equal(ra["num_accepted"], r["num_accepted"]) and np.array_equal(rb["num_accepted"],
                                                                                      r["num_accepted"])
    for b in range(B):
        n = int(r["num_accepted"][b])
        assert ra["out_tokens"][b, n] <= rb["out_tokens"][b, n]


@SETTINGS
@given(chain_batch(), st.integers(0, 3), st.floats(0.0, 1.0, width=32))
def test_acceptance_monotone_in_its_uniforms(d, pos, scale):
    g = d["draft_tokens"].shape[1]
    if g == 0:
        return
    pos = pos % g
    r = run(d)
    lower = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in d.items()}
    lower["u_accept"][:, pos] = (lower["u_accept"][:, pos] * np.float32(scale)).astype(np.float32)
    r2 = run(lower)
    assert (r2["num_accepted"] >= r["num_accepted"]).all()
