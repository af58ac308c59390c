"""Pins of the oracle's lossless multi-candidate tree verification (no GPU).

At a node the children are tried in index order, each against the current
distribution r (first P_t of the node); a rejected child replaces r by
norm(max(0, r - P_d[child])) [Primer 考点2: acceptance min(1, P_t/P_d), residual
P']; if no child is accepted the final token is drawn from r. Tree layout and
conventions as in verify_tree [Primer 考点3].

Pinned by:
* a three-token example worked by hand (acceptance threshold, a residual with
  one surviving token, a sibling that the residual rejects for sure and one
  it accepts for sure);
* losslessness (the identity of [Primer 考点2], extended to siblings): with
  each child's token drawn from its own draft row, the first emitted token
  follows P_t of the root (Pearson chi-square, 2, 3 and 4 siblings), and the
  token after an accepted child follows P_t of that child; planted mistakes
  (no residual update, no renormalisation) and the lowest-child rule of
  verify_tree fail the same test;
* chain-shaped trees give exactly the chain verification's tokens;
* greedy: the walk equals a brute-force walk that follows the first child
  holding the argmax (duplicated tokens included);
* unusable inputs give -1.
"""
import numpy as np
import pytest
import scipy.special
import scipy.stats

import inputgen
import oracle


def _log(p):
    return np.log(np.asarray(p, np.float64)).astype(np.float32)


def _tree(target_rows, draft_rows, parents, tokens, ua, us, T=1.0, max_depth=None):
    """Single-request inputs for the oracle (B = 1)."""
    N = len(parents)
    par = np.asarray(parents, np.int32)[None]
    depth = [0] * N
    for v in range(1, N):
        depth[v] = depth[parents[v]] + 1
    return dict(target=np.asarray(target_rows, np.float32)[None], draft=np.asarray(draft_rows, np.float32)[None],
                node_tokens=np.asarray(tokens, np.int32)[None], parents=par,
                u_accept=np.asarray(ua, np.float32)[None], u_sample=np.asarray(us, np.float32)[None],
                temperature=np.array([T], np.float32), max_depth=max_depth or max(depth) + 1)


def _run(d, fn=oracle.verify_tree_lossless, **kw):
    return fn(d["target"], d["draft"], d["node_tokens"], d["parents"], d["u_accept"], d["u_sample"],
              d["temperature"], d["max_depth"], **kw)


def test_worked_example_by_hand():
    # root: P_t = (0.5, 0.3, 0.2); child 1 drafts token 1 from (0.2, 0.6, 0.2): ratio 0.3/0.6 = 0.5;
    # after its rejection r = norm(max(0, P_t - q1)) = (1, 0, 0). Child 2 drafts from (0.1, 0.1, 0.8).
    tgt = [_log([0.5, 0.3, 0.2]), _log([0.2, 0.3, 0.5]), _log([0.6, 0.2, 0.2])]
    dft = [_log([0.2, 0.6, 0.2]), _log([0.1, 0.1, 0.8])]
    par = [-1, 0, 0]
    # child 1 accepted below the ratio
    r = _run(_tree(tgt, dft, par, [0, 1, 2], [0, 0.49, 0.5], [0.5, 0.0, 0.5]))
    assert r["num_accepted"][0] == 1 and r["out_nodes"][0, 0] == 1 and r["out_tokens"][0, :2].tolist() == [1, 0]
    # rejected: child 2's token 2 has no mass in r, so it is rejected whatever its uniform; r stays (1, 0, 0)
    for u2 in (0.0, 0.5, 0.999):
        for us0 in (0.0, 0.5, 0.999):
            r = _run(_tree(tgt, dft, par, [0, 1, 2], [0, 0.51, u2], [us0, 0.5, 0.5]))
            assert r["num_accepted"][0] == 0 and r["out_tokens"][0, 0] == 0
    # child 2 drafting token 0 instead: r(0) / q2(0) = 10, accepted whatever its uniform
    r = _run(_tree(tgt, dft, par, [0, 1, 0], [0, 0.51, 0.999], [0.5, 0.5, 0.0]))
    assert r["num_accepted"][0] == 1 and r["out_nodes"][0, 0] == 2 and r["out_tokens"][0, :2].tolist() == [0, 0]
    # the lowest-child rule of verify_tree draws from max(0, P_t - q1) as well here, but it tests
    # child 2 against P_t: 0.5 / 0.1 -> accepted; the lossless walk agrees on this one
    assert _run(_tree(tgt, dft, par, [0, 1, 0], [0, 0.51, 0.999], [0.5, 0.5, 0.0]),
                fn=oracle.verify_tree)["out_nodes"][0, 0] == 2


def _trial_batch(n_trials, parents, V, seed, noise=1.0):
    """n_trials copies of one tree with fixed logits; every child's token drawn afresh from its own
    draft row (independent inverse-CDF draws in double precision)."""
    rng = np.random.default_rng(seed)
    N = len(parents)
    tgt = rng.normal(0.0, 1.5, size=(N, V)).astype(np.float32)
    dft = np.stack([tgt[parents[v]] + rng.normal(0.0, noise, V) for v in range(1, N)]).astype(np.float32)
    q = scipy.special.softmax(dft.astype(np.float64), axis=1)
    u = rng.random((n_trials, N - 1))
    cdf = np.cumsum(q, axis=1)
    tok = np.zeros((n_trials, N), np.int32)
    for v in range(1, N):
        tok[:, v] = np.minimum((cdf[v - 1][None, :] <= u[:, v - 1:v]).sum(axis=1), V - 1)
    depth = [0] * N
    for v in range(1, N):
        depth[v] = depth[parents[v]] + 1
    return dict(target=np.ascontiguousarray(np.broadcast_to(tgt, (n_trials, N, V))),
                draft=np.ascontiguousarray(np.broadcast_to(dft, (n_trials, N - 1, V))),
                node_tokens=tok, parents=np.ascontiguousarray(np.broadcast_to(np.int32(parents), (n_trials, N))),
                u_accept=rng.random((n_trials, N)).astype(np.float32) * np.float32(1 - 2 ** -24),
                u_sample=rng.random((n_trials, N)).astype(np.float32) * np.float32(1 - 2 ** -24),
                temperature=np.ones(n_trials, np.float32), max_depth=max(depth) + 1), tgt


def _chi2_p(samples, p):
    counts = np.bincount(samples, minlength=len(p))
    e = samples.size * p
    return scipy.stats.chi2.sf(((counts - e) ** 2 / e).sum(), len(p) - 1)


@pytest.mark.parametrize("k", [2, 3, 4])
def test_lossless_one_level(k):
    V, n = 16, 200_000
    d, tgt = _trial_batch(n, [-1] + [0] * k, V, seed=20 + k, noise=2.0)
    p_root = scipy.special.softmax(tgt[0].astype(np.float64))
    r = _run(d)
    assert _chi2_p(r["out_tokens"][:, 0], p_root) > 1e-3
    acc = (r["num_accepted"] > 0).mean()
    assert 0.2 < acc < 0.98  # both branches exercised
    for mutant in (oracle.MUT_TREE_NO_UPDATE, oracle.MUT_TREE_NO_RENORM):
        bad = _run(d, mutant=mutant)
        assert _chi2_p(bad["out_tokens"][:, 0], p_root) < 1e-6, mutant
    assert _chi2_p(_run(d, fn=oracle.verify_tree)["out_tokens"][:, 0], p_root) < 1e-6


def test_lossless_two_levels():
    V, n = 16, 200_000
    par = [-1, 0, 0, 0, 1, 1, 2, 2, 3, 3]
    d, tgt = _trial_batch(n, par, V, seed=31)
    r = _run(d)
    p = scipy.special.softmax(tgt.astype(np.float64), axis=1)
    assert _chi2_p(r["out_tokens"][:, 0], p[0]) > 1e-3
    for c in (1, 2, 3):
        sel = r["out_nodes"][:, 0] == c
        assert sel.sum() > 10_000
        assert _chi2_p(r["out_tokens"][sel, 1], p[c]) > 1e-3, c
    # structure: kept nodes form a root path
    for i in range(200):
        na = r["num_accepted"][i]
        nodes = r["out_nodes"][i, :na].tolist()
        prev = 0
        for v in nodes:
            assert par[v] == prev
            prev = v


def test_chain_shaped_tree_equals_chain():
    d = inputgen.make("tiny")
    B, g = d["draft_tokens"].shape
    ref = oracle.verify_chain(d["target"], d["draft"], d["draft_tokens"], d["u_accept"], d["u_sample"],
                              d["temperature"])
    par = np.tile(np.arange(-1, g, dtype=np.int32), (B, 1))
    tok = np.concatenate([np.zeros((B, 1), np.int32), d["draft_tokens"]], axis=1)
    ua = np.concatenate([np.zeros((B, 1), np.float32), d["u_accept"]], axis=1)
    r = oracle.verify_tree_lossless(d["target"], d["draft"], tok, par, ua, d["u_sample"], d["temperature"], g)
    assert np.array_equal(r["num_accepted"], ref["num_accepted"])
    assert np.array_equal(r["out_tokens"], ref["out_tokens"])


def test_greedy_walk_by_brute_force():
    rng = np.random.default_rng(5)
    B, N, V = 300, 12, 6
    tgt = rng.integers(-3, 4, size=(B, N, V)).astype(np.float32)  # ties in the argmax
    dft = rng.normal(size=(B, N - 1, V)).astype(np.float32)
    par = np.zeros((B, N), np.int32)
    par[:, 0] = -1
    for v in range(1, N):
        par[:, v] = rng.integers(0, v, size=B)
    tok = rng.integers(0, V, size=(B, N)).astype(np.int32)
    depth = np.zeros((B, N), np.int32)
    for v in range(1, N):
        depth[:, v] = depth[np.arange(B), par[:, v]] + 1
    md = int(depth.max())
    z = np.zeros((B, N), np.float32)
    r = oracle.verify_tree_lossless(tgt, dft, tok, par, z, z, np.zeros(B, np.float32), md)
    for b in range(B):
        v, path = 0, []
        while True:
            a = int(np.argmax(tgt[b, v]))
            kids = [c for c in range(1, N) if par[b, c] == v and tok[b, c] == a]
            if not kids:
                break
            v = kids[0]
            path.append(v)
        assert r["num_accepted"][b] == len(path)
        assert r["out_nodes"][b, :len(path)].tolist() == path
        assert r["out_tokens"][b, len(path)] == int(np.argmax(tgt[b, v]))


def test_unusable_inputs():
    tgt = [_log([0.5, 0.3, 0.2])] * 3
    dft = [_log([0.2, 0.6, 0.2])] * 2
    bad = [
        _tree(tgt, dft, [-1, 0, 0], [0, 1, 3], [0, 0.5, 0.5], [0.5] * 3),         # token out of range
        _tree(tgt, dft, [-1, 0, 2], [0, 1, 1], [0, 0.5, 0.5], [0.5] * 3),         # parent not before child
        _tree(tgt, dft, [-1, 0, 0], [0, 1, 1], [0, 1.0, 0.5], [0.5] * 3),         # uniform out of [0, 1)
        _tree(tgt, dft, [-1, 0, 0], [0, 1, 1], [0, 0.5, 0.5], [0.5] * 3, T=-1.0),  # temperature
        _tree(tgt, dft, [-1, 0, 1], [0, 1, 1], [0, 0.5, 0.5], [0.5] * 3, max_depth=1),  # too deep
    ]
    for d in bad:
        r = _run(d)
        assert r["num_accepted"][0] == -1 and (r["out_tokens"][0] == -1).all()
