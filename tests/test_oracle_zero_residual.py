"""Pins of the oracle's zero-residual branches (no GPU).

The residual max(0, P_t - P_d) / sum of [Primer 考点2, P'] sums to a positive number on every
rejection in exact arithmetic when the two rows differ; when the target and draft rows are equal
and the drafted token has zero probability in both, the token is rejected (u * 0 < 0 is false)
and the residual is identically 0. The oracle then draws from P_t of the same row with the same
uniform (chain, and the lowest-child tree rule), or keeps the current distribution r (lossless
walk), and raises its `fallback` flag. Every expected value below is worked out by hand from the
probabilities in the comments; the rows are logits whose softmax is those probabilities.
"""
import numpy as np

import oracle

NEG = -np.inf
# softmax of [0, 0, -inf, 0] is (1/3, 1/3, 0, 1/3): cumulative 1/3, 2/3, 2/3, 1
THIRDS = np.array([0.0, 0.0, NEG, 0.0], np.float32)


def _chain(target_rows, draft_rows, tokens, ua, us, T=1.0):
    target = np.asarray(target_rows, np.float32)[None]
    draft = np.asarray(draft_rows, np.float32).reshape(1, len(tokens), -1)
    return oracle.verify_chain(target, draft, np.array([tokens], np.int32), np.array([ua], np.float32),
                               np.array([us], np.float32), np.array([T], np.float32))


def test_chain_zero_residual_draws_from_the_target_row():
    """gamma = 1: equal rows, drafted token 2 of zero mass: n = 0, and y follows (1/3, 1/3, 0, 1/3)
    at u_s: 0.1 -> 0, 0.4 -> 1, 0.5 -> 1, 0.9 -> 3. The bonus row (0.7, 0.1, 0.1, 0.1) would give
    0, 0, 0, 3 and a fixed token 0 (the prior-art listing's answer to a zero sum) 0 everywhere."""
    bonus = np.log(np.array([0.7, 0.1, 0.1, 0.1])).astype(np.float32)
    for us, y in ((0.1, 0), (0.4, 1), (0.5, 1), (0.9, 3)):
        for ua in (0.0, 0.5, 1.0 - 2.0 ** -24):
            r = _chain([THIRDS, bonus], [THIRDS], [2], [ua], [us, 0.99])
            assert r["num_accepted"][0] == 0
            assert r["out_tokens"][0].tolist() == [y, -1], (us, ua)
            assert bool(r["fallback"][0])
            assert r["p_t"][0] == 0.0 and r["p_d"][0] == 0.0


def test_chain_zero_residual_at_a_later_position():
    """gamma = 2: position 0 drafts token 3 from equal rows (ratio 1, accepted for every u < 1);
    position 1 has equal rows (0.25, 0, 0, 0.75) and drafts token 1 of zero mass: n = 1 and y follows
    (0.25, 0, 0, 0.75): u_s 0.2 -> 0, 0.3 -> 3, 0.9 -> 3."""
    row0 = np.array([0.0, 1.0, 2.0, 3.0], np.float32)
    row1 = np.log(np.array([0.25, 0.0, 0.0, 0.75])).astype(np.float32)
    bonus = np.log(np.array([0.1, 0.6, 0.2, 0.1])).astype(np.float32)
    for us, y in ((0.2, 0), (0.3, 3), (0.9, 3)):
        r = _chain([row0, row1, bonus], [row0, row1], [3, 1], [0.99, 0.3], [0.5, us, 0.5])
        assert r["num_accepted"][0] == 1
        assert r["out_tokens"][0].tolist() == [3, y, -1], us
        assert bool(r["fallback"][0])


def test_chain_nonzero_residual_is_not_flagged():
    """A rejection with differing rows leaves a positive residual and no fallback flag: target
    (0.3, 0.7), draft (0.5, 0.5), token 0 (ratio 0.6) rejected at u = 0.9; the residual is (0, 0.2),
    so y = 1 for every u_s."""
    t = np.log(np.array([0.3, 0.7])).astype(np.float32)
    d = np.log(np.array([0.5, 0.5])).astype(np.float32)
    for us in (0.0, 0.5, 0.99):
        r = _chain([t, t], [d], [0], [0.9], [us, 0.5])
        assert r["num_accepted"][0] == 0 and r["out_tokens"][0].tolist() == [1, -1]
        assert not bool(r["fallback"][0])


def _tree(draft_node2, ua2, us, target_node2, lossless):
    """Root 0 with children 1 and 2. Root target row (1/3, 1/3, 0, 1/3); node 1 drafts token 2
    from a row equal to the root's target row (zero mass: rejected); node 2 drafts token 0 from
    draft_node2. target rows of nodes 1 and 2 as given."""
    V = 4
    target = np.stack([THIRDS, np.zeros(V, np.float32), np.asarray(target_node2, np.float32)])[None]
    draft = np.stack([THIRDS, np.asarray(draft_node2, np.float32)])[None]
    tokens = np.array([[0, 2, 0]], np.int32)
    parents = np.array([[-1, 0, 0]], np.int32)
    ua = np.array([[0.0, 0.5, ua2]], np.float32)
    us = np.asarray([us], np.float32)
    f = oracle.verify_tree_lossless if lossless else oracle.verify_tree
    return f(target, draft, tokens, parents, ua, us, np.array([1.0], np.float32), 1)


ONE_HOT0 = np.array([0.0, NEG, NEG, NEG], np.float32)          # (1, 0, 0, 0)
HALVES = np.array([0.0, 0.0, NEG, NEG], np.float32)           # (1/2, 1/2, 0, 0)


def test_tree_lowest_child_zero_residual():
    """Lowest-child rule: node 2 (token 0, draft (1, 0, 0, 0) against the root's 1/3) is accepted
    iff u < 1/3. At u = 0.9 both children are rejected, the end node is the root and the residual
    against its first child (node 1, a row equal to the root's) is 0: y follows the root's
    (1/3, 1/3, 0, 1/3) at u_s[0]: 0.5 -> 1, 0.9 -> 3. At u = 0.2 node 2 is the end node (a leaf):
    bonus from (1/2, 1/2, 0, 0) at u_s[2] = 0.7 -> 1, with no fallback."""
    for us0, y in ((0.5, 1), (0.9, 3)):
        r = _tree(ONE_HOT0, 0.9, [us0, 0.5, 0.5], HALVES, lossless=False)
        assert r["num_accepted"][0] == 0 and r["out_tokens"][0].tolist() == [y, -1], us0
        assert bool(r["fallback"][0])
    r = _tree(ONE_HOT0, 0.2, [0.5, 0.5, 0.7], HALVES, lossless=False)
    assert r["num_accepted"][0] == 1 and r["out_tokens"][0].tolist() == [0, 1]
    assert r["out_nodes"][0].tolist() == [2, -1]
    assert not bool(r["fallback"][0])


def test_lossless_zero_residual_keeps_r():
    """Lossless walk: node 1's rejection leaves max(0, r - P_d[1]) = 0, so r stays (1/3, 1/3, 0, 1/3)
    (fallback flagged). Node 2 is then tested against that r: accepted iff u < 1/3.
      u = 0.2: accepted, node 2 is a leaf, y from (1/2, 1/2, 0, 0) at u_s[2] = 0.7 -> 1.
      u = 0.5: rejected, r becomes max(0, r - (1, 0, 0, 0)) normalised = (0, 1/2, 0, 1/2), y at
               u_s[0]: 0.3 -> 1, 0.7 -> 3.
    A walk that zeroed or NaN-ed r at node 1 would reject node 2 at u = 0.2."""
    r = _tree(ONE_HOT0, 0.2, [0.5, 0.5, 0.7], HALVES, lossless=True)
    assert r["num_accepted"][0] == 1 and r["out_tokens"][0].tolist() == [0, 1]
    assert bool(r["fallback"][0])
    for us0, y in ((0.3, 1), (0.7, 3)):
        r = _tree(ONE_HOT0, 0.5, [us0, 0.5, 0.5], HALVES, lossless=True)
        assert r["num_accepted"][0] == 0 and r["out_tokens"][0].tolist() == [y, -1], us0
        assert bool(r["fallback"][0])


def test_lossless_zero_residual_as_the_last_sibling():
    """Both children draft token 2 from rows equal to the root's: both rejections leave r unchanged,
    and the final token follows the root's (1/3, 1/3, 0, 1/3) at u_s[0]: 0.1 -> 0, 0.5 -> 1."""
    V = 4
    target = np.stack([THIRDS, np.zeros(V, np.float32), HALVES])[None]
    draft = np.stack([THIRDS, THIRDS])[None]
    tokens = np.array([[0, 2, 2]], np.int32)
    parents = np.array([[-1, 0, 0]], np.int32)
    for us0, y in ((0.1, 0), (0.5, 1)):
        r = oracle.verify_tree_lossless(target, draft, tokens, parents, np.array([[0.0, 0.3, 0.6]], np.float32),
                                        np.array([[us0, 0.5, 0.5]], np.float32), np.array([1.0], np.float32), 1)
        assert r["num_accepted"][0] == 0 and r["out_tokens"][0].tolist() == [y, -1]
        assert bool(r["fallback"][0])
