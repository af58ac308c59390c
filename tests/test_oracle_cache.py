"""Pins of the oracle's KV-cache steps (no GPU).

Sink + ring cache [Edge 环形上下文与注意力沉淀机制; Edge C++ 环形 KV 缓存管理内核实现]:
* Slot(pos) values worked by hand;
* an independent ring with a wrapping write pointer (no modulo) puts every
  position where Slot(pos) does, and holds exactly the positions valid_slots
  lists;
* commit over many verify steps: reading the cache through valid_slots gives,
  for every listed position, the keys and values of the token kept at that
  position, and the length counts the kept tokens; the in-place scheme (write
  every scored position into the ring, then move the length back) fails this
  once the ring has wrapped, and moving back by the accepted count fails the
  length;
* two kept positions on one slot (W < n+1): the later one is kept.

Draft-KV window [Window 窗口数学; Window block table 的裁剪方式]:
* the worked example the page prints (tests/golden/window_worked_example.json);
* the start is the largest block multiple not above max(L + K - W, 0), found
  by enumeration;
* windowed index t addresses the same KV block and offset as absolute position
  start + t;
* the window holds the last W - K positions (all of them while L + K <= W) and
  at most W - K + b - 1;
* the block count never passes ceil((W + b - 1) / b) and reaches it; the
  bound W//b + 1 holds only when W mod b is 0 or 1.
"""
import json
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


# ------------------------------------------------------------------ ring

def test_slot_by_hand():
    S, W = 4, 8
    got = [oracle.slot(p, S, W) for p in [0, 3, 4, 11, 12, 13, 20, 27, 28]]
    assert got == [0, 3, 4, 11, 4, 5, 4, 11, 4]
    assert oracle.valid_slots(7, 2, 3) == ([0, 1, 4, 2, 3], [0, 1, 4, 5, 6])
    assert oracle.valid_slots(3, 2, 3) == ([0, 1, 2], [0, 1, 2])
    assert oracle.valid_slots(5, 2, 3) == ([0, 1, 2, 3, 4], [0, 1, 2, 3, 4])
    assert oracle.valid_slots(0, 2, 3) == ([], [])


class PointerRing:
    """A sink + ring store written through a wrapping pointer (no modulo)."""

    def __init__(self, S, W):
        self.S, self.W = S, W
        self.held = [-1] * (S + W)
        self.n = 0
        self.ptr = S

    def append(self, pos):
        assert pos == self.n
        if pos < self.S:
            idx = pos
        else:
            idx = self.ptr
            self.ptr += 1
            if self.ptr == self.S + self.W:
                self.ptr = self.S
        self.held[idx] = pos
        self.n += 1
        return idx

    def listing(self):
        pairs = sorted((p, i) for i, p in enumerate(self.held) if p >= 0)
        return [i for _, i in pairs], [p for p, _ in pairs]


@pytest.mark.parametrize("S,W", [(0, 1), (0, 5), (4, 8), (3, 1), (1, 2), (4, 60), (7, 3)])
def test_slot_matches_pointer_ring(S, W):
    ring = PointerRing(S, W)
    for p in range(3 * (S + W) + 7):
        assert oracle.slot(p, S, W) == ring.append(p), p
        assert oracle.valid_slots(p + 1, S, W) == ring.listing(), p


def _step_data(rng, B, gamma, R, E):
    return (rng.integers(0, 256, size=(B, gamma + 1, R, E), dtype=np.uint8),
            rng.integers(0, 256, size=(B, gamma + 1, R, E), dtype=np.uint8))


def _check_cache(kc, vc, lengths, truth, S, W):
    for b in range(len(truth)):
        assert lengths[b] == len(truth[b])
        slots, pos = oracle.valid_slots(int(lengths[b]), S, W)
        expect = sorted(p for p in truth[b] if p < S or p >= lengths[b] - W)
        if pos != expect:
            return False
        for s, p in zip(slots, pos):
            if not (np.array_equal(kc[b, :, s], truth[b][p][0]) and np.array_equal(vc[b, :, s], truth[b][p][1])):
                return False
    return True


def _run_steps(commit, S, W, gamma, steps=40, B=6, R=2, E=3, seed=5):
    """Verify steps with random outcomes; truth[b][pos] holds the KV kept at pos."""
    rng = np.random.default_rng(seed)
    kc = np.zeros((B, R, S + W, E), np.uint8)
    vc = np.zeros_like(kc)
    lengths = np.zeros(B, np.int32)
    truth = [dict() for _ in range(B)]
    ok = True
    for _ in range(steps):
        kn, vn = _step_data(rng, B, gamma, R, E)
        n = rng.integers(0, gamma + 1, size=B).astype(np.int32)
        new = commit(kc, vc, kn, vn, lengths, n, S, W)
        for b in range(B):
            for j in range(n[b] + 1):
                truth[b][int(lengths[b]) + j] = (kn[b, j], vn[b, j])
        lengths = np.asarray(new, np.int32)
        ok = ok and _check_cache(kc, vc, lengths, truth, S, W)
    return ok


@pytest.mark.parametrize("S,W,gamma", [(4, 16, 5), (2, 3, 5), (0, 7, 4), (3, 1, 2)])
def test_commit_keeps_every_window_position(S, W, gamma):
    assert _run_steps(oracle.kv_commit, S, W, gamma)


def _inplace_then_rollback(kc, vc, kn, vn, lengths, n, S, W, by_accepted=False):
    """Every scored position written to its slot, then the length moved back."""
    gamma = kn.shape[1] - 1
    out = lengths.copy()
    for b in range(len(lengths)):
        P = int(lengths[b])
        for j in range(gamma + 1):
            s = oracle.slot(P + j, S, W)
            kc[b, :, s] = kn[b, j]
            vc[b, :, s] = vn[b, j]
        back = n[b] if by_accepted else gamma - n[b]
        out[b] = P + gamma + 1 - back
    return out


def test_inplace_rollback_loses_window_positions():
    # before the ring wraps the in-place scheme is harmless ...
    assert _run_steps(_inplace_then_rollback, 4, 400, 5, steps=20)
    # ... after it, rejected positions have overwritten live ones
    assert not _run_steps(_inplace_then_rollback, 4, 16, 5)


def test_rollback_by_accepted_count_is_wrong():
    with pytest.raises(AssertionError):
        _run_steps(lambda *a: _inplace_then_rollback(*a, by_accepted=True), 4, 400, 5, steps=5)


def test_commit_later_position_wins_a_shared_slot():
    S, W, gamma = 1, 2, 3
    kc = np.zeros((1, 1, 3, 1), np.uint8)
    vc = np.zeros_like(kc)
    kn = np.arange(10, 14, dtype=np.uint8).reshape(1, 4, 1, 1)
    vn = kn + 100
    new = oracle.kv_commit(kc, vc, kn, vn, np.array([1], np.int32), np.array([3], np.int32), S, W)
    # positions 1, 2, 3, 4 -> slots 1, 2, 1, 2: positions 3 and 4 (j = 2, 3) stay
    assert new.tolist() == [5]
    assert kc[0, 0, :, 0].tolist() == [0, 12, 13]
    assert vc[0, 0, :, 0].tolist() == [0, 112, 113]
    assert oracle.valid_slots(5, S, W) == ([0, 1, 2], [0, 3, 4])


def test_commit_leaves_bad_requests_alone():
    S, W, gamma = 2, 5, 3
    rng = np.random.default_rng(3)
    kn, vn = _step_data(rng, 4, gamma, 2, 4)
    kc = np.zeros((4, 2, S + W, 4), np.uint8)
    vc = np.zeros_like(kc)
    lengths = np.array([3, 3, -5, 2 ** 31 - 3], np.int32)
    n = np.array([-1, gamma + 1, 1, 3], np.int32)
    new = oracle.kv_commit(kc, vc, kn, vn, lengths, n, S, W)
    assert new.tolist() == lengths.tolist()
    assert not kc.any() and not vc.any()


def test_kv_valid_slots_batched():
    r = oracle.kv_valid_slots(np.array([0, 3, 7, -2, 100], np.int32), 2, 3)
    assert r["counts"].tolist() == [0, 3, 5, 0, 5]
    assert r["slots"][2].tolist() == [0, 1, 4, 2, 3]
    assert r["positions"][4].tolist() == [0, 1, 97, 98, 99]
    assert r["slots"][1].tolist() == [0, 1, 2, -1, -1]
    assert (r["slots"][0] == -1).all() and (r["positions"][3] == -1).all()


# ---------------------------------------------------------------- window

def test_window_worked_example():
    g = json.load(open(os.path.join(HERE, "golden", "window_worked_example.json")))
    table = np.arange(len(g["seq_lens"]) * 16, dtype=np.int32).reshape(len(g["seq_lens"]), 16) + 1
    r = oracle.draft_window(g["seq_lens"], g["window"], g["block_size"], g["future_offset"], table,
                            oracle.max_window_blocks(g["window"], g["block_size"]))
    assert r["windowed_lens"].tolist() == g["windowed_lens"]


def _brute_start(L, W, b, K):
    lo = max(L + K - W, 0)
    s = 0
    while s + b <= lo:
        s += b
    return s


@pytest.mark.parametrize("W,b,K", [(64, 16, 3), (64, 16, 0), (63, 16, 0), (50, 7, 5), (8, 8, 8), (2048, 128, 5),
                                   (5, 1, 2)])
def test_window_start_and_coverage(W, b, K):
    for L in range(0, 3 * W + 2 * b):
        start, wl, sb, needed = oracle.window_one(L, W, b, K)
        assert start == _brute_start(L, W, b, K)
        assert start % b == 0 and sb * b == start and wl == L - start
        # the last W - K positions (all of them while L + K <= W) are inside the window
        assert start <= max(L - (W - K), 0)
        if L + K <= W:
            assert wl == L
        assert 0 <= wl <= W - K + b - 1
        # blocks touched by [start, L)
        assert needed == len({t // b for t in range(start, L)})


@pytest.mark.parametrize("W,b", [(64, 16), (63, 16), (65, 16), (66, 16), (2048, 128), (100, 7), (1, 1), (3, 4)])
def test_window_block_bound(W, b):
    cap = oracle.max_window_blocks(W, b)
    most = max(oracle.window_one(L, W, b, 0)[3] for L in range(0, 4 * W + 4 * b))
    assert most == cap
    # the page's W//b + 1 holds exactly when W mod b is 0 or 1
    assert (most <= W // b + 1) == (W % b in (0, 1))
    for K in range(0, min(W, 9) + 1):
        assert max(oracle.window_one(L, W, b, K)[3] for L in range(0, 3 * W + 3 * b)) <= cap


def test_window_counterexample_to_the_page_bound():
    start, wl, sb, needed = oracle.window_one(78, 63, 16, 0)
    assert (start, wl, needed) == (0, 78, 5) and 63 // 16 + 1 == 4


def test_windowed_index_addresses_same_kv():
    rng = np.random.default_rng(11)
    W, b, K = 64, 16, 3
    B, cols = 40, 30
    seq = rng.integers(0, cols * b + 1, size=B).astype(np.int32)
    table = rng.permutation(B * cols * 3)[:B * cols].reshape(B, cols).astype(np.int32) + 1
    r = oracle.draft_window(seq, W, b, K, table, oracle.max_window_blocks(W, b))
    for i in range(B):
        wl = int(r["windowed_lens"][i])
        start = int(seq[i]) - wl
        for t in range(wl):
            a = start + t
            assert r["block_table"][i, t // b] * b + t % b == table[i, a // b] * b + a % b
        needed = -(-wl // b)
        assert (r["block_table"][i, needed:] == 0).all()


def test_window_zero_columns_and_bad_lengths():
    W, b, K = 32, 8, 2
    table = np.arange(1, 1 + 3 * 4, dtype=np.int32).reshape(3, 4)  # full table covers 32 tokens
    r = oracle.draft_window(np.array([-1, 100, 31], np.int32), W, b, K, table, oracle.max_window_blocks(W, b))
    assert r["windowed_lens"].tolist() == [-1, 100 - 64, 31 - 0]
    assert (r["block_table"][0] == 0).all()
    # L = 100: start block 8 lies past the 4 columns of the full table -> zeros
    assert (r["block_table"][1] == 0).all()
    assert r["block_table"][2].tolist() == [9, 10, 11, 12, 0]
