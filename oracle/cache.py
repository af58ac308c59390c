"""CPU oracle of the two KV-cache steps around verification.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use this module; the HIP library shares no
code with it.

1. Sink + ring KV cache [Edge 环形上下文与注意力沉淀机制: attention sinks, the
   rolling window, the Slot(pos) equation; Edge C++ 环形 KV 缓存管理内核实现:
   pool layout ((layer*heads + head)*(S+W) + slot)*dim, the list of valid
   slots (sinks first, then the window in logical order)].
   Commit after verification: of the gamma+1 positions the target pass scored,
   the pending token and the n accepted drafts (n+1 positions, P .. P+n) are
   kept; the rest are dropped [Primer 考点1, 考点4]. The kept positions are
   written one after another, so a later position wins a slot that two of them
   share (possible when W < n+1).

2. Draft-KV sliding window [Window 窗口数学: start, windowed length, start
   block, blocks needed; Window block table 的裁剪方式: gather of the
   block-table row from the start block into a zero-filled clone, columns past
   the needed count or past the full width are zero].

Plain integer arithmetic in Python loops and numpy row copies; no blocking or
reordering beyond the definitions.
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------- sink + ring

def slot(pos: int, S: int, W: int) -> int:
    """Physical slot of logical position pos [Edge 环形上下文与注意力沉淀机制, the
    Slot(pos) equation]: sinks keep their index, later positions take the
    window slots modulo W."""
    if pos < S:
        return pos
    return S + (pos - S) % W


def valid_slots(P: int, S: int, W: int):
    """(slots, positions) the cache holds after P positions, in logical order
    [Edge C++ 环形 KV 缓存管理内核实现: all slots while P <= S+W; else the S
    sink slots, then the slots of the last W positions]."""
    if P <= 0:
        return [], []
    if P <= S + W:
        pos = list(range(P))
    else:
        pos = list(range(S)) + list(range(P - W, P))
    return [slot(p, S, W) for p in pos], pos


def kv_valid_slots(lengths, S: int, W: int):
    """Batched valid_slots: slots and positions [B, S+W] padded with -1, counts [B]."""
    lengths = np.asarray(lengths)
    B = lengths.shape[0]
    cap = S + W
    slots = np.full((B, cap), -1, np.int32)
    poss = np.full((B, cap), -1, np.int32)
    counts = np.zeros(B, np.int32)
    for b in range(B):
        s, p = valid_slots(int(lengths[b]), S, W)
        slots[b, :len(s)] = s
        poss[b, :len(p)] = p
        counts[b] = len(s)
    return {"slots": slots, "positions": poss, "counts": counts}


INT32_MAX = 2 ** 31 - 1


def kv_commit(k_cache, v_cache, k_new, v_new, lengths, num_accepted, S: int, W: int):
    """Commit of one verify step into sink + ring caches (updates the caches in
    place, returns the new lengths).

    k_cache, v_cache  [B, R, S+W, E]   R = layers*heads rows per position, E bytes
    k_new, v_new      [B, gamma+1, R, E]  KV the target pass produced for
                      positions P .. P+gamma (P = lengths[b])
    num_accepted      [B] n from verification, 0..gamma

    Positions P .. P+n are written to Slot(pos) in ascending order; the new
    length is P+n+1. A request with n outside [0, gamma], a negative length or
    a length past 2^31-1 keeps its cache and length.
    """
    lengths = np.asarray(lengths)
    num_accepted = np.asarray(num_accepted)
    B = lengths.shape[0]
    gamma = k_new.shape[1] - 1
    out = lengths.astype(np.int32).copy()
    for b in range(B):
        P = int(lengths[b])
        n = int(num_accepted[b])
        if n < 0 or n > gamma or P < 0 or P + n + 1 > INT32_MAX:
            continue
        for j in range(n + 1):
            s = slot(P + j, S, W)
            k_cache[b, :, s, :] = k_new[b, j, :, :]
            v_cache[b, :, s, :] = v_new[b, j, :, :]
        out[b] = P + n + 1
    return out


# ---------------------------------------------------------- draft KV window

def max_window_blocks(W: int, b: int) -> int:
    """Largest number of blocks a windowed range can span: the windowed length
    reaches W + b - 1 (start rounded down to a block boundary, future offset
    0), and the range starts on a block boundary."""
    return -(-(W + b - 1) // b)


def window_one(seq_len: int, W: int, b: int, K: int):
    """(start, windowed_len, start_block, needed) of one request [Window
    窗口数学]; None for a negative length."""
    if seq_len < 0:
        return None
    start = (max(seq_len + K - W, 0) // b) * b
    wl = seq_len - start
    return start, wl, start // b, -(-wl // b)


def draft_window(seq_lens, W: int, b: int, K: int, block_table, clone_cols: int):
    """Windowed lengths [B] and the windowed block table [B, clone_cols].

    Row i of the clone holds block_table[i, start_block + j] for j < needed
    while start_block + j lies inside the full table; every other column is 0.
    A negative length gives windowed length -1 and a zero row.
    """
    seq_lens = np.asarray(seq_lens)
    block_table = np.asarray(block_table)
    B = seq_lens.shape[0]
    full_cols = block_table.shape[1] if block_table.ndim == 2 else 0
    lens = np.empty(B, np.int32)
    clone = np.zeros((B, clone_cols), np.int32)
    for i in range(B):
        w = window_one(int(seq_lens[i]), W, b, K)
        if w is None:
            lens[i] = -1
            continue
        start, wl, sb, needed = w
        lens[i] = wl
        for j in range(min(needed, clone_cols)):
            if sb + j < full_cols:
                clone[i, j] = block_table[i, sb + j]
    return {"windowed_lens": lens, "block_table": clone}
