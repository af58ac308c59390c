"""GPU parity of the KV-cache steps through the C ABI against the oracle:
spec_kv_commit (sink + ring caches), spec_kv_valid_slots and
spec_draft_window. Integer and byte work: every cache byte, length, slot,
position and block id must equal the oracle's."""
import numpy as np
import pytest

import inputgen
import oracle
from _parity import device_inputs, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    import torch

    import rejection_sampling_verify_spec_amd as m
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    return m


def _alloc(a, offset=0):
    """Device copy of a uint8 array at `offset` bytes past a fresh allocation (to reach the 4- and
    1-byte access paths)."""
    import torch
    buf = torch.empty(a.size + offset, dtype=torch.uint8, device="cuda")
    t = buf[offset:].view(a.shape)
    t.copy_(torch.from_numpy(np.ascontiguousarray(a)))
    return t


def _commit_steps(sv, B, gamma, R, E, S, W, steps, seed, offset=0, lengths=None, bad=True):
    import torch
    rng = np.random.default_rng(seed)
    cap = S + W
    kc_h = rng.integers(0, 256, size=(B, R, cap, E), dtype=np.uint8)
    vc_h = rng.integers(0, 256, size=(B, R, cap, E), dtype=np.uint8)
    kc, vc = _alloc(kc_h, offset), _alloc(vc_h, offset)
    if lengths is None:
        lengths = rng.integers(0, 3 * cap, size=B).astype(np.int32)
    lengths = np.asarray(lengths, np.int32)
    print(f"[commit] B {B} gamma {gamma} R {R} E {E} S {S} W {W} offset {offset}", flush=True)
    for step in range(steps):
        d = inputgen.kv_inputs(B, gamma, R, E, S, W, seed * 100 + step)
        n = d["num_accepted"].copy()
        if bad and B >= 3:
            n[0] = -1
            n[1] = gamma + 1
        kn, vn = _alloc(d["k_new"], offset), _alloc(d["v_new"], offset)
        new = sv.kv_commit(kc, vc, kn, vn, to_dev(lengths), to_dev(n), S, W)
        ref = oracle.kv_commit(kc_h, vc_h, d["k_new"], d["v_new"], lengths, n, S, W)
        torch.cuda.synchronize()
        assert np.array_equal(new.cpu().numpy(), ref), f"step {step}: lengths"
        assert np.array_equal(kc.cpu().numpy(), kc_h), f"step {step}: k_cache"
        assert np.array_equal(vc.cpu().numpy(), vc_h), f"step {step}: v_cache"
        lengths = ref


@pytest.mark.parametrize("E,offset", [(48, 0), (256, 16), (12, 4), (7, 1), (6, 2)])
def test_commit_access_paths(sv, E, offset):
    """16-, 4- and 1-byte accesses (row size and base alignment), several steps, wrapped rings."""
    _commit_steps(sv, B=13, gamma=5, R=3, E=E, S=3, W=7, steps=5, seed=E + offset)


@pytest.mark.parametrize("S,W,gamma", [(0, 1, 4), (1, 2, 5), (0, 5, 5), (4, 3, 7), (6, 60, 0), (4, 1020, 5)])
def test_commit_ring_shapes(sv, S, W, gamma):
    """Rings shorter than the kept positions (a later position wins its slot), no sinks, gamma 0."""
    _commit_steps(sv, B=9, gamma=gamma, R=2, E=32, S=S, W=W, steps=4, seed=S * 7 + W + gamma)


def test_commit_long_rows(sv):
    """Rows of 40000 bytes: one row per workgroup, many accesses per thread."""
    _commit_steps(sv, B=3, gamma=3, R=2, E=40000, S=2, W=3, steps=2, seed=3, bad=False)


def test_commit_lengths_near_the_int32_limit(sv):
    top = 2 ** 31 - 1
    _commit_steps(sv, B=6, gamma=3, R=2, E=16, S=3, W=7, steps=1, seed=4, bad=False,
                  lengths=[top - 3, top - 4, top - 10, top, 0, 5])


def test_commit_empty_batch(sv):
    import torch
    z = torch.empty((0, 2, 10, 16), dtype=torch.uint8, device="cuda")
    zn = torch.empty((0, 4, 2, 16), dtype=torch.uint8, device="cuda")
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    assert sv.kv_commit(z, z.clone(), zn, zn.clone(), e, e.clone(), 3, 7).numel() == 0


def test_commit_after_verify(sv):
    """The commit consumes what verification returns: accepted counts of a verify call on the
    tiny workload decide which staged positions are kept."""
    import torch
    d = inputgen.make("tiny")
    t = device_inputs(d)
    out, na = sv.verify_chain(t["target"], t["draft"], t["draft_tokens"], t["u_accept"], t["u_sample"],
                              t["temperature"])
    ref_v = oracle.verify_chain(d["target"], d["draft"], d["draft_tokens"], d["u_accept"], d["u_sample"],
                                d["temperature"])
    torch.cuda.synchronize()
    assert np.array_equal(na.cpu().numpy(), ref_v["num_accepted"])
    B, gamma = d["draft_tokens"].shape
    S, W, R, E = 4, 6, 3, 32
    kv = inputgen.kv_inputs(B, gamma, R, E, S, W, 77)
    kc_h = np.zeros((B, R, S + W, E), np.uint8)
    vc_h = np.zeros_like(kc_h)
    kc, vc = _alloc(kc_h), _alloc(vc_h)
    new = sv.kv_commit(kc, vc, _alloc(kv["k_new"]), _alloc(kv["v_new"]), to_dev(kv["lengths"]), na, S, W)
    ref = oracle.kv_commit(kc_h, vc_h, kv["k_new"], kv["v_new"], kv["lengths"], ref_v["num_accepted"], S, W)
    torch.cuda.synchronize()
    assert np.array_equal(new.cpu().numpy(), ref)
    assert np.array_equal(kc.cpu().numpy(), kc_h) and np.array_equal(vc.cpu().numpy(), vc_h)


def test_commit_full_size(sv):
    """The measured workload (B=256, gamma=5, 256 rows of 256 bytes, S=4, W=1020; 2 x 17.2 GB caches):
    every kept row equals its staged row at the slot the oracle names, every other byte keeps its fill,
    and the lengths equal the oracle's."""
    import torch
    d = inputgen.make("kv")
    B, gamma, R, E, S, W = (d[k] for k in ("lengths", "gamma", "rows", "row_bytes", "sink", "window"))
    B = B.shape[0]
    cap = S + W
    print(f"[commit-full] B {B} R {R} E {E} cap {cap}", flush=True)
    fill = 0x5A
    kc = torch.full((B, R, cap, E), fill, dtype=torch.uint8, device="cuda")
    vc = torch.full((B, R, cap, E), fill, dtype=torch.uint8, device="cuda")
    kn, vn = _alloc(d["k_new"]), _alloc(d["v_new"])
    new = sv.kv_commit(kc, vc, kn, vn, to_dev(d["lengths"]), to_dev(d["num_accepted"]), S, W)
    # lengths and kept (request, position) -> slot from the oracle (zero-width rows)
    zc = np.zeros((B, 1, cap, 0), np.uint8)
    zn = np.zeros((B, gamma + 1, 1, 0), np.uint8)
    ref_len = oracle.kv_commit(zc, zc.copy(), zn, zn.copy(), d["lengths"], d["num_accepted"], S, W)
    torch.cuda.synchronize()
    assert np.array_equal(new.cpu().numpy(), ref_len)
    owner = {}
    for b in range(B):
        P, n = int(d["lengths"][b]), int(d["num_accepted"][b])
        for j in range(n + 1):
            owner[(b, oracle.slot(P + j, S, W))] = j
    bi = torch.tensor([k[0] for k in owner], device="cuda")
    si = torch.tensor([k[1] for k in owner], device="cuda")
    ji = torch.tensor(list(owner.values()), device="cuda")
    for cache, staged in ((kc, kn), (vc, vn)):
        got = cache[bi, :, si, :]
        assert torch.equal(got, staged[bi, ji]), "kept rows"
        cache[bi, :, si, :] = fill
        flat = cache.view(-1)
        step = 1 << 30
        for o in range(0, flat.numel(), step):
            assert not bool((flat[o:o + step] != fill).any()), f"stray write near byte {o}"
    del kc, vc
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- valid slots

@pytest.mark.parametrize("S,W", [(4, 1020), (0, 1), (3, 7), (0, 300), (600, 1), (1, 1)])
def test_valid_slots(sv, S, W):
    import torch
    cap = S + W
    rng = np.random.default_rng(cap)
    edge = [-5, 0, 1, max(S - 1, 0), S, cap - 1, cap, cap + 1, 2 * cap + 3, 2 ** 31 - 1, -(2 ** 31)]
    lengths = np.concatenate([edge, rng.integers(0, 5 * cap, size=300)]).astype(np.int32)
    print(f"[valid-slots] S {S} W {W} B {lengths.size}", flush=True)
    slots, pos, counts = sv.kv_valid_slots(to_dev(lengths), S, W)
    slots2, none, counts2 = sv.kv_valid_slots(to_dev(lengths), S, W, positions=False)
    ref = oracle.kv_valid_slots(lengths, S, W)
    torch.cuda.synchronize()
    assert none is None
    assert np.array_equal(slots.cpu().numpy(), ref["slots"])
    assert np.array_equal(pos.cpu().numpy(), ref["positions"])
    assert np.array_equal(counts.cpu().numpy(), ref["counts"])
    assert torch.equal(slots, slots2) and torch.equal(counts, counts2)


# ---------------------------------------------------------------- draft window

def _window_case(sv, seq, W, bs, K, table, cols=None):
    import torch
    cols = sv.spec_draft_window_max_blocks(W, bs) if cols is None else cols
    lens, tab = sv.draft_window(to_dev(seq), to_dev(table), W, bs, K, window_cols=cols)
    ref = oracle.draft_window(seq, W, bs, K, table, cols)
    torch.cuda.synchronize()
    assert np.array_equal(lens.cpu().numpy(), ref["windowed_lens"])
    assert np.array_equal(tab.cpu().numpy(), ref["block_table"])
    return lens, tab


def test_window_worked_example(sv):
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "window_worked_example.json")))
    table = (np.arange(4 * 16, dtype=np.int32).reshape(4, 16) + 1)
    lens, _ = _window_case(sv, np.array(g["seq_lens"], np.int32), g["window"], g["block_size"],
                           g["future_offset"], table)
    assert lens.cpu().numpy().tolist() == g["windowed_lens"]


@pytest.mark.parametrize("W,bs,K,cols", [(64, 16, 3, 20), (63, 16, 0, 12), (2048, 128, 5, 320), (50, 7, 5, 40),
                                         (1, 1, 0, 9), (8, 8, 8, 6), (300, 16, 2, 1)])
def test_window_shapes(sv, W, bs, K, cols):
    rng = np.random.default_rng(W + bs + K)
    top = cols * bs
    seq = np.concatenate([[-1, 0, 1, W - K, W - K + 1, top, top + 5 * bs, 2 ** 31 - 1, -(2 ** 31)],
                          rng.integers(0, top + 1, size=200)]).astype(np.int32)
    table = (rng.permutation(seq.size * cols * 2)[:seq.size * cols].reshape(seq.size, cols) + 1).astype(np.int32)
    print(f"[window] W {W} b {bs} K {K} cols {cols}", flush=True)
    _window_case(sv, seq, W, bs, K, table)
    _window_case(sv, seq, W, bs, K, table, cols=sv.spec_draft_window_max_blocks(W, bs) + 3)


def test_window_in_place_and_host_copies(sv):
    """Device lengths windowed in place, and host copies through spec_draft_window_host: one transform."""
    import torch
    d = inputgen.make("window")
    W, bs, K = d["window"], d["block_size"], d["future_offset"]
    seq = to_dev(d["seq_lens"])
    table = to_dev(d["block_table"])
    B, cols = d["block_table"].shape
    wc = sv.spec_draft_window_max_blocks(W, bs)
    out_tab = torch.empty((B, wc), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    assert sv.spec_draft_window(seq, B, W, bs, K, table, cols, seq, out_tab, wc, stream) == 0
    host = d["seq_lens"].copy()
    assert sv.spec_draft_window_host(host.ctypes.data, B, W, bs, K, host.ctypes.data) == 0
    ref = oracle.draft_window(d["seq_lens"], W, bs, K, d["block_table"], wc)
    torch.cuda.synchronize()
    assert np.array_equal(seq.cpu().numpy(), ref["windowed_lens"])
    assert np.array_equal(host, ref["windowed_lens"])
    assert np.array_equal(out_tab.cpu().numpy(), ref["block_table"])


def test_window_full_table_untouched(sv):
    """The full table (what KV writes address) is never changed by the window."""
    import torch
    d = inputgen.make("window")
    table = to_dev(d["block_table"])
    before = table.clone()
    _window_case(sv, d["seq_lens"], d["window"], d["block_size"], d["future_offset"], d["block_table"])
    sv.draft_window(to_dev(d["seq_lens"]), table, d["window"], d["block_size"], d["future_offset"])
    torch.cuda.synchronize()
    assert torch.equal(table, before)
