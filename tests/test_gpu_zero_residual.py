"""GPU parity of the zero-residual branches (through the C ABI) against the oracle.

A drafted token of zero probability in equal target and draft rows is rejected and leaves a
residual max(0, P_t - P_d) that is identically 0 [Primer 考点2, P']. The chain and the
lowest-child tree rule then draw from P_t of the same row with the same uniform; the lossless
walk keeps its current distribution. The hand cases of tests/test_oracle_zero_residual.py run
here as they are (f32) and in bf16, then the same construction inside batches of full-size rows
(several chunks and sampling tiles, aligned and misaligned rows, normal and Student-t logits).
Every constructed request must be flagged `fallback` by the oracle, and tokens, counts (and tree
paths) must equal the oracle's.
"""
import numpy as np
import pytest

import inputgen
import oracle
from _parity import assert_tokens_match, device_inputs

pytestmark = pytest.mark.gpu

NEG = -np.inf
THIRDS = np.array([0.0, 0.0, NEG, 0.0], np.float32)


@pytest.fixture(scope="module")
def sv():
    import torch

    import rejection_sampling_verify_spec_amd as m
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    return m


def bf16_bits(a):
    """float32 -> bf16 bit patterns, round to nearest even (exact for 0, +-inf and small integers)."""
    b = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def _as(dtype, a):
    return a if dtype == "f32" else bf16_bits(a)


def run_chain(sv, d):
    import torch
    t = device_inputs(d)
    out, na = sv.verify_chain(t["target"], t["draft"], t["draft_tokens"], t["u_accept"], t["u_sample"],
                              t["temperature"])
    torch.cuda.synchronize()
    ref = oracle.verify_chain(d["target"], d["draft"], d["draft_tokens"], d["u_accept"], d["u_sample"],
                              d["temperature"])
    return out.cpu().numpy(), na.cpu().numpy(), ref


def run_tree(sv, d, lossless):
    import torch
    t = device_inputs(d)
    f = sv.verify_tree_lossless if lossless else sv.verify_tree
    out, nodes, na = f(t["target"], t["draft"], t["node_tokens"], t["parents"], t["u_accept"], t["u_sample"],
                       t["temperature"], d["max_depth"])
    torch.cuda.synchronize()
    g = oracle.verify_tree_lossless if lossless else oracle.verify_tree
    ref = g(d["target"], d["draft"], d["node_tokens"], d["parents"], d["u_accept"], d["u_sample"],
            d["temperature"], d["max_depth"])
    return out.cpu().numpy(), nodes.cpu().numpy(), na.cpu().numpy(), ref


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chain_hand_cases(sv, dtype):
    """Equal rows, token 2 of zero mass: n = 0 and y from (1/3, 1/3, 0, 1/3) at u_s (0.1 -> 0,
    0.5 -> 1, 0.9 -> 3); one request per u_s in one batch."""
    bonus = np.log(np.array([0.7, 0.1, 0.1, 0.1])).astype(np.float32)
    us_list = [0.1, 0.4, 0.5, 0.9]
    B = len(us_list)
    target = np.stack([np.stack([THIRDS, bonus])] * B)
    d = dict(target=_as(dtype, target), draft=_as(dtype, np.stack([THIRDS[None]] * B)),
             draft_tokens=np.full((B, 1), 2, np.int32), u_accept=np.full((B, 1), 0.5, np.float32),
             u_sample=np.array([[u, 0.99] for u in us_list], np.float32), temperature=np.ones(B, np.float32))
    print(f"[zero residual hand chain {dtype}]", flush=True)
    out, na, ref = run_chain(sv, d)
    assert ref["fallback"].all()
    assert_tokens_match(out, na, ref, f"hand chain {dtype}")
    if dtype == "f32":
        assert out[:, 0].tolist() == [0, 1, 1, 3] and (na == 0).all()


def _zero_residual_chain(d, reqs, pos):
    """Request b in reqs: draft rows 0..pos equal to the target rows, the drafted token at `pos` of
    -inf logit in both rows (positions before pos then have ratio 1 and are accepted)."""
    for b in reqs:
        for i in range(pos + 1):
            d["draft"][b, i] = d["target"][b, i]
        x = int(d["draft_tokens"][b, pos])
        neg = np.float32(NEG) if d["target"].dtype == np.float32 else np.uint16(0xFF80)
        d["target"][b, pos, x] = neg
        d["draft"][b, pos, x] = neg


@pytest.mark.parametrize("dtype,V,dist", [("f32", 40001, inputgen.DIST_NORMAL),
                                          ("bf16", 40001, inputgen.DIST_NORMAL),
                                          ("bf16", 65536, inputgen.DIST_T3),
                                          ("f32", 32768, inputgen.DIST_T3)])
def test_chain_full_rows(sv, dtype, V, dist):
    """24 requests, gamma = 3: 8 fall back at position 0, 8 at position 2, 8 are ordinary
    (rows of several chunks and tiles; V = 40001 misaligns rows, the Student-t rows leave chunks of
    negligible mass)."""
    d = inputgen.chain_inputs(24, 3, V, seed=900 + V % 97, dtype=dtype, dist=dist, scale=2.5, noise_sd=0.8,
                              temperature=np.linspace(0.6, 1.4, 24))
    _zero_residual_chain(d, range(0, 8), 0)
    _zero_residual_chain(d, range(8, 16), 2)
    print(f"[zero residual chain {dtype} V={V}]", flush=True)
    out, na, ref = run_chain(sv, d)
    assert ref["fallback"][:16].all()
    assert (ref["num_accepted"][:8] == 0).all() and (ref["num_accepted"][8:16] == 2).all()
    assert_tokens_match(out, na, ref, f"zero residual chain {dtype} V={V}")


def _tree_hand(dtype, ua2, us, lossless):
    """The oracle pin's tree: root (1/3, 1/3, 0, 1/3); node 1 drafts token 2 from an equal row;
    node 2 drafts token 0 from (1, 0, 0, 0); node 2's target row (1/2, 1/2, 0, 0)."""
    one_hot0 = np.array([0.0, NEG, NEG, NEG], np.float32)
    halves = np.array([0.0, 0.0, NEG, NEG], np.float32)
    B = len(us)
    target = np.stack([np.stack([THIRDS, np.zeros(4, np.float32), halves])] * B)
    draft = np.stack([np.stack([THIRDS, one_hot0])] * B)
    return dict(target=_as(dtype, target), draft=_as(dtype, draft),
                node_tokens=np.tile(np.array([0, 2, 0], np.int32), (B, 1)),
                parents=np.tile(np.array([-1, 0, 0], np.int32), (B, 1)),
                u_accept=np.array([[0.0, 0.5, a] for a in ua2], np.float32),
                u_sample=np.asarray(us, np.float32), temperature=np.ones(B, np.float32), max_depth=1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("lossless", [False, True])
def test_tree_hand_cases(sv, dtype, lossless):
    """Node 2 is accepted iff u < 1/3 (against the root's 1/3, kept by the lossless walk).
    Lowest-child rule: when node 2 is rejected the root is the end node and the draw falls back to
    (1/3, 1/3, 0, 1/3) at u_s[0]. Lossless walk: node 2's rejection leaves (0, 1/2, 0, 1/2).
    Cases (u for node 2, u_s[0]) -> y: (0.9, 0.3) -> 0 / 1, (0.9, 0.9) -> 3 / 3, (0.5, 0.7) -> 3 / 3,
    (0.5, 0.4) -> 1 / 1; and (0.2, -) accepts node 2, whose row (1/2, 1/2, 0, 0) gives 1 at 0.7."""
    ua2 = [0.9, 0.9, 0.2, 0.5, 0.5]
    us = [[0.3, 0.5, 0.5], [0.9, 0.5, 0.5], [0.5, 0.5, 0.7], [0.7, 0.5, 0.5], [0.4, 0.5, 0.5]]
    d = _tree_hand(dtype, ua2, us, lossless)
    print(f"[zero residual hand tree {dtype} lossless={lossless}]", flush=True)
    out, nodes, na, ref = run_tree(sv, d, lossless)
    assert_tokens_match(out, na, ref, f"hand tree {dtype}")
    assert (nodes == ref["out_nodes"]).all()
    if dtype == "f32":
        first = 1 if lossless else 0
        assert out.tolist() == [[first, -1], [3, -1], [0, 1], [3, -1], [1, -1]]
        assert ref["fallback"].tolist() == ([True] * 5 if lossless else [True, True, False, True, True])


def _zero_residual_tree(d, reqs, lossless):
    """Request b in reqs: the root's first child drafts from a row equal to the root's target row,
    with its token's logit -inf in both. Lowest-child rule: every child of the root drafts that
    token (zero target mass: all rejected), so the root is the end node and its residual against
    the first child is 0. Lossless walk: only the first child changes; its rejection keeps r."""
    neg = np.float32(NEG) if d["target"].dtype == np.float32 else np.uint16(0xFF80)
    for b in reqs:
        kids = [v for v in range(1, d["parents"].shape[1]) if d["parents"][b, v] == 0]
        c = kids[0]
        x = int(d["node_tokens"][b, c])
        d["draft"][b, c - 1] = d["target"][b, 0]
        d["target"][b, 0, x] = neg
        d["draft"][b, c - 1, x] = neg
        if not lossless:
            for v in kids[1:]:
                d["node_tokens"][b, v] = x


@pytest.mark.parametrize("lossless", [False, True])
@pytest.mark.parametrize("dtype,V", [("bf16", 30001), ("f32", 20000)])
def test_tree_full_rows(sv, lossless, dtype, V):
    d = inputgen.tree_inputs(16, V, seed=910 + V % 89, n_nodes=21, fanout=(4, 4, 1), dtype=dtype, noise_sd=0.7)
    _zero_residual_tree(d, range(0, 10), lossless)
    print(f"[zero residual tree {dtype} V={V} lossless={lossless}]", flush=True)
    out, nodes, na, ref = run_tree(sv, d, lossless)
    assert ref["fallback"][:10].all()
    assert_tokens_match(out, na, ref, f"zero residual tree {dtype} V={V}")
    same = na == ref["num_accepted"]
    assert (nodes[same] == ref["out_nodes"][same]).all()
