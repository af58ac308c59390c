"""GPU parity of the lossless multi-candidate tree verification
(spec_verify_tree_lossless through the C ABI) against the oracle's
verify_tree_lossless on the same seeded trees and uniforms. Bar as for the
other verify paths (tests/_parity.py): tokens, accepted counts and the path's
nodes equal the oracle's, apart from near-ties the oracle flags."""
import numpy as np
import pytest
import scipy.special
import scipy.stats

import inputgen
import oracle
from _parity import assert_tokens_match, device_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    import torch

    import rejection_sampling_verify_spec_amd as m
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    return m


def _check(sv, d, label):
    import torch
    print(f"[{label}] target {d['target'].shape}", flush=True)
    t = device_inputs(d)
    out, nodes, na = sv.verify_tree_lossless(t["target"], t["draft"], t["node_tokens"], t["parents"],
                                             t["u_accept"], t["u_sample"], t["temperature"], d["max_depth"])
    torch.cuda.synchronize()
    out, nodes, na = out.cpu().numpy(), nodes.cpu().numpy(), na.cpu().numpy()
    ref = oracle.verify_tree_lossless(d["target"], d["draft"], d["node_tokens"], d["parents"], d["u_accept"],
                                      d["u_sample"], d["temperature"], d["max_depth"])
    assert_tokens_match(out, na, ref, label)
    same = na == ref["num_accepted"]
    assert (nodes[same] == ref["out_nodes"][same]).all()
    return out, nodes, na


def test_small_trees(sv):
    d = inputgen.tree_inputs(16, 3000, seed=71, n_nodes=21, fanout=(4, 4, 1), dtype="f32", noise_sd=1.5)
    _, _, na = _check(sv, d, "small f32")
    assert (na >= 0).all()


def test_tree_full_size(sv):
    """B=32, 64-node trees (4, 4, 2-3 children), V=152064 bf16: the measured workload."""
    _, _, na = _check(sv, inputgen.make("tree"), "tree full")
    assert (na >= 0).all()


def test_tree_variants(sv):
    _check(sv, inputgen.tree_inputs(32, 30000, seed=72, iid_draft=True), "iid drafts (many rejected siblings)")
    d = inputgen.tree_inputs(24, 5000, seed=73, dtype="f32", noise_sd=1.5, temperature=0.7)
    d["temperature"][::3] = 0.0
    _check(sv, d, "mixed greedy")
    _check(sv, inputgen.tree_inputs(8, 999, seed=74, n_nodes=1, fanout=(), dtype="f32"), "root only")
    _check(sv, inputgen.tree_inputs(8, 4097, seed=75, n_nodes=200, fanout=(5, 5, 7), dtype="bf16", noise_sd=2.0),
           "200 nodes, ragged V")
    _check(sv, inputgen.tree_inputs(4, 2049, seed=76, n_nodes=1024, fanout=(1023,), dtype="bf16", noise_sd=3.0),
           "1023 siblings")
    _check(sv, inputgen.tree_inputs(8, 600_001, seed=80, n_nodes=21, fanout=(4, 4, 1), dtype="bf16", noise_sd=1.5),
           "V=600001")
    # fp32 rows of 782 segments over 96 waves: each wave keeps 6 segments' residual in LDS, the rest
    # in the workspace
    _check(sv, inputgen.tree_inputs(32, 200_003, seed=82, n_nodes=21, fanout=(4, 4, 1), dtype="f32",
                                    iid_draft=True), "f32 V=200003, iid drafts")
    bad = inputgen.tree_inputs(6, 100, seed=77, n_nodes=10, fanout=(3, 2, 1), dtype="f32")
    bad["parents"] = bad["parents"].copy()
    bad["parents"][2, 5] = 7
    bad["u_accept"] = bad["u_accept"].copy()
    bad["u_accept"][4, 3] = 1.0
    _, _, na = _check(sv, bad, "bad parents / uniform")
    assert na[2] == -1 and na[4] == -1 and (np.delete(na, [2, 4]) >= 0).all()


def test_tiny_vocab(sv):
    """Rows shorter than one 16-byte vector or one segment (V = 1 .. 17, bf16 rows off the 16-byte
    grid), every fourth tree greedy."""
    for V in (1, 3, 7, 9, 17):
        for dtype in ("f32", "bf16"):
            d = inputgen.tree_inputs(12, V, seed=900 + V, n_nodes=10, fanout=(3, 2, 1), dtype=dtype, noise_sd=1.0,
                                     temperature=0.8)
            d["temperature"][::4] = 0.0
            _, _, na = _check(sv, d, f"lossless V={V} {dtype}")
            assert (na >= 0).all()


def test_teams_loop_over_requests(sv):
    """More requests than resident teams (one workgroup per team at this batch size): a team walks
    several requests in turn, reusing its shared state and its LDS residual; mixed dtypes and
    temperatures, greedy requests among them."""
    d = inputgen.tree_inputs(600, 1500, seed=83, n_nodes=21, fanout=(4, 4, 1), dtype="bf16", noise_sd=1.0,
                             temperature=0.9)
    d["temperature"][::5] = 0.0
    _, _, na = _check(sv, d, "600 requests bf16")
    assert (na >= 0).all()
    d = inputgen.tree_inputs(520, 2100, seed=84, n_nodes=21, fanout=(4, 4, 1), dtype="f32", iid_draft=True)
    _, _, na = _check(sv, d, "520 requests f32, iid drafts")
    assert (na >= 0).all()


def test_temperature_extremes(sv):
    """The walk over temperatures from 1e-30 to 1e6 and over logits near the fp32 range."""
    d = inputgen.tree_inputs(32, 3000, seed=79, n_nodes=21, fanout=(4, 4, 1), dtype="f32", noise_sd=1.0,
                             temperature=np.geomspace(1e-30, 1e6, 32).astype(np.float32))
    _, _, na = _check(sv, d, "T extremes")
    assert (na >= 0).all()
    d = inputgen.tree_inputs(8, 500, seed=81, n_nodes=10, fanout=(3, 2, 1), dtype="f32", scale=1e37, noise_sd=0.0,
                             temperature=0.05)
    _check(sv, d, "overflowing offsets")


def test_chain_shaped_tree_equals_chain(sv):
    import torch
    d = inputgen.chain_inputs(32, 4, 3000, seed=78, dtype="bf16", scale=2.0, noise_sd=1.2)
    d["temperature"][::4] = 0.0
    B, N = 32, 5
    t = device_inputs(d)
    oc, nc = sv.verify_chain(t["target"], t["draft"], t["draft_tokens"], t["u_accept"], t["u_sample"],
                             t["temperature"])
    par = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    tok = np.zeros((B, N), np.int32)
    tok[:, 1:] = d["draft_tokens"]
    ua = np.zeros((B, N), np.float32)
    ua[:, 1:] = d["u_accept"]
    td = dict(target=d["target"], draft=d["draft"], node_tokens=tok, parents=par, u_accept=ua,
              u_sample=d["u_sample"], temperature=d["temperature"], max_depth=4)
    out, _, na = _check(sv, td, "chain-shaped")
    torch.cuda.synchronize()
    assert np.array_equal(na, nc.cpu().numpy()) and np.array_equal(out, oc.cpu().numpy())


def test_first_token_follows_the_root_target_row(sv):
    """200,000 one-level trees (root + 3 children, V = 16) with each child's token drawn from its own
    draft row: the emitted first token follows the root's target row (chi-square), bit-equal to the
    oracle."""
    rng = np.random.default_rng(79)
    n, V, k = 200_000, 16, 3
    tgt = rng.normal(0.0, 1.5, size=(k + 1, V)).astype(np.float32)
    dft = np.stack([tgt[0] + rng.normal(0.0, 2.0, V) for _ in range(k)]).astype(np.float32)
    q = scipy.special.softmax(dft.astype(np.float64), axis=1)
    tok = np.zeros((n, k + 1), np.int32)
    u = rng.random((n, k))
    for c in range(k):
        tok[:, c + 1] = np.minimum((np.cumsum(q[c])[None, :] <= u[:, c:c + 1]).sum(axis=1), V - 1)
    d = dict(target=np.ascontiguousarray(np.broadcast_to(tgt, (n, k + 1, V))),
             draft=np.ascontiguousarray(np.broadcast_to(dft, (n, k, V))), node_tokens=tok,
             parents=np.ascontiguousarray(np.broadcast_to(np.int32([-1] + [0] * k), (n, k + 1))),
             u_accept=inputgen.uniform24(79, inputgen.S_UACC, n * (k + 1)).reshape(n, k + 1),
             u_sample=inputgen.uniform24(79, inputgen.S_USAMP, n * (k + 1)).reshape(n, k + 1),
             temperature=np.ones(n, np.float32), max_depth=1)
    out, _, na = _check(sv, d, "chi-square")
    p = scipy.special.softmax(tgt[0].astype(np.float64))
    counts = np.bincount(out[:, 0], minlength=V)
    stat = ((counts - n * p) ** 2 / (n * p)).sum()
    assert scipy.stats.chi2.sf(stat, V - 1) > 1e-3
    assert 0.2 < (na > 0).mean() < 0.98


@pytest.mark.parametrize("dtype,noise", [("f32", 0.01), ("f32", 0.2), ("bf16", 0.05), ("bf16", 0.2)])
def test_near_identical_drafts(sv, dtype, noise):
    """Draft rows within a small noise of their parent's target row, with the first children of the
    root and of each depth-1 node forced towards rejection (u near 1): the residual left by a rejected
    sibling is small (about the rows' total variation), so its support and normalisation depend on the
    exact ratio of the two rows' normalisers, not on an estimate of it."""
    d = inputgen.near_identical_trees(48, 30000, 81 + int(noise * 100), dtype=dtype, noise_sd=noise)
    _, _, na = _check(sv, d, f"near-identical {dtype} sd={noise}")
    assert (na >= 0).all()
