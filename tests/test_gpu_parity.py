"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same
seeded inputs (bar documented in tests/_parity.py)."""
import numpy as np
import pytest

import inputgen
import oracle
from _parity import assert_probs_match, assert_tokens_match, device_inputs, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    import torch

    import rejection_sampling_verify_spec_amd as m
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    return m


def _sync():
    import torch
    torch.cuda.synchronize()


def run_chain(sv, d):
    t = device_inputs(d)
    out, na, dg = sv.verify_chain(t["target"], t["draft"], t["draft_tokens"], t["u_accept"], t["u_sample"],
                                  t["temperature"], diag=True)
    _sync()
    return out.cpu().numpy(), na.cpu().numpy(), dg.cpu().numpy()


def check_chain(sv, d, label):
    print(f"[{label}] target {d['target'].shape} {d['target'].dtype}", flush=True)
    out, na, dg = run_chain(sv, d)
    ref = oracle.verify_chain(d["target"], d["draft"], d["draft_tokens"], d["u_accept"], d["u_sample"],
                              d["temperature"])
    nm = assert_tokens_match(out, na, ref, label)
    B, g = d["draft_tokens"].shape
    valid = np.repeat((ref["num_accepted"] >= 0) & (d["temperature"] > 0), g)
    tol = 1e-5 if d["target"].dtype == np.float32 else 2e-3
    if g:
        assert_probs_match(dg.reshape(-1, 2), ref, valid, tol, label)
    return out, na, ref, nm


@pytest.mark.parametrize("name", ["tiny", "mid"])
def test_chain_workloads(sv, name):
    check_chain(sv, inputgen.make(name), name)


def test_chain_large_full_size(sv):
    """B=256, gamma=5, V=128256, bf16 Student-t logits (the measured workload)."""
    check_chain(sv, inputgen.make("large"), "large")


@pytest.mark.parametrize("dtype,V,seed", [("f32", 20000, 1), ("bf16", 20000, 2), ("bf16", 40001, 3),
                                          ("f32", 9999, 4), ("bf16", 16385, 5)])
def test_chain_multi_chunk_ragged_tail(sv, dtype, V, seed):
    """Several row chunks and sampling tiles with a ragged tail; odd V misaligns rows."""
    d = inputgen.chain_inputs(48, 4, V, seed=100 + seed, dtype=dtype, scale=2.5, noise_sd=0.8,
                              temperature=np.linspace(0.3, 1.8, 48))
    d["temperature"][::7] = 0.0
    check_chain(sv, d, f"{dtype} V={V}")


def test_chain_edge_shapes(sv):
    for (B, g, V) in [(1, 0, 1), (3, 0, 50), (5, 1, 1), (4, 3, 7), (2, 2, 9), (7, 1, 8193), (1, 8, 300),
                      (6, 130, 40)]:
        for dtype in ("f32", "bf16"):
            d = inputgen.chain_inputs(B, g, V, seed=B * 1000 + g * 10 + V, dtype=dtype, scale=1.5, noise_sd=0.6,
                                      temperature=0.9)
            check_chain(sv, d, f"B={B} g={g} V={V} {dtype}")


@pytest.mark.parametrize("dtype,V", [("bf16", 600_001), ("f32", 300_007)])
def test_chain_rows_of_many_tiles(sv, dtype, V):
    """Rows of more than 256 sampling tiles, where the pick reads the tile records from memory instead
    of staging them in LDS: residual and bonus draws, every fifth request greedy."""
    d = inputgen.chain_inputs(16, 3, V, seed=V % 1000, dtype=dtype, scale=2.5, noise_sd=0.8,
                              temperature=np.linspace(0.5, 1.5, 16))
    d["temperature"][::5] = 0.0
    _, na, _, _ = check_chain(sv, d, f"{dtype} V={V}")
    assert ((na >= 0) & (na < 3)).any() and (na == 3).any()  # residual and bonus draws both happen


def test_chain_beyond_2_31_logits(sv):
    """One call over more than 2^31 target logits: B=112, gamma=0, V=20,000,003 bf16 (2.24e9 logits,
    4.5 GB; the last rows lie wholly past logit 2^31 and byte 2^32), with V above 2^24, so row offsets
    need 64-bit arithmetic and in-row indices exact integer arithmetic. Odd requests are greedy
    (argmax), even ones draw the bonus token; several drawn tokens lie above 2^24."""
    B, V = 112, 20_000_003
    d = inputgen.chain_inputs(B, 0, V, seed=4343, dtype="bf16", scale=2.5, noise_sd=0.8,
                              temperature=np.tile(np.float32([1.0, 0.0]), B // 2))
    out, na, ref, _ = check_chain(sv, d, "2^31+ logits")
    assert (na == 0).all() and (out[:, 0] >= 2 ** 24).sum() >= 1


def test_temperature_extremes(sv):
    d = inputgen.chain_inputs(32, 3, 3000, seed=7, dtype="f32", scale=3.0, noise_sd=0.5,
                              temperature=np.geomspace(1e-30, 1e6, 32))
    check_chain(sv, d, "T extremes")
    # logits so large that |max * log2(e)/T| leaves the fp32 range
    d = inputgen.chain_inputs(8, 2, 500, seed=8, dtype="f32", scale=1e37, noise_sd=0.0, temperature=0.05)
    check_chain(sv, d, "overflowing offsets")


def test_residual_undecided_band(sv, monkeypatch):
    """Draft almost equal to the target with forced rejections: many tokens lie in the band where the
    fp32 estimate of Z_t/Z_d cannot decide the residual's sign, so tiles are recomputed token by token;
    the switch SPECVERIFY_FORCE_EXACT_RESIDUAL=1 recomputes every tile."""
    for dtype in ("f32", "bf16"):
        d = inputgen.chain_inputs(64, 3, 30000, seed=71, dtype=dtype, scale=2.0, noise_sd=1e-3 if dtype == "f32"
                                  else 0.05)
        d["u_accept"][:, 1] = 0.9999
        out, na, ref, _ = check_chain(sv, d, f"near-identical draft {dtype}")
        assert (na == 1).sum() > 10
        monkeypatch.setenv("SPECVERIFY_FORCE_EXACT_RESIDUAL", "1")
        check_chain(sv, d, f"near-identical draft {dtype}, every tile exact")
        monkeypatch.delenv("SPECVERIFY_FORCE_EXACT_RESIDUAL")
    monkeypatch.setenv("SPECVERIFY_FORCE_EXACT_RESIDUAL", "1")
    check_chain(sv, inputgen.make("mid"), "mid, every tile exact")


def test_request_errors(sv):
    base = inputgen.make("tiny", seed=11, B=16)
    d = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in base.items()}
    d["temperature"][1] = np.nan
    d["temperature"][2] = -0.5
    d["temperature"][3] = 1e-40
    d["draft_tokens"][4, 2] = 256
    d["u_accept"][5, 0] = 1.0
    d["u_sample"][6, 4] = np.nan
    d["target"][7, 3, 100] = np.nan
    d["target"][8, 0, 5] = np.inf
    d["draft"][9, 1, :] = -np.inf
    d["target"][10, 2, :200] = -np.inf  # allowed: finite values remain
    d["temperature"][11] = 0.0
    d["draft"][11] = np.nan  # greedy requests do not read draft rows
    d["draft"][12, 3, 0] = np.nan
    out, na, ref, _ = check_chain(sv, d, "errors")
    assert list(na[1:10]) == [-1] * 9 and na[12] == -1
    assert na[10] >= 0 and na[11] >= 0 and na[0] >= 0
    assert (out[na == -1] == -1).all()


def test_bonus_negligible_chunks(sv):
    """Near one-hot bonus rows: every chunk of the streaming pass but the last holds masses far below
    2^-50 of the row maximum, so the draw takes those chunks' mass from the streaming pass instead of
    reading them again. u_sample = 0 puts u*S at 0, i.e. on the first token with positive mass, which
    lies inside such a chunk: the pick then walks the chunk token by token. Other uniforms land on the
    maximum. Row maxima sit in the last chunk; drafts equal the target, so every draft is accepted."""
    rng = np.random.default_rng(21)
    B, g, V = 24, 2, 70000
    for dtype in ("f32", "bf16"):
        tgt = np.full((B, g + 1, V), -40.0, np.float32)
        tgt += rng.integers(0, 4, size=tgt.shape).astype(np.float32) * 0.25
        tgt[:, :, V - 7] = 0.0
        tgt[:, :, V - 3] = -1.5
        T = np.full(B, 1.0, np.float32)
        T[1::4] = 0.9
        arr = tgt if dtype == "f32" else (tgt.view(np.uint32) >> 16).astype(np.uint16)
        d = dict(target=arr, draft=arr[:, :g].copy(), draft_tokens=np.full((B, g), V - 7, np.int32),
                 u_accept=rng.random((B, g)).astype(np.float32) * 0.99,
                 u_sample=np.zeros((B, g + 1), np.float32), temperature=T)
        d["u_sample"][B // 2:, g] = rng.random(B - B // 2).astype(np.float32)
        out, na, ref, _ = check_chain(sv, d, f"negligible chunks {dtype}")
        assert (na == g).all()
        assert (out[: B // 2, g] < V - 7).all()  # drawn inside a chunk that was not read again


def test_greedy_ties(sv):
    """Integer logits: many tied maxima; the lowest index must win everywhere."""
    rng = np.random.default_rng(5)
    B, g, V = 64, 4, 20000
    tgt = rng.integers(-2, 3, size=(B, g + 1, V)).astype(np.float32)
    amax = tgt.argmax(-1)
    tok = amax[:, :g].copy()
    tok[::3, 1] = (tok[::3, 1] + 1) % V
    tok[1::4, 3] = V - 1 - tok[1::4, 3]
    d = dict(target=tgt, draft=np.zeros((B, g, V), np.float32), draft_tokens=tok.astype(np.int32),
             u_accept=np.zeros((B, g), np.float32), u_sample=np.zeros((B, g + 1), np.float32),
             temperature=np.zeros(B, np.float32))
    check_chain(sv, d, "greedy ties f32")
    bits = (tgt.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    d["target"] = bits
    d["draft"] = np.zeros((B, g, V), np.uint16)
    check_chain(sv, d, "greedy ties bf16")
    # odd V: rows start off 16-byte boundaries, so ties span head, vector and tail elements
    V2 = 4099
    t2 = rng.integers(-1, 2, size=(B, g + 1, V2)).astype(np.float32)
    t2[:, :, :3] = 1.0
    t2[:, :, V2 - 2:] = 1.0
    a2 = t2.argmax(-1)
    d2 = dict(target=(t2.view(np.uint32) >> 16).astype(np.uint16), draft=np.zeros((B, g, V2), np.uint16),
              draft_tokens=a2[:, :g].astype(np.int32), u_accept=np.zeros((B, g), np.float32),
              u_sample=np.zeros((B, g + 1), np.float32), temperature=np.zeros(B, np.float32))
    d2["draft_tokens"][::2, 2] = 5
    check_chain(sv, d2, "greedy ties misaligned bf16")


def test_row_softmax_stats(sv):
    import torch
    rng = np.random.default_rng(3)
    for dtype, V in (("f32", 1), ("f32", 33), ("bf16", 7), ("bf16", 4097), ("f32", 32000), ("bf16", 151937)):
        rows = 40
        x = (rng.standard_t(3, size=(rows, V)) * 3).astype(np.float32)
        x[1, V // 2] = x[1].max() + 1
        x[2, :] = -np.inf
        x[2, V - 1] = 1.0
        x[3, 0] = np.nan
        x[4, V // 3] = np.inf
        if V > 2:
            x[5, 1] = x[5, V - 1] = x[5].max() + 2  # tie
        x[6, :] = -np.inf
        T = np.where(np.arange(rows) % 2 == 0, 0.0, np.linspace(0.2, 3.0, rows)).astype(np.float32)
        arr = x if dtype == "f32" else (x.view(np.uint32) >> 16).astype(np.uint16)
        if dtype == "bf16":
            arr = np.where(np.isnan(x), np.uint16(0x7fc0), arr).astype(np.uint16)
        mx, lz, am = sv.row_softmax_stats(to_dev(arr), torch.from_numpy(T).cuda())
        _sync()
        mx, lz, am = mx.cpu().numpy(), lz.cpu().numpy(), am.cpu().numpy()
        ref = oracle.row_stats(arr, T)
        for r in range(rows):
            if not ref["valid"][r]:
                assert np.isnan(mx[r]), (dtype, V, r)
                continue
            assert mx[r] == np.float32(ref["max"][r]), (dtype, V, r)
            if T[r] == 0:
                assert am[r] == ref["argmax"][r], (dtype, V, r)
            else:
                assert abs(lz[r] - ref["logz"][r]) <= 2e-5 * max(1.0, abs(ref["logz"][r])), (dtype, V, r)


def _ragged_check(sv, d, label):
    print(f"[{label}] rows {d['target'].shape}", flush=True)
    t = device_inputs(d)
    out, na, dg = sv.verify_ragged(t["target"], t["draft"], t["cu_gamma"], d["total_draft"], t["draft_tokens"],
                                   t["u_accept"], t["u_sample"], t["temperature"], d["gamma_max"], diag=True)
    _sync()
    out, na, dg = out.cpu().numpy(), na.cpu().numpy(), dg.cpu().numpy()
    ref = oracle.verify_chain(d["target"], d["draft"], d["draft_tokens"], d["u_accept"], d["u_sample"],
                              d["temperature"], gamma=d["gamma_max"], cu_gamma=d["cu_gamma"])
    assert_tokens_match(out, na, ref, label)
    db = np.repeat(np.arange(len(d["temperature"])), np.diff(d["cu_gamma"]))
    valid = (ref["num_accepted"][db] >= 0) & (d["temperature"][db] > 0)
    if d["total_draft"]:
        assert_probs_match(dg[:d["total_draft"]], ref, valid, 1e-5 if d["target"].dtype == np.float32 else 2e-3,
                           label)
    return out, na


def test_ragged_small(sv):
    d = inputgen.ragged_inputs(96, 0, 8, 12000, seed=21, dtype="bf16", n_greedy=24)
    _ragged_check(sv, d, "ragged small bf16")
    d = inputgen.ragged_inputs(64, 1, 5, 5001, seed=22, dtype="f32", n_greedy=16)
    _ragged_check(sv, d, "ragged small f32")


def test_ragged_full_size(sv):
    """B=1024, gamma_b in 1..8, V=151936, 256 greedy requests."""
    _ragged_check(sv, inputgen.make("ragged"), "ragged full")


def test_ragged_mid_batches(sv):
    """600 requests (gamma_b 0..8, odd V, greedy requests; more tail workgroups than are resident at
    once) and 256 (fp32)."""
    d = inputgen.ragged_inputs(600, 0, 8, 3001, seed=24, dtype="bf16", n_greedy=100)
    _ragged_check(sv, d, "ragged 600 bf16")
    d = inputgen.ragged_inputs(256, 1, 6, 2000, seed=25, dtype="f32", n_greedy=40)
    _ragged_check(sv, d, "ragged 256 f32")


def test_ragged_bad_layout_large_batch(sv):
    """A malformed cu_gamma in a batch of 300: every request fails (-1)."""
    d = inputgen.ragged_inputs(300, 1, 4, 300, seed=26, dtype="f32")
    d["cu_gamma"] = d["cu_gamma"].copy()
    d["cu_gamma"][150] = d["cu_gamma"][151] + 3
    t = device_inputs(d)
    out, na = sv.verify_ragged(t["target"], t["draft"], t["cu_gamma"], d["total_draft"], t["draft_tokens"],
                               t["u_accept"], t["u_sample"], t["temperature"], d["gamma_max"])
    _sync()
    assert (na.cpu().numpy() == -1).all() and (out.cpu().numpy() == -1).all()


def test_ragged_bad_layout(sv):
    d = inputgen.ragged_inputs(16, 1, 4, 300, seed=23, dtype="f32")
    d["cu_gamma"] = d["cu_gamma"].copy()
    d["cu_gamma"][5] = d["cu_gamma"][6] + 1
    t = device_inputs(d)
    out, na = sv.verify_ragged(t["target"], t["draft"], t["cu_gamma"], d["total_draft"], t["draft_tokens"],
                               t["u_accept"], t["u_sample"], t["temperature"], d["gamma_max"])
    _sync()
    assert (na.cpu().numpy() == -1).all() and (out.cpu().numpy() == -1).all()


def test_tree_tiny_vocab(sv):
    """Rows shorter than one 16-byte vector or one tile (V = 1 .. 17, bf16 rows off the 16-byte grid),
    every fourth tree greedy."""
    for V in (1, 3, 7, 9, 17):
        for dtype in ("f32", "bf16"):
            d = inputgen.tree_inputs(12, V, seed=900 + V, n_nodes=10, fanout=(3, 2, 1), dtype=dtype, noise_sd=1.0,
                                     temperature=0.8)
            d["temperature"][::4] = 0.0
            na = _tree_check(sv, d, f"tree V={V} {dtype}")
            assert (na >= 0).all()


def test_dense_equals_ragged(sv):
    import torch
    d = inputgen.chain_inputs(40, 5, 7000, seed=31, dtype="bf16", scale=3.0, noise_sd=1.0)
    d["temperature"][::5] = 0.0
    t = device_inputs(d)
    o1, n1 = sv.verify_chain(t["target"], t["draft"], t["draft_tokens"], t["u_accept"], t["u_sample"],
                             t["temperature"])
    cu = torch.arange(0, 41 * 5, 5, dtype=torch.int32, device="cuda")
    o2, n2 = sv.verify_ragged(t["target"].reshape(-1, 7000), t["draft"].reshape(-1, 7000), cu, 200,
                              t["draft_tokens"].reshape(-1), t["u_accept"].reshape(-1), t["u_sample"].reshape(-1),
                              t["temperature"], 5)
    _sync()
    assert torch.equal(o1, o2) and torch.equal(n1, n2)


def _tree_check(sv, d, label):
    print(f"[{label}] target {d['target'].shape}", flush=True)
    t = device_inputs(d)
    out, nodes, na = sv.verify_tree(t["target"], t["draft"], t["node_tokens"], t["parents"], t["u_accept"],
                                    t["u_sample"], t["temperature"], d["max_depth"])
    _sync()
    out, nodes, na = out.cpu().numpy(), nodes.cpu().numpy(), na.cpu().numpy()
    ref = oracle.verify_tree(d["target"], d["draft"], d["node_tokens"], d["parents"], d["u_accept"], d["u_sample"],
                             d["temperature"], d["max_depth"])
    assert_tokens_match(out, na, ref, label)
    ok = (na == ref["num_accepted"])
    assert (nodes[ok] == ref["out_nodes"][ok]).all()
    return na


def test_tree_full_size(sv):
    """B=32, 64-node trees, V=152064, draft of node v = target of its parent + N(0, 0.7)."""
    _tree_check(sv, inputgen.make("tree"), "tree full")


def test_tree_variants(sv):
    na = _tree_check(sv, inputgen.tree_inputs(32, 30000, seed=41, iid_draft=True), "tree iid drafts")
    assert (na < 3).any()
    d = inputgen.tree_inputs(24, 5000, seed=42, dtype="f32", noise_sd=1.5, temperature=0.7)
    d["temperature"][::3] = 0.0
    _tree_check(sv, d, "tree mixed greedy")
    d = inputgen.tree_inputs(8, 999, seed=43, n_nodes=1, fanout=(), dtype="f32")
    _tree_check(sv, d, "tree root only")
    d = inputgen.tree_inputs(8, 2000, seed=44, n_nodes=200, fanout=(5, 5, 7), dtype="bf16", noise_sd=2.0)
    _tree_check(sv, d, "tree 200 nodes")
    d = inputgen.tree_inputs(8, 600_001, seed=80, n_nodes=21, fanout=(4, 4, 1), dtype="bf16", noise_sd=1.5)
    _tree_check(sv, d, "tree V=600001 (more than 256 sampling tiles per row)")
    bad = inputgen.tree_inputs(6, 100, seed=45, n_nodes=10, fanout=(3, 2, 1), dtype="f32")
    bad["parents"] = bad["parents"].copy()
    bad["parents"][2, 5] = 7
    na = _tree_check(sv, bad, "tree bad parents")
    assert na[2] == -1 and (np.delete(na, 2) >= 0).all()


def test_tree_temperature_extremes(sv):
    """Lowest-child tree rule over temperatures from 1e-30 to 1e6 and over logits near the fp32
    range (|max * log2(e)/T| far beyond 2^22)."""
    d = inputgen.tree_inputs(32, 3000, seed=46, n_nodes=21, fanout=(4, 4, 1), dtype="f32", noise_sd=1.0,
                             temperature=np.geomspace(1e-30, 1e6, 32).astype(np.float32))
    _tree_check(sv, d, "tree T extremes")
    d = inputgen.tree_inputs(8, 500, seed=47, n_nodes=10, fanout=(3, 2, 1), dtype="f32", scale=1e37, noise_sd=0.0,
                             temperature=0.05)
    _tree_check(sv, d, "tree overflowing offsets")


def test_chain_shaped_tree_equals_chain(sv):
    d = inputgen.chain_inputs(32, 4, 3000, seed=51, dtype="bf16", scale=2.0, noise_sd=1.2)
    d["temperature"][::4] = 0.0
    out_c, na_c, _ = run_chain(sv, d)
    B, N = 32, 5
    par = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    tok = np.zeros((B, N), np.int32)
    tok[:, 1:] = d["draft_tokens"]
    ua = np.zeros((B, N), np.float32)
    ua[:, 1:] = d["u_accept"]
    td = dict(target=d["target"], draft=d["draft"], node_tokens=tok, parents=par, u_accept=ua,
              u_sample=d["u_sample"], temperature=d["temperature"], max_depth=4)
    na_t = _tree_check(sv, td, "chain-shaped tree")
    assert (na_t == na_c).all()


def test_determinism(sv):
    d = inputgen.make("large", seed=61, B=32)
    a = run_chain(sv, d)
    b = run_chain(sv, d)
    for x, y in zip(a, b):
        assert np.array_equal(x, y, equal_nan=True)


def test_lossless_chi_square_on_gpu(sv):
    """[Primer 考点2] identity on the GPU: 10^6 requests at V=16; the emitted token at
    position 0 follows p_target of that position."""
    import scipy.special
    import scipy.stats
    rng = np.random.default_rng(100)
    t = rng.normal(0, 1.0, size=(2, 16)).astype(np.float32)
    dr = (t[:1] + rng.normal(0, 1.0, size=(1, 16))).astype(np.float32)
    B = 1_000_000
    target = np.ascontiguousarray(np.broadcast_to(t, (B, 2, 16)))
    draft = np.ascontiguousarray(np.broadcast_to(dr, (B, 1, 16)))
    tok = inputgen.sample_tokens(101, draft.reshape(-1, 16), np.ones(B, np.float32), np.arange(B)).reshape(B, 1)
    d = dict(target=target, draft=draft, draft_tokens=tok, u_accept=inputgen.uniform24(102, 5, B).reshape(B, 1),
             u_sample=inputgen.uniform24(102, 6, 2 * B).reshape(B, 2), temperature=np.ones(B, np.float32))
    out, na, _ = run_chain(sv, d)
    counts = np.bincount(out[:, 0], minlength=16)
    p = scipy.special.softmax(t[0].astype(np.float64))
    stat = ((counts - B * p) ** 2 / (B * p)).sum()
    assert scipy.stats.chi2.sf(stat, 15) > 1e-3
    ref = oracle.verify_chain(target, draft, tok, d["u_accept"], d["u_sample"], d["temperature"])
    assert_tokens_match(out, na, ref, "chi-square batch")
