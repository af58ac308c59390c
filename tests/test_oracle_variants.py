"""Tree and ragged variants of the oracle, pinned by reduction to the chain, brute force
and invariants (no GPU)."""
import numpy as np
import scipy.special
import scipy.stats

import inputgen
import oracle


def _chain_as_tree(d):
    """A chain of gamma drafts is a tree with parents[v] = v-1 (node v = position v-1)."""
    B, g1, V = d["target"].shape
    N = g1
    par = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    tok = np.zeros((B, N), np.int32)
    tok[:, 1:] = d["draft_tokens"]
    ua = np.zeros((B, N), np.float32)
    ua[:, 1:] = d["u_accept"]
    return par, tok, ua


def test_chain_shaped_tree_equals_chain():
    for name, seed in (("tiny", 31), ("tiny", 32)):
        d = inputgen.make(name, seed=seed, B=64)
        d["temperature"][::5] = 0.0
        rc = oracle.verify_chain(d["target"], d["draft"], d["draft_tokens"], d["u_accept"], d["u_sample"],
                                 d["temperature"])
        par, tok, ua = _chain_as_tree(d)
        rt = oracle.verify_tree(d["target"], d["draft"], tok, par, ua, d["u_sample"], d["temperature"],
                                max_depth=4)
        assert (rt["num_accepted"] == rc["num_accepted"]).all()
        assert (rt["out_tokens"] == rc["out_tokens"]).all()
        for b in range(64):
            n = rt["num_accepted"][b]
            assert list(rt["out_nodes"][b, :n]) == list(range(1, n + 1))


def _brute_greedy_tree(target, tok, par):
    N = par.shape[0]
    amax = target.argmax(-1)
    best, best_depth = 0, 0
    for v in range(1, N):
        path, u = [], v
        while u != 0:
            path.append(u)
            u = par[u]
        if all(tok[w] == amax[par[w]] for w in path) and len(path) > best_depth:
            best, best_depth = v, len(path)
    return best, best_depth, amax[best]


def test_greedy_tree_brute_force():
    d = inputgen.tree_inputs(24, 40, seed=41, n_nodes=17, fanout=(2, 2, 3), scale=1.0, dtype="f32")
    # integer logits create argmax ties; make several drafted tokens hit the argmax
    d["target"] = np.round(d["target"])
    rng = np.random.default_rng(4)
    amax = d["target"].argmax(-1)
    for b in range(24):
        for v in range(1, 17):
            if rng.random() < 0.6:
                d["node_tokens"][b, v] = amax[b, d["parents"][b, v]]
    T = np.zeros(24, np.float32)
    r = oracle.verify_tree(d["target"], d["draft"], d["node_tokens"], d["parents"], d["u_accept"],
                           d["u_sample"], T, d["max_depth"])
    deep = 0
    for b in range(24):
        e, depth, y = _brute_greedy_tree(d["target"][b], d["node_tokens"][b], d["parents"][b])
        assert r["num_accepted"][b] == depth
        assert r["out_tokens"][b, depth] == y
        if depth:
            assert r["out_nodes"][b, depth - 1] == e
        deep += depth >= 2
    assert deep > 3


def test_tree_invariants_sampling():
    d = inputgen.tree_inputs(48, 64, seed=42, n_nodes=64, fanout=(4, 4, 3), scale=2.0, noise_sd=1.0, dtype="f32")
    r = oracle.verify_tree(d["target"], d["draft"], d["node_tokens"], d["parents"], d["u_accept"],
                           d["u_sample"], d["temperature"], d["max_depth"])
    par = d["parents"]
    lengths = []
    for b in range(48):
        n = int(r["num_accepted"][b])
        lengths.append(n)
        nodes = list(r["out_nodes"][b, :n])
        # accepted nodes form a root path
        prev = 0
        for v in nodes:
            assert par[b, v] == prev
            prev = v
        e = prev
        assert list(r["out_tokens"][b, :n]) == [d["node_tokens"][b, v] for v in nodes]
        pt = scipy.special.softmax(d["target"][b].astype(np.float64), axis=-1)
        pdr = scipy.special.softmax(d["draft"][b].astype(np.float64), axis=-1)
        kids = [c for c in range(1, 64) if par[b, c] == e]
        for c in kids:  # every child of the end node is rejected
            x = d["node_tokens"][b, c]
            assert not (d["u_accept"][b, c] * pdr[c - 1, x] < pt[e, x])
        y = int(r["out_tokens"][b, n])
        if kids:
            c = min(kids)
            assert pt[e, y] > pdr[c - 1, y]
        assert (r["out_tokens"][b, n + 1:] == -1).all()
    assert max(lengths) == 3 and min(lengths) <= 2


def test_tree_validation():
    d = inputgen.tree_inputs(6, 32, seed=43, n_nodes=10, fanout=(3, 2, 1), dtype="f32")
    bad = d["parents"].copy()
    bad[1, 4] = 7          # parent after child
    bad[2, 0] = 0          # root must have parent -1
    tok = d["node_tokens"].copy()
    tok[3, 5] = 32         # out of range
    T = d["temperature"].copy()
    T[4] = -1.0
    r = oracle.verify_tree(d["target"], d["draft"], tok, bad, d["u_accept"], d["u_sample"], T, d["max_depth"])
    assert list(r["num_accepted"][1:5]) == [-1, -1, -1, -1]
    assert r["num_accepted"][0] >= 0 and r["num_accepted"][5] >= 0
    r = oracle.verify_tree(d["target"], d["draft"], d["node_tokens"], d["parents"], d["u_accept"],
                           d["u_sample"], d["temperature"], d["max_depth"] - 1)
    assert (r["num_accepted"] == -1).all()  # depth exceeds max_depth


def _dense_to_ragged(d):
    B, g = d["draft_tokens"].shape
    V = d["target"].shape[-1]
    cu = (np.arange(B + 1) * g).astype(np.int32)
    return dict(target=d["target"].reshape(-1, V), draft=d["draft"].reshape(-1, V),
                draft_tokens=d["draft_tokens"].reshape(-1), u_accept=d["u_accept"].reshape(-1),
                u_sample=d["u_sample"].reshape(-1), temperature=d["temperature"], cu_gamma=cu)


def test_ragged_constant_gamma_equals_dense():
    d = inputgen.make("tiny", seed=51, B=96)
    d["temperature"][::4] = 0.0
    rd = oracle.verify_chain(d["target"], d["draft"], d["draft_tokens"], d["u_accept"], d["u_sample"],
                             d["temperature"])
    rg = _dense_to_ragged(d)
    rr = oracle.verify_chain(rg["target"], rg["draft"], rg["draft_tokens"], rg["u_accept"], rg["u_sample"],
                             rg["temperature"], gamma=4, cu_gamma=rg["cu_gamma"])
    assert (rr["num_accepted"] == rd["num_accepted"]).all()
    assert (rr["out_tokens"] == rd["out_tokens"]).all()
    np.testing.assert_array_equal(rr["p_t"], rd["p_t"])


def test_ragged_permutation_and_padding():
    d = inputgen.ragged_inputs(64, 0, 6, 200, seed=52, dtype="f32", scale=2.0, n_greedy=16)
    g = d["gamma_max"]
    r = oracle.verify_chain(d["target"], d["draft"], d["draft_tokens"], d["u_accept"], d["u_sample"],
                            d["temperature"], gamma=g, cu_gamma=d["cu_gamma"])
    cu = d["cu_gamma"]
    gam = np.diff(cu)
    assert (gam == 0).any() and (gam == 6).any()
    for b in range(64):
        n = r["num_accepted"][b]
        assert 0 <= n <= gam[b]
        assert (r["out_tokens"][b, n + 1:] == -1).all()
    # permute requests
    perm = np.random.default_rng(0).permutation(64)
    tgt, dft, tok, ua, us, ncu = [], [], [], [], [], [0]
    for b in perm:
        tgt.append(d["target"][cu[b] + b: cu[b + 1] + b + 1])
        us.append(d["u_sample"][cu[b] + b: cu[b + 1] + b + 1])
        dft.append(d["draft"][cu[b]: cu[b + 1]])
        tok.append(d["draft_tokens"][cu[b]: cu[b + 1]])
        ua.append(d["u_accept"][cu[b]: cu[b + 1]])
        ncu.append(ncu[-1] + gam[b])
    rp = oracle.verify_chain(np.concatenate(tgt), np.concatenate(dft), np.concatenate(tok), np.concatenate(ua),
                             np.concatenate(us), d["temperature"][perm], gamma=g,
                             cu_gamma=np.array(ncu, np.int32))
    assert (rp["num_accepted"] == r["num_accepted"][perm]).all()
    assert (rp["out_tokens"] == r["out_tokens"][perm]).all()


def test_ragged_cu_validation():
    d = inputgen.ragged_inputs(8, 1, 3, 50, seed=53, dtype="f32")
    cu = d["cu_gamma"].copy()
    cu[3] = cu[4] + 1  # request 2 would own a negative count, request 3 too many
    r = oracle.verify_chain(d["target"], d["draft"], d["draft_tokens"], d["u_accept"], d["u_sample"],
                            d["temperature"], gamma=d["gamma_max"], cu_gamma=cu)
    assert (r["num_accepted"] == -1).all()  # a malformed layout fails the whole batch
    ok = oracle.verify_chain(d["target"], d["draft"], d["draft_tokens"], d["u_accept"], d["u_sample"],
                             d["temperature"], gamma=d["gamma_max"], cu_gamma=d["cu_gamma"])
    assert (ok["num_accepted"] >= 0).all()


# Lowest-child tree rule (one reading of [Primer 考点3], tree verified in one pass): its
# output distribution on a five-node tree, derived by enumerating which nodes pass their
# tests, against the oracle's histogram over many seeded uniforms.
_PAR = (-1, 0, 0, 0, 2)   # root 0; children 1, 2, 3; node 4 under node 2


def _lowest_child_distribution(pt, pd, tok, *, tie="lowest", depth_first=True, residual_child="lowest",
                               test_row="parent"):
    """P(end node e, final token y) for the tree _PAR, by enumerating the 2^4 pass/fail outcomes.

    pt [5, V], pd [4, V] (row v-1 belongs to node v). The keyword arguments select a
    plausible mistake instead of the rule; the defaults are the rule itself."""
    N, V = pt.shape
    par = _PAR
    a = np.zeros(N)
    for v in range(1, N):
        row = pt[par[v]] if test_row == "parent" else pt[v]
        a[v] = min(1.0, row[tok[v]] / pd[v - 1, tok[v]])
    depth = [0, 1, 1, 1, 2]
    dist = np.zeros((N, V))
    for mask in range(1 << (N - 1)):
        acc = [True] + [bool(mask >> (v - 1) & 1) for v in range(1, N)]
        prob = np.prod([a[v] if acc[v] else 1.0 - a[v] for v in range(1, N)])
        kept = [v for v in range(N) if all(acc[w] for w in _path(v))]
        key = (lambda v: (-depth[v], v if tie == "lowest" else -v)) if depth_first else \
              (lambda v: (v == 0, v if tie == "lowest" else -v))
        e = min(kept, key=key)
        kids = [c for c in range(1, N) if par[c] == e]
        if kids:
            c = min(kids) if residual_child == "lowest" else max(kids)
            q = np.maximum(pt[e] - pd[c - 1], 0.0)
        else:
            q = pt[e].copy()
        dist[e] += prob * q / q.sum()
    return dist


def _path(v):
    out = []
    while v > 0:
        out.append(v)
        v = _PAR[v]
    return out


def test_lowest_child_rule_distribution():
    B, V = 200_000, 5
    rng = np.random.default_rng(20261205)
    tl = rng.normal(0.0, 1.0, (5, V)).astype(np.float32)
    dl = rng.normal(0.0, 1.0, (4, V)).astype(np.float32)
    pt = scipy.special.softmax(tl.astype(np.float64), axis=-1)
    pd = scipy.special.softmax(dl.astype(np.float64), axis=-1)
    # each node drafts the token whose acceptance probability is nearest 1/2
    tok = np.zeros(5, np.int32)
    for v in range(1, 5):
        tok[v] = np.argmin(np.abs(np.minimum(1.0, pt[_PAR[v]] / pd[v - 1]) - 0.5))
    expect = _lowest_child_distribution(pt, pd, tok)
    a = [min(1.0, pt[_PAR[v], tok[v]] / pd[v - 1, tok[v]]) for v in range(1, 5)]
    assert all(0.1 < x < 0.95 for x in a), a   # every branch of the rule is exercised
    r = oracle.verify_tree(np.broadcast_to(tl, (B, 5, V)).copy(), np.broadcast_to(dl, (B, 4, V)).copy(),
                           np.broadcast_to(tok, (B, 5)).copy(), np.broadcast_to(np.int32(_PAR), (B, 5)).copy(),
                           rng.random((B, 5), dtype=np.float32), rng.random((B, 5), dtype=np.float32),
                           np.ones(B, np.float32), max_depth=2)
    n = r["num_accepted"]
    e = np.where(n > 0, r["out_nodes"][np.arange(B), np.maximum(n - 1, 0)], 0)
    y = r["out_tokens"][np.arange(B), n]
    obs = np.zeros((5, V))
    np.add.at(obs, (e, y), 1)
    # the emitted drafted tokens are the nodes on the root path of e
    for v in range(1, 5):
        sel = e == v
        path = _path(v)[::-1]
        assert (r["out_tokens"][sel][:, :len(path)] == tok[path]).all()

    def chi2(dist):
        """Pearson statistic and degrees of freedom; infinite when a token the distribution
        gives no mass was drawn."""
        exp = B * dist.reshape(-1)
        m = exp > 0
        if obs.reshape(-1)[~m].sum() > 0:
            return np.inf, int(m.sum()) - 1
        return ((obs.reshape(-1)[m] - exp[m]) ** 2 / exp[m]).sum(), int(m.sum()) - 1

    stat, df = chi2(expect)
    assert scipy.stats.chi2.sf(stat, df) > 1e-3, (stat, df)
    # the same counts reject each plausible mistake in the rule
    crit = scipy.stats.chi2.isf(1e-6, df)
    for kw in (dict(residual_child="highest"), dict(tie="highest"), dict(depth_first=False),
               dict(test_row="own")):
        bad, _ = chi2(_lowest_child_distribution(pt, pd, tok, **kw))
        assert bad > crit, (kw, bad, crit)
