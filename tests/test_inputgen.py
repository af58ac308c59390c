"""The seeded input generator: determinism, known-answer values, distributions (no GPU)."""
import numpy as np
import scipy.special
import scipy.stats

import inputgen


def test_philox_known_answers():
    """Philox4x32-10 known-answer vectors published with the Random123 library."""
    kat = [
        ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
        ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
        ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
         [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
    ]
    for ctr, key, out in kat:
        assert list(inputgen.philox4x32_10(ctr, key)) == out


def test_determinism_and_seed_sensitivity():
    a = inputgen.make("tiny")
    b = inputgen.make("tiny")
    c = inputgen.make("tiny", seed=2)
    for k in ("target", "draft", "draft_tokens", "u_accept", "u_sample"):
        assert a[k].tobytes() == b[k].tobytes()
        assert a[k].tobytes() != c[k].tobytes()


def test_uniforms_grid_and_moments():
    u = inputgen.uniform24(3, 5, 2_000_000)
    assert u.min() >= 0 and u.max() <= 1 - 2 ** -24
    assert np.all(u * 2 ** 24 == np.round(u * 2 ** 24))
    assert abs(u.mean() - 0.5) < 1e-3
    assert scipy.stats.kstest(u[:200_000], "uniform").pvalue > 1e-3


def test_normal_and_student_t():
    z = inputgen.normal(4, 1, 1_000_000)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3
    assert scipy.stats.kstest(z[:200_000], "norm").pvalue > 1e-3
    t = inputgen.logit_rows(5, 200_000, np.array([0]), dist=inputgen.DIST_T3, scale=1.0)[0].astype(np.float64)
    assert scipy.stats.kstest(t, scipy.stats.t(3).cdf).pvalue > 1e-3


def test_bf16_round_to_nearest_even():
    x = inputgen.logit_rows(6, 4096, np.array([0]), scale=3.0, dtype="f32")[0]
    b = inputgen.logit_rows(6, 4096, np.array([0]), scale=3.0, dtype="bf16")[0]
    dec = (b.astype(np.uint32) << 16).view(np.float32)
    # the nearest bf16 is within half a bf16 ulp
    ulp = np.spacing(np.abs(dec).astype(np.float32)) * 2 ** 16
    assert np.all(np.abs(dec - x) <= ulp / 2)
    # draft noise is added in fp32 before rounding, independently per row
    d = inputgen.logit_rows(6, 4096, np.array([0]), scale=3.0, noise_sd=0.5, noise_row=np.array([9]), dtype="f32")
    assert 0.45 < np.std(d[0] - x) < 0.55


def test_spikes_distinct():
    r = inputgen.logit_rows(7, 1000, np.arange(50), scale=0.0, n_spikes=20, spike_height=8.0)
    assert ((r == 8.0).sum(axis=1) == 20).all()


def test_token_sampler_matches_softmax():
    """Gumbel-max draws follow scipy's softmax(row / T); T == 0 picks the first argmax."""
    row = np.array([0.0, 1.0, -1.0, 2.0, 2.0, -np.inf, 0.5, 1.5], np.float32)
    n = 400_000
    rows = np.tile(row, (n, 1))
    tok = inputgen.sample_tokens(8, rows, np.full(n, 0.8, np.float32), np.arange(n))
    p = scipy.special.softmax(row.astype(np.float64) / np.float64(np.float32(0.8)))
    counts = np.bincount(tok, minlength=8)
    assert counts[5] == 0
    keep = p > 0
    stat = ((counts[keep] - n * p[keep]) ** 2 / (n * p[keep])).sum()
    assert scipy.stats.chi2.sf(stat, keep.sum() - 1) > 1e-3
    assert (inputgen.sample_tokens(8, rows[:10], np.zeros(10, np.float32), np.arange(10)) == 3).all()


def test_workload_shapes():
    d = inputgen.tree_inputs(4, 64, seed=4)
    par = d["parents"]
    assert par.shape == (4, 64) and (par[:, 0] == -1).all()
    assert all((par[:, v] < v).all() and (par[:, v] >= 0).all() for v in range(1, 64))
    depth = np.zeros((4, 64), int)
    for v in range(1, 64):
        depth[:, v] = depth[np.arange(4), par[:, v]] + 1
    for b in range(4):
        assert list(np.bincount(depth[b])) == [1, 4, 16, 43]
        kids = np.bincount(par[b, 21:], minlength=64)[5:21]
        assert sorted(kids) == [2] * 5 + [3] * 11
    r = inputgen.ragged_inputs(1024, 1, 8, 16, seed=5, n_greedy=256)
    g = np.diff(r["cu_gamma"])
    assert g.min() == 1 and g.max() == 8
    assert (r["temperature"] == 0).sum() == 256
    pos = r["temperature"][r["temperature"] > 0]
    assert pos.min() >= 0.5 and pos.max() <= 1.2
    assert r["target"].shape == (r["total_draft"] + 1024, 16)


def test_words_are_philox_outputs_in_counter_order():
    w = inputgen.words(9, inputgen.S_KV, 10)
    ref = [inputgen.philox4x32_10([i, 0, 0, inputgen.S_KV], [9, 0]).tolist() for i in range(3)]
    assert w.tolist() == (ref[0] + ref[1] + ref[2])[:10]


def test_kv_and_window_workloads():
    d = inputgen.kv_inputs(16, 5, 3, 10, 4, 12, 1)
    assert d["k_new"].shape == (16, 6, 3, 10) and d["k_new"].dtype == np.uint8
    assert not np.array_equal(d["k_new"], d["v_new"])
    assert ((d["lengths"] >= 0) & (d["lengths"] < 64)).all()
    assert ((d["num_accepted"] >= 0) & (d["num_accepted"] <= 5)).all()
    n = inputgen.acceptance_counts(3, 200000, 5, 0.8)
    # P(n = k) = 0.8^k * 0.2 for k < 5, 0.8^5 for k = 5
    p = np.array([0.8 ** k * 0.2 for k in range(5)] + [0.8 ** 5])
    assert np.allclose(np.bincount(n, minlength=6) / n.size, p, atol=0.005)
    w = inputgen.window_inputs(8, 64, 16, 3, 12, 2)
    assert w["block_table"].shape == (8, 12) and len(np.unique(w["block_table"])) == 96
    assert ((w["seq_lens"] >= 0) & (w["seq_lens"] <= 192)).all()
