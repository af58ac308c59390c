"""The measurement's host logic on the CPU: the byte counts bench.py prices kernels against, the
lossless walk's row count, the scaling of the HBM counters and the rocprofv3 summaries. Expected
values are worked out by hand from the definitions in the docstrings, not by calling the code."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _shape(shape, dtype):
    """An array of the given shape and dtype that occupies no memory (the accounting reads shapes)."""
    return np.broadcast_to(np.zeros((), dtype), shape)


def test_chain_bytes_large_workload():
    """B=256, gamma=5, V=128256 bf16: the streaming pass reads 256 x 11 rows (722,337,792 B), and the
    formula adds one drawn row per request (788,004,864 B per step)."""
    B, g, V = 256, 5, 128256
    d = {"target": _shape((B, g + 1, V), np.uint16), "draft": _shape((B, g, V), np.uint16),
         "draft_tokens": _shape((B, g), np.int32), "temperature": np.ones(B, np.float32)}
    positions, formula, algo = bench.workload_accounting("large", d)
    assert positions == 1280
    assert algo == 722_337_792 == 2816 * 128256 * 2
    assert formula == 788_004_864 == (256 * 11 + 256) * 128256 * 2


def test_chain_bytes_greedy_requests_skip_draft_rows():
    """A greedy request (T = 0) reads its g + 1 target rows only."""
    B, g, V = 4, 3, 1000
    T = np.array([1.0, 0.0, 0.7, 0.0], np.float32)
    d = {"target": _shape((B, g + 1, V), np.float32), "draft": _shape((B, g, V), np.float32),
         "draft_tokens": _shape((B, g), np.int32), "temperature": T}
    positions, formula, algo = bench.workload_accounting("mid", d)
    assert positions == 12
    assert algo == (4 * 4 + 2 * 3) * 1000 * 4
    assert formula == (4 * 7 + 4) * 1000 * 4


def test_ragged_bytes():
    """gamma_b = 2, 0, 3 (cu_gamma 0, 2, 2, 5), the second request greedy: rows read 3 + 1 + 4 target
    rows and 2 + 3 draft rows."""
    V = 500
    cu = np.array([0, 2, 2, 5], np.int32)
    T = np.array([1.0, 0.0, 0.9], np.float32)
    d = {"target": _shape((8, V), np.uint16), "draft": _shape((5, V), np.uint16), "cu_gamma": cu,
         "temperature": T}
    positions, formula, algo = bench.workload_accounting("ragged", d)
    assert positions == 5
    assert algo == (8 + 5) * V * 2
    assert formula == ((5 + 1 + 7) + 3) * V * 2


def test_tree_bytes():
    """B=2 trees of N=4 nodes, one greedy: target rows of every node, draft rows of the sampling tree's
    non-root nodes; the formula counts (2N - 1) rows plus one drawn row per tree."""
    B, N, V = 2, 4, 300
    d = {"target": _shape((B, N, V), np.float32), "draft": _shape((B, N - 1, V), np.float32),
         "temperature": np.array([1.0, 0.0], np.float32)}
    positions, formula, algo = bench.workload_accounting("tree", d)
    assert positions == 6
    assert algo == (2 * 4 + 3) * V * 4
    assert formula == (2 * 7 + 2) * V * 4


def test_sampler_bytes():
    rows, V = 10, 256
    d = {"logits": _shape((rows, V), np.uint16)}
    positions, formula, algo = bench.workload_accounting("sample", d)
    assert (positions, formula, algo) == (10, 2 * 10 * 256 * 2, 10 * 256 * 2)


def test_lossless_walk_rows():
    """Tree: root 0 with children 1, 2, 3; node 2 with child 4. The k-th rejected sibling at a node
    costs one pass over the node's target row and the k rejected draft rows so far (1 + k rows); an
    end node with no rejected child costs one pass over its target row."""
    V = 100
    par = np.array([[-1, 0, 0, 0, 2]] * 4, np.int32)
    d = {"target": _shape((4, 5, V), np.float32), "parents": par,
         "temperature": np.array([1.0, 1.0, 1.0, 0.0], np.float32)}
    out_nodes = np.array([[2, 4], [-1, -1], [3, -1], [1, -1]], np.int32)
    na = np.array([2, 0, 1, 1], np.int32)
    # request 0: at the root child 1 is rejected (2 rows), child 2 accepted; at node 2 its only child 4
    #   is accepted; node 4 is a leaf: 1 row. Total 3.
    # request 1: every child of the root rejected: 2 + 3 + 4 = 9 rows.
    # request 2: children 1 and 2 rejected (2 + 3), child 3 accepted, a leaf (1): 6 rows.
    # request 3: greedy, no passes.
    assert bench.lossless_walk_bytes(d, out_nodes, na) == (3 + 9 + 6) * V * 4


def _counter_csv(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "x_counter_collection.csv"), "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for k, c, v in rows:
            f.write(f'"{k}",{c},{v}\n')


def test_write_pmc_scaling(tmp_path, monkeypatch):
    """A copy kernel of 1 GiB that reads 524,288 FETCH_SIZE units and writes 1,048,576 WRITE_SIZE units
    scales them by 2048 and 1024 B per unit; the streaming kernel's averages over its dispatches are
    scaled by the same factors, and the step sums every library kernel but the read probe."""
    rs = "void sv::k_row_stats<1, 2>(args)"
    rq = "void sv::k_request<1, true>(args)"
    probe = "svp::k_read_probe(args)"
    copy = "void at::native::vectorized_elementwise_kernel<...>(args)"
    _counter_csv(tmp_path / "f", [(rs, "FETCH_SIZE", 100.0), (rs, "FETCH_SIZE", 300.0), (rq, "FETCH_SIZE", 10.0),
                                  (probe, "FETCH_SIZE", 9999.0)])
    _counter_csv(tmp_path / "w", [(rs, "WRITE_SIZE", 4.0), (rq, "WRITE_SIZE", 2.0), (probe, "WRITE_SIZE", 1.0)])
    _counter_csv(tmp_path / "cf", [(copy, "FETCH_SIZE", 524288.0)])
    _counter_csv(tmp_path / "cw", [(copy, "WRITE_SIZE", 1048576.0)])
    out = tmp_path / "pmc.json"
    monkeypatch.setattr(bench, "PMC_FILE", str(out))
    import inputgen
    B, g, V = 256, 5, 128256
    monkeypatch.setattr(inputgen, "make", lambda name: {
        "target": _shape((B, g + 1, V), np.uint16), "draft": _shape((B, g, V), np.uint16),
        "draft_tokens": _shape((B, g), np.int32), "temperature": np.ones(B, np.float32)})
    assert bench.write_pmc([str(tmp_path / x) for x in ("f", "w", "cf", "cw")], "large") == 0
    r = json.loads(out.read_text())
    assert r["fetch_scale_bytes_per_unit"] == 2048.0 and r["write_scale_bytes_per_unit"] == 1024.0
    assert r["hbm_fetch_bytes_per_launch"] == 200.0 * 2048 and r["hbm_write_bytes_per_launch"] == 4.0 * 1024
    assert r["algorithmic_bytes_per_launch"] == 722_337_792
    assert r["traffic_over_algorithmic"] == pytest.approx((200 * 2048 + 4 * 1024) / 722_337_792)
    assert set(r["step_kernels"]) == {"void sv::k_row_stats<1, 2>", "void sv::k_request<1, true>"}
    assert r["step_hbm_bytes"] == 200 * 2048 + 4 * 1024 + 10 * 2048 + 2 * 1024
    assert r["kernel_source_hash"] == bench.kernel_source_hash()
    assert r["step_source_hash"] == bench.step_source_hash()


def test_summarize_rocprof(tmp_path, capsys):
    p = tmp_path / "run"
    p.mkdir()
    (p / "k_kernel_stats.csv").write_text(
        "Name,Calls,TotalDurationNs,AverageNs,Percentage,MinNs,MaxNs\n"
        '"void sv::k_row_stats<1, 2>(void const*)",10,1000,100.5,90.25,90,120\n')
    assert bench.summarize_rocprof(str(p)) == 0
    txt = capsys.readouterr().out
    assert "| void sv::k_row_stats<1, 2> | 10 | 100.5 | 90 | 120 | 90.25 |" in txt


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "only one GPU" in r.stderr
