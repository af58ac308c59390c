#!/usr/bin/env python3
"""Benchmark of the batched speculative-decoding verify step on one MI355X.

A step is one full verify call (row statistics -> acceptance scan -> residual /
bonus sampling) over one synthetic batch already resident in HBM. Default
workload: B=256 requests, gamma=5 drafted tokens, V=128256, bf16 logits
(target 2.5 * Student-t(3), draft = target + N(0, 1), T = 1).

Prints ONE JSON line: verified draft positions/s, logits GB/s against the
MI355X HBM peak (formula bytes B*(2g+1)*V*s + B*V*s per step), the roofline
entry of the dominant kernel (row statistics; durations from HIP events
recorded on the launch stream), and the CPU oracle timed on the host cores.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload large]
  python bench.py --copy-calibration          # plain copy kernel of known size (PMC scale)
  python bench.py --summarize-rocprof DIR     # text summary of rocprofv3 output in DIR
  python bench.py --write-pmc F W CF CW       # PMC traffic file from four rocprofv3 --pmc runs
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified draft positions/s + logits HBM GB/s (% of peak), B=256 γ=5 V=128256"
HBM_PEAK_GBPS = 8000.0
KERNEL = "k_row_stats"
PMC_FILE = os.path.join(ROOT, "profiles", "row_stats_large_pmc.json")
KERNEL_SOURCES = ["rejection_sampling_verify_spec_amd/csrc/row_stats.hip",
                  "rejection_sampling_verify_spec_amd/csrc/stream.h",
                  "rejection_sampling_verify_spec_amd/csrc/sv_internal.h"]

WORKLOAD_TEXT = {
    "large": "large-vocab chain verify: B=256, gamma=5, V=128256, bf16 logits, target 2.5*Student-t(3), "
             "draft = target + N(0,1), T=1.0",
    "tiny": "tiny chain verify: B=8, gamma=4, V=256, fp32",
    "mid": "mid chain verify: B=64, gamma=5, V=32000, fp32, 20 spikes +8, T=0.8",
    "tree": "token-tree verify: B=32, 64 nodes, V=152064, bf16",
    "tree_lossless": "lossless multi-candidate token-tree verify: B=32, 64 nodes, V=152064, bf16",
    "ragged": "ragged mixed verify: B=1024, gamma_b in 1..8, V=151936, bf16, 256 greedy",
    "sample": "draft-token sampling: one token per row of the large workload's 1280 draft rows "
              "(V=128256, bf16, Student-t), T=1.0",
    "kv": "KV commit into sink + ring caches after a B=256, gamma=5 verify step: 256 rows (32 layers x 8 KV "
          "heads) x 256 B (head dim 128, bf16) per position, S=4 sinks + W=1020 ring slots, lengths ~ U[0, 4096), "
          "accepted drafts from 5 Bernoulli(0.8) trials",
    "window": "draft-KV window: B=256, W=2048, block 128, future offset 5, lengths ~ U{0..40960}, "
              "full block table 256 x 320",
}
CACHE_WORKLOADS = ("kv", "window")
SAMPLE_METRIC = "sampled draft tokens/s + logits HBM GB/s (% of peak), 1280 rows V=128256"


def make_inputs(name):
    """Seeded synthetic inputs of a workload (numpy)."""
    import numpy as np

    import inputgen
    if name == "tree_lossless":
        return inputgen.make("tree")
    if name == "sample":
        d = inputgen.make("large")
        rows = np.ascontiguousarray(d["draft"].reshape(-1, d["draft"].shape[-1]))
        n = rows.shape[0]
        return {"logits": rows, "temperature": np.ones(n, np.float32),
                "u": inputgen.uniform24(41, inputgen.S_USAMP, n)}
    return inputgen.make(name)


def device_inputs(d, dev):
    """Generator arrays to device tensors (bf16 bit patterns become torch.bfloat16)."""
    import numpy as np
    import torch
    out = {}
    for k, a in d.items():
        if not isinstance(a, np.ndarray):
            continue
        if a.dtype == np.uint16:
            out[k] = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            out[k] = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return out


def _hash_files(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_source_hash() -> str:
    """Hash of the sources of the streaming statistics kernel."""
    return _hash_files(KERNEL_SOURCES)


def step_source_hash() -> str:
    """Hash of every source of the library (any kernel of a step)."""
    csrc = "rejection_sampling_verify_spec_amd/csrc"
    files = sorted(os.path.join(csrc, f) for f in os.listdir(os.path.join(ROOT, csrc)))
    return _hash_files(files + ["include/specverify.h"])


def host_cores() -> int:
    """Threads for the multi-threaded oracle: the CPUs this process may run on, at most 16 (the host
    share of one GPU on the measuring machines; nproc and the model are reported beside it)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def workload_accounting(name, d):
    """(positions, formula bytes, row-statistics algorithmic bytes) per step."""
    import numpy as np
    if name == "sample":
        rows, V = d["logits"].shape
        es = 4 if d["logits"].dtype == np.float32 else 2
        # one read of every row, and one extra pass over each row for the draw
        return rows, 2 * rows * V * es, rows * V * es
    es = 4 if d["target"].dtype == np.float32 else 2
    V = d["target"].shape[-1]
    T = d["temperature"]
    B = T.shape[0]
    if name in ("tree", "tree_lossless"):
        N = d["target"].shape[1]
        positions = B * (N - 1)
        formula = B * (2 * N - 1) * V * es + B * V * es
        rows_read = B * N + int((T > 0).sum()) * (N - 1)
    elif name == "ragged":
        g = np.diff(d["cu_gamma"]).astype(np.int64)
        positions = int(g.sum())
        formula = int((2 * g + 1).sum()) * V * es + B * V * es
        rows_read = int((g + 1).sum() + g[T > 0].sum())
    else:
        g = d["draft_tokens"].shape[1]
        positions = B * g
        formula = B * (2 * g + 1) * V * es + B * V * es
        rows_read = B * (g + 1) + int((T > 0).sum()) * g
    return positions, formula, rows_read * V * es


def lossless_walk_bytes(d, out_nodes, num_accepted):
    """Logit bytes the lossless tree walk reads in its passes, from the walk's own outputs: at each
    node of the emitted path, every sibling rejected before the accepted child (all children at the
    end node) costs one pass over the node's target row and the draft rows of the siblings rejected
    so far; an end node with no rejected child costs one pass over its target row."""
    import numpy as np
    B, N, V = d["target"].shape
    es = 2 if d["target"].dtype == np.uint16 else 4
    rows = 0
    for b in range(B):
        na = int(num_accepted[b])
        if na < 0 or d["temperature"][b] == 0.0:
            continue
        par = d["parents"][b]
        path = [0] + [int(x) for x in out_nodes[b, :na]]
        for i, v in enumerate(path):
            kids = [c for c in range(1, N) if par[c] == v]
            k = len(kids) if i == len(path) - 1 else sum(1 for c in kids if c < path[i + 1])
            rows += sum(1 + j for j in range(1, k + 1))
            if i == len(path) - 1 and k == 0:
                rows += 1
    return rows * V * es


def make_call(sv, name, t, d):
    """Closure running one verify step on device tensors t."""
    if name == "sample":
        return lambda tt: sv.sample_rows(tt["logits"], tt["temperature"], tt["u"])
    if name == "tree_lossless":
        return lambda tt: sv.verify_tree_lossless(tt["target"], tt["draft"], tt["node_tokens"], tt["parents"],
                                                  tt["u_accept"], tt["u_sample"], tt["temperature"], d["max_depth"])
    if name == "tree":
        return lambda tt: sv.verify_tree(tt["target"], tt["draft"], tt["node_tokens"], tt["parents"],
                                         tt["u_accept"], tt["u_sample"], tt["temperature"], d["max_depth"])
    if name == "ragged":
        return lambda tt: sv.verify_ragged(tt["target"], tt["draft"], tt["cu_gamma"], d["total_draft"],
                                           tt["draft_tokens"], tt["u_accept"], tt["u_sample"], tt["temperature"],
                                           d["gamma_max"])
    return lambda tt: sv.verify_chain(tt["target"], tt["draft"], tt["draft_tokens"], tt["u_accept"],
                                      tt["u_sample"], tt["temperature"])


def oracle_call(name, d, nthreads):
    import oracle
    if name == "sample":
        return oracle.sample_rows(d["logits"], d["temperature"], d["u"], nthreads=nthreads)
    if name == "tree_lossless":
        return oracle.verify_tree_lossless(d["target"], d["draft"], d["node_tokens"], d["parents"], d["u_accept"],
                                           d["u_sample"], d["temperature"], d["max_depth"], nthreads=nthreads)
    if name == "tree":
        return oracle.verify_tree(d["target"], d["draft"], d["node_tokens"], d["parents"], d["u_accept"],
                                  d["u_sample"], d["temperature"], d["max_depth"], nthreads=nthreads)
    if name == "ragged":
        return oracle.verify_chain(d["target"], d["draft"], d["draft_tokens"], d["u_accept"], d["u_sample"],
                                   d["temperature"], gamma=d["gamma_max"], cu_gamma=d["cu_gamma"], nthreads=nthreads)
    return oracle.verify_chain(d["target"], d["draft"], d["draft_tokens"], d["u_accept"], d["u_sample"],
                               d["temperature"], nthreads=nthreads)


def _load_pmc(name):
    if not os.path.exists(PMC_FILE):
        return None
    with open(PMC_FILE) as f:
        pmc = json.load(f)
    return pmc if pmc.get("workload") == WORKLOAD_TEXT[name] else None


def load_traffic(name):
    """HBM bytes per launch of the streaming kernel from committed PMC counters, if they were taken on
    this workload and match the current kernel source."""
    pmc = _load_pmc(name)
    if pmc is None or pmc.get("kernel_source_hash") != kernel_source_hash():
        return None
    return pmc.get("hbm_bytes_per_launch")


def load_step_bytes(name):
    """HBM bytes of a whole step (every kernel of the library, read + written) from committed PMC
    counters, if they were taken on this workload and every library source is unchanged since."""
    pmc = _load_pmc(name)
    if pmc is None or pmc.get("step_source_hash") != step_source_hash() or "step_kernels" not in pmc:
        return None
    return {"total": round(pmc["step_hbm_bytes"]), "per_kernel": {k: round(v) for k, v in pmc["step_kernels"].items()},
            "source": "rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a copy kernel of known size"}


def _percentile(xs, q):
    import numpy as np
    return float(np.percentile(np.asarray(xs, np.float64), q)) if len(xs) else float("nan")


def _timed_loop(args, sv, call, copies, pairs_per_call=1):
    """Warm-up, the timed region and two untimed measurement passes.

    Warm-up: args.warmup calls, with the library's kernel timing switched on once, so that its
    event pool (created on the first enable) and every other first-use cost lie before the timed
    region; then untimed calls until args.settle_ms have passed (GPU clocks). Timed region: exactly args.steps calls bracketed by torch.cuda.synchronize() (the wall
    clock gives `elapsed`), with one HIP event pair around the whole loop on the launch stream.
    Then an extra pass with an event between consecutive calls (per-step durations: median, p10,
    p90) and one with the library's kernel events on every call (at least 20 launches of the
    timed kernel). Returns a dict."""
    import torch
    n = len(copies)
    t_warm = time.perf_counter()
    events = not args.no_kernel_events
    if events:
        sv.spec_verify_timing_enable(True)
    for i in range(max(args.warmup, 1)):
        call(copies[i % n])
    if events:
        sv.spec_verify_timing_enable(False)
    torch.cuda.synchronize()
    sv.spec_verify_timing_reset()
    # settle: more untimed calls until args.settle_ms of wall time have passed since the warm-up
    # began, so that the GPU's clocks have left their idle state (a few warm-up calls of a
    # fraction of a millisecond each do not get there)
    settle = 0
    while (time.perf_counter() - t_warm) * 1e3 < args.settle_ms:
        for _ in range(20):
            call(copies[settle % n])
            settle += 1
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start = time.perf_counter()
    e0.record(stream)
    outs = None
    for i in range(args.steps):
        outs = call(copies[i % n])
    e1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - start
    gpu_ms = e0.elapsed_time(e1)

    nd = max(20, min(args.steps, 200))
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nd + 1)]
    evs[0].record(stream)
    for i in range(nd):
        call(copies[i % n])
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    step_ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(nd)]

    k_ms = []
    if events:
        nk = max(20, min(args.steps, 200))
        sv.spec_verify_timing_enable(True)
        for i in range(nk):
            call(copies[i % n])
        sv.spec_verify_timing_enable(False)
        torch.cuda.synchronize()
        k_ms = sv.spec_verify_timing_read(nk * pairs_per_call)
        sv.spec_verify_timing_reset()
    return {"elapsed": elapsed, "gpu_ms": gpu_ms, "step_ms": step_ms, "k_ms": k_ms, "outs": outs,
            "settle_calls": settle}


def _step_stats(t, steps):
    """Per-step figures of a _timed_loop result for the JSON line."""
    return {
        "settle_calls": t["settle_calls"],
        "ms_per_step_gpu_events": round(t["gpu_ms"] / steps, 5),
        "step_ms_distribution": {"median": round(_percentile(t["step_ms"], 50), 5),
                                 "p10": round(_percentile(t["step_ms"], 10), 5),
                                 "p90": round(_percentile(t["step_ms"], 90), 5),
                                 "samples": len(t["step_ms"]),
                                 "how": "extra pass after the timed region, one HIP event between consecutive "
                                        "calls on the launch stream"},
    }


def host_info(threads):
    """Host CPU facts for the CPU baseline: logical CPUs, CPUs this process may run on, model, and the
    oracle's thread count."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = os.cpu_count() or 1
    return {"nproc": os.cpu_count(), "cpus_allowed": aff, "cpu_model": model, "threads": threads}


def kv_copied_positions(d):
    """Positions a commit copies: the kept positions P..P+n, less those whose ring slot a later kept
    position takes."""
    S, W = d["sink"], d["window"]
    total = 0
    for P, n in zip(d["lengths"].tolist(), d["num_accepted"].tolist()):
        total += sum(1 for p in range(P, P + n + 1) if p < S or p + W > P + n)
    return total


def run_cache_bench(args):
    """The KV-cache steps: the commit into sink + ring caches (kv) and the draft-KV window (window)."""
    import numpy as np
    import torch

    import oracle
    import rejection_sampling_verify_spec_amd as sv

    name = args.workload
    d = make_inputs(name)
    dev = torch.device("cuda:0")
    cores = 1  # the oracle of these steps is single-threaded numpy
    if name == "kv":
        B = d["lengths"].shape[0]
        S, W, R, E, gamma = d["sink"], d["window"], d["rows"], d["row_bytes"], d["gamma"]
        cap = S + W
        kc = torch.empty((B, R, cap, E), dtype=torch.uint8, device=dev)
        vc = torch.empty_like(kc)
        copies = [device_inputs({"k_new": d["k_new"], "v_new": d["v_new"]}, dev) for _ in range(args.copies)]
        lens_t = torch.from_numpy(d["lengths"]).to(dev)
        n_t = torch.from_numpy(d["num_accepted"]).to(dev)

        def call(t):
            return sv.kv_commit(kc, vc, t["k_new"], t["v_new"], lens_t, n_t, S, W)
        units = int((d["num_accepted"] + 1).sum())
        algo = kv_copied_positions(d) * R * E * 2 * 2  # K and V rows, read once and written once
        kernel, unit, dtype = "k_kv_commit", "committed KV positions/s", "u8"
        metric = "committed KV positions/s + KV HBM GB/s (% of peak), B=256 gamma=5, 256 rows x 256 B"
    else:
        B, cols = d["block_table"].shape
        W, bs, K = d["window"], d["block_size"], d["future_offset"]
        wc = sv.spec_draft_window_max_blocks(W, bs)
        copies = [device_inputs({"seq_lens": d["seq_lens"], "block_table": d["block_table"]}, dev)
                  for _ in range(args.copies)]

        def call(t):
            return sv.draft_window(t["seq_lens"], t["block_table"], W, bs, K, window_cols=wc)
        units = B
        ref_all = oracle.draft_window(d["seq_lens"], W, bs, K, d["block_table"], wc)
        gathered = int((ref_all["block_table"] != 0).sum())
        algo = 4 * (B + gathered + B * wc + B)  # lengths read, block ids gathered, table and lengths written
        kernel, unit, dtype = "k_draft_window", "windowed requests/s", "int32"
        metric = "windowed requests/s + table HBM GB/s, B=256 W=2048 block 128"

    tl = _timed_loop(args, sv, call, copies)
    elapsed, k_ms, outs = tl["elapsed"], tl["k_ms"], tl["outs"]
    print(f"bench: {args.steps} steps in {elapsed * 1e3:.2f} ms", file=sys.stderr, flush=True)
    k_avg_ms = float(np.mean(k_ms)) if k_ms else float("nan")
    k_gbps = algo / (k_avg_ms * 1e-3) / 1e9

    ref = None
    cpu_calls, cpu_s, cpu_units = 0, 0.0, 0
    parity_ok = None
    if name == "kv":
        # the oracle on a sample of 8 requests, from the caches the GPU left after the warmup and timed
        # steps (every step commits the same batch, so a further commit changes nothing)
        ns = 8
        kc_h = kc[:ns].cpu().numpy()
        vc_h = vc[:ns].cpu().numpy()
        zc = np.zeros((B, 1, cap, 0), np.uint8)
        zn = np.zeros((B, gamma + 1, 1, 0), np.uint8)
        ref_len = oracle.kv_commit(zc, zc.copy(), zn, zn.copy(), d["lengths"], d["num_accepted"], S, W)
        lens_ok = bool(np.array_equal(outs.cpu().numpy(), ref_len))
        sample_units = int((d["num_accepted"][:ns] + 1).sum())
        if not args.skip_cpu_baseline:
            # start the oracle from other contents, so that its writes are the ones compared
            kc_o = np.zeros_like(kc_h)
            vc_o = np.zeros_like(vc_h)
            tc = time.perf_counter()
            while cpu_calls == 0 or cpu_s < args.cpu_seconds:
                oracle.kv_commit(kc_o, vc_o, d["k_new"][:ns], d["v_new"][:ns], d["lengths"][:ns],
                                 d["num_accepted"][:ns], S, W)
                cpu_calls += 1
                cpu_s = time.perf_counter() - tc
            cpu_units = sample_units * cpu_calls
            # the slots this step wrote must agree; the others hold what earlier contents left
            rows_ok = True
            for b in range(ns):
                P, n = int(d["lengths"][b]), int(d["num_accepted"][b])
                for s_ in {oracle.slot(p, S, W) for p in range(P, P + n + 1)}:
                    rows_ok &= bool(np.array_equal(kc_o[b, :, s_], kc_h[b, :, s_]) and
                                    np.array_equal(vc_o[b, :, s_], vc_h[b, :, s_]))
            parity_ok = lens_ok and rows_ok
            sample = (f"{cpu_calls} commits of 8 of the 256 requests ({sample_units} kept positions each), numpy "
                      f"oracle, 1 thread, {cpu_s:.2f} s wall")
    else:
        got_l, got_t = (o.cpu().numpy() for o in outs)
        parity_ok = bool(np.array_equal(got_l, ref_all["windowed_lens"]) and
                         np.array_equal(got_t, ref_all["block_table"]))
        if not args.skip_cpu_baseline:
            tc = time.perf_counter()
            while cpu_calls == 0 or cpu_s < args.cpu_seconds:
                oracle.draft_window(d["seq_lens"], W, bs, K, d["block_table"], wc)
                cpu_calls += 1
                cpu_s = time.perf_counter() - tc
            cpu_units = B * cpu_calls
            sample = f"{cpu_calls} calls over all {B} requests, numpy oracle, 1 thread, {cpu_s:.2f} s wall"
    line = {
        "metric": metric,
        "value": round(units * args.steps / elapsed, 1),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[name], "B": int(B), "units_per_step": units,
                   "input_copies_rotated": args.copies},
        "hbm_gbps_algorithmic": round(algo * args.steps / elapsed / 1e9, 1),
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "achieved": round(k_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(k_gbps / HBM_PEAK_GBPS, 4),
            "traffic": None,
            "algorithmic_bytes_per_launch": algo,
            "avg_launch_ms": round(k_avg_ms, 5),
            "launches_timed": len(k_ms),
            "launches_timed_how": "extra pass after the timed region, HIP events on the launch stream",
        },
        "cpu_baseline": None if cpu_calls == 0 else {
            "value": round(cpu_units / cpu_s, 1), "unit": unit, "cores": cores, "kind": "oracle",
            "sample": sample, **host_info(cores),
        },
        "parity_vs_oracle": parity_ok,
    }
    line.update(_step_stats(tl, args.steps))
    print(json.dumps(line), flush=True)
    return 0 if parity_ok is not False else 1


def read_ceiling(sv, tensors, reps=20):
    """The practical read rate (GB/s) of a plain probe kernel over the given device tensors, with the
    streaming kernel's load pattern; events on the launch stream around `reps` rounds."""
    import torch
    outs = [sv.read_probe(t) for t in tensors]  # warm-up, and the output buffers
    nbytes = sum(t.numel() * t.element_size() // 16 * 16 for t in tensors)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        for t, o in zip(tensors, outs):
            sv.read_probe(t, o)
    e1.record()
    torch.cuda.synchronize()
    return nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def run_bench(args):
    import numpy as np
    import torch

    import inputgen
    import rejection_sampling_verify_spec_amd as sv

    name = args.workload
    t0 = time.time()
    d = make_inputs(name)
    print(f"bench: generated {name} inputs in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    copies = [device_inputs(d, dev) for _ in range(args.copies)]
    call = make_call(sv, name, copies[0], d)
    positions, formula_bytes, k1_bytes = workload_accounting(name, d)

    tl = _timed_loop(args, sv, call, copies, pairs_per_call=2 if name == "tree_lossless" else 1)
    elapsed, k1_ms, outs = tl["elapsed"], tl["k_ms"], tl["outs"]
    print(f"bench: {args.steps} steps in {elapsed * 1e3:.2f} ms", file=sys.stderr, flush=True)

    ms_per_step = elapsed * 1e3 / args.steps
    value = positions * args.steps / elapsed
    gbps = formula_bytes * args.steps / elapsed / 1e9
    walk_ms = None
    if name == "tree_lossless":  # two event pairs per call: the streaming kernel, then the walk
        walk_ms, k1_ms = k1_ms[1::2], k1_ms[0::2]
    k1_avg_ms = float(np.mean(k1_ms)) if k1_ms else float("nan")
    k1_gbps = k1_bytes / (k1_avg_ms * 1e-3) / 1e9

    ceiling = read_ceiling(sv, [copies[0]["logits"]] if name == "sample" else
                           [copies[0]["target"], copies[0]["draft"]])

    # CPU oracle on the host cores: whole verify steps of the same batch, repeated until about
    # args.cpu_seconds of wall time have passed (at least one step), then on one thread
    cores = host_cores()
    ref = None
    cpu_steps = cpu1_steps = 0
    cpu_s = cpu1_s = 0.0
    if not args.skip_cpu_baseline:
        tc = time.perf_counter()
        while cpu_steps == 0 or cpu_s < args.cpu_seconds:
            ref = oracle_call(name, d, cores)
            cpu_steps += 1
            cpu_s = time.perf_counter() - tc
        print(f"bench: oracle {cpu_steps} steps in {cpu_s:.2f} s on {cores} threads", file=sys.stderr, flush=True)
        tc = time.perf_counter()
        while cpu1_steps == 0 or cpu1_s < args.cpu1_seconds:
            oracle_call(name, d, 1)
            cpu1_steps += 1
            cpu1_s = time.perf_counter() - tc
        print(f"bench: oracle {cpu1_steps} steps in {cpu1_s:.2f} s on 1 thread", file=sys.stderr, flush=True)
    sample = name == "sample"
    if sample:
        tok = outs.cpu().numpy()
        parity_ok = None if ref is None else bool(np.array_equal(tok, ref["tokens"]))
    else:
        na = outs[-1].cpu().numpy()
        out_tok = outs[0].cpu().numpy()
        parity_ok = None if ref is None else bool(np.array_equal(na, ref["num_accepted"]) and
                                                  np.array_equal(out_tok, ref["out_tokens"]))
    unit = "sampled draft tokens/s" if sample else "verified draft positions/s"
    what = "sampling calls" if sample else "full verify steps"
    per = "rows" if sample else "positions"
    in_dt = "bf16" if d["logits" if sample else "target"].dtype == np.uint16 else "f32"

    line = {
        "metric": SAMPLE_METRIC if sample else (METRIC if name == "large" else
                                                f"verified draft positions/s + logits HBM GB/s (% of peak), {name}"),
        "value": round(value, 1),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # arithmetic of the path: the streaming statistics (nearly all of the time) in fp32, the
        # acceptance scan and the draw in fp64; the logits are read as stored (input_dtype)
        "dtype": "f32",
        "arith": "fp32 streaming statistics; fp64 acceptance scan and draw",
        "input_dtype": in_dt,
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[name], "B": int(d["temperature"].shape[0]),
                   "V": int(d["logits" if sample else "target"].shape[-1]), "positions_per_step": positions,
                   "input_copies_rotated": args.copies},
        "logits_gbps_formula": round(gbps, 1),
        "hbm_peak_frac_formula": round(gbps / HBM_PEAK_GBPS, 4),
        "formula_bytes_per_step": formula_bytes,
        "measured_bytes_per_step": load_step_bytes(name),
        "roofline": {
            "bound": "hbm",
            "kernel": KERNEL,
            "achieved": round(k1_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(k1_gbps / HBM_PEAK_GBPS, 4),
            "traffic": load_traffic(name),
            "algorithmic_bytes_per_launch": k1_bytes,
            "avg_launch_ms": round(k1_avg_ms, 5),
            "launches_timed": len(k1_ms),
            "launches_timed_how": "extra pass after the timed region, HIP events on the launch stream",
        },
        "cpu_baseline": None if ref is None else {
            "value": round(positions * cpu_steps / cpu_s, 1),
            "unit": unit,
            "cores": cores,
            "kind": "oracle",
            "sample": f"{cpu_steps} {what} of the same batch ({positions} {per} each), "
                      f"fp64 oracle, {cores} threads, {cpu_s:.2f} s wall; then {cpu1_steps} on 1 thread, "
                      f"{cpu1_s:.2f} s wall",
            "single_thread_value": round(positions * cpu1_steps / cpu1_s, 1),
            **host_info(cores),
        },
        "parity_vs_oracle": parity_ok,
        "read_ceiling": {"kernel": "k_read_probe", "gbps": round(ceiling, 1),
                         "frac_of_peak": round(ceiling / HBM_PEAK_GBPS, 4),
                         "row_stats_frac_of_ceiling": round(k1_gbps / ceiling, 4)},
    }
    line.update(_step_stats(tl, args.steps))
    if not sample:
        line["mean_num_accepted"] = round(float(np.mean(na[na >= 0])), 4)
    if walk_ms:
        # the walk kernel takes most of the step: its passes are latency-bound, the streaming
        # kernel's entry moves to row_stats_roofline
        walk_avg = float(np.mean(walk_ms))
        wb = lossless_walk_bytes(d, outs[1].cpu().numpy(), na)
        line["row_stats_roofline"] = line["roofline"]
        line["roofline"] = {
            "bound": "hbm", "kernel": "k_tree_lossless", "achieved": round(wb / (walk_avg * 1e-3) / 1e9, 1),
            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(wb / (walk_avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "traffic": None, "algorithmic_bytes_per_launch": wb, "avg_launch_ms": round(walk_avg, 5),
            "launches_timed": len(walk_ms),
            "launches_timed_how": "extra pass after the timed region, HIP events on the launch stream",
        }
    print(json.dumps(line), flush=True)
    return 0 if parity_ok is not False else 1


# Pooled parity: seeds 1000 + k of a workload until at least 10^4 requests (the near-tie rate of
# the parity bar is a fraction of requests, so it needs that many to be measured at all)
POOL_SEEDS = {"tiny": 1250, "mid": 157, "large": 40, "ragged": 10, "tree_near": 40, "tree_rule": 40,
              "tree_walk": 40}
FLAG = 1e-5
# tree_near: lossless multi-candidate trees with near-identical drafts and forced rejections, 250
# trees of V=30000 per seed; seed k takes case k % 4 (dtype, noise of the draft rows)
NEAR_CASES = (("f32", 0.003), ("f32", 0.01), ("f32", 0.03), ("bf16", 0.05))
# tree_rule / tree_walk: the lowest-child rule and the lossless walk on 64-node trees (4 children of
# the root, 4 under each, 2-3 under those), 250 trees of V=10007 per seed; seed k takes case k % 4
# (dtype, noise of the draft rows, temperature)
TREE_CASES = (("bf16", 0.7, 1.0), ("f32", 1.5, 0.8), ("bf16", 0.3, 1.2), ("f32", 3.0, 0.6))


def pooled_inputs(name, seed):
    """The inputs of one pooled seed and the workload whose call and oracle they take."""
    import inputgen
    if name == "tree_near":
        dtype, noise = NEAR_CASES[(seed - 1000) % len(NEAR_CASES)]
        return inputgen.near_identical_trees(250, 30000, seed, dtype=dtype, noise_sd=noise), "tree_lossless"
    if name in ("tree_rule", "tree_walk"):
        dtype, noise, temp = TREE_CASES[(seed - 1000) % len(TREE_CASES)]
        d = inputgen.tree_inputs(250, 10007, seed, dtype=dtype, noise_sd=noise, temperature=temp)
        return d, "tree" if name == "tree_rule" else "tree_lossless"
    return inputgen.make(name, seed=seed), name


def run_pooled(args):
    """GPU against the oracle on many seeds of each named workload: every differing request must be
    flagged by the oracle (a uniform within 1e-5 of its acceptance ratio, or u*S within 1e-5*S of a
    CDF boundary) and differing requests must stay below 1e-4 of all requests. Prints one JSON line
    with the counts and rates per workload."""
    import torch

    import rejection_sampling_verify_spec_amd as sv
    dev = torch.device("cuda:0")
    names = [n for n in args.pooled_parity.split(",") if n]
    result = {}
    ok = True
    for name in names:
        seeds = POOL_SEEDS[name] if args.pool_seeds is None else args.pool_seeds
        c = dict(seeds=seeds, requests=0, mismatches=0, unflagged_mismatches=0, flagged_requests=0,
                 fallback_requests=0, error_requests=0)
        t0 = time.time()
        for k in range(seeds):
            d, kind = pooled_inputs(name, 1000 + k)
            t = device_inputs(d, dev)
            outs = make_call(sv, kind, t, d)(t)
            torch.cuda.synchronize()
            out, na = outs[0].cpu().numpy(), outs[-1].cpu().numpy()
            ref = oracle_call(kind, d, host_cores())
            mism = (na != ref["num_accepted"]) | (out != ref["out_tokens"]).any(axis=1)
            flagged = (ref["acc_margin"] < FLAG) | (ref["cdf_margin"] < FLAG)
            c["requests"] += int(na.shape[0])
            c["mismatches"] += int(mism.sum())
            c["unflagged_mismatches"] += int((mism & ~flagged).sum())
            c["flagged_requests"] += int(flagged.sum())
            c["fallback_requests"] += int(ref["fallback"].sum())
            c["error_requests"] += int((ref["num_accepted"] < 0).sum())
            if k % max(1, seeds // 10) == 0 or k == seeds - 1:
                print(f"pooled {name}: seed {1000 + k} ({k + 1}/{seeds}), {c['requests']} requests, "
                      f"{c['mismatches']} mismatches, {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
        c["flag_rate"] = c["flagged_requests"] / c["requests"]
        c["mismatch_rate"] = c["mismatches"] / c["requests"]
        c["pass"] = c["unflagged_mismatches"] == 0 and c["mismatch_rate"] < 1e-4
        ok &= c["pass"]
        result[name] = c
    print(json.dumps({"pooled_parity": result,
                      "bar": "every differing request flagged by the oracle (1e-5 band); differing requests "
                             "below 1e-4 of requests",
                      "seeds": "1000 + k"}), flush=True)
    return 0 if ok else 1


COPY_BYTES = 1 << 30


def copy_calibration(args):
    """A plain copy kernel of known size (an elementwise float32 multiply by one, 1 GiB read and
    1 GiB written per launch), for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = COPY_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": COPY_BYTES, "copy_bytes_written_per_launch": COPY_BYTES,
                      "launches": args.steps}), flush=True)
    return 0


def _counter_avgs(path):
    """{(kernel short name, counter): average value per dispatch} over rocprofv3 counter CSVs under path."""
    agg = {}
    for p in glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True):
        with open(p) as f:
            for r in csv.DictReader(f):
                key = (r.get("Kernel_Name", "").split("(")[0], r.get("Counter_Name"))
                agg.setdefault(key, []).append(float(r.get("Counter_Value", 0)))
    return {k: sum(v) / len(v) for k, v in agg.items()}


def _pick(avgs, counter, want=None):
    """Average of `counter` for the kernel whose name contains `want` (else the largest one)."""
    rows = [(k, v) for (k, c), v in avgs.items() if c == counter and (want is None or want in k)]
    if not rows:
        raise SystemExit(f"no {counter} rows" + (f" for {want}" if want else ""))
    return max(rows, key=lambda kv: kv[1])


def write_pmc(dirs, workload):
    """profiles/row_stats_<workload>_pmc.json from four rocprofv3 --pmc runs: FETCH_SIZE and
    WRITE_SIZE of the bench, then of --copy-calibration. Counter units are KiB per dispatch; each is
    scaled by bytes/KiB of the copy kernel of known size."""
    import inputgen
    fetch_dir, write_dir, cfetch_dir, cwrite_dir = dirs
    kf_name, kf = _pick(_counter_avgs(fetch_dir), "FETCH_SIZE", KERNEL)
    kw_name, kw = _pick(_counter_avgs(write_dir), "WRITE_SIZE", KERNEL)
    cf_name, cf = _pick(_counter_avgs(cfetch_dir), "FETCH_SIZE")
    cw_name, cw = _pick(_counter_avgs(cwrite_dir), "WRITE_SIZE")
    f_scale = COPY_BYTES / cf
    w_scale = COPY_BYTES / cw
    fetch_b = kf * f_scale
    write_b = kw * w_scale
    _, _, algo = workload_accounting(workload, inputgen.make(workload))
    out = {
        "kernel": kf_name, "workload": WORKLOAD_TEXT[workload],
        "fetch_kib_per_dispatch": kf, "write_kib_per_dispatch": kw,
        "copy_kernel": cf_name, "copy_fetch_kib_per_dispatch": cf, "copy_write_kib_per_dispatch": cw,
        "copy_bytes_per_dispatch": COPY_BYTES, "fetch_scale_bytes_per_unit": f_scale,
        "write_scale_bytes_per_unit": w_scale,
        "hbm_fetch_bytes_per_launch": fetch_b, "hbm_write_bytes_per_launch": write_b,
        "hbm_bytes_per_launch": fetch_b + write_b, "algorithmic_bytes_per_launch": algo,
        "traffic_over_algorithmic": (fetch_b + write_b) / algo,
        "kernel_source_hash": kernel_source_hash(),
    }
    # every library kernel of the step (the read-ceiling probe is a measurement aid, not a step)
    fa, wa = _counter_avgs(fetch_dir), _counter_avgs(write_dir)
    step = {}
    for (k, c), v in fa.items():
        if c == "FETCH_SIZE" and (k.startswith("void sv::") or k.startswith("sv::")):
            step[k] = v * f_scale + wa.get((k, "WRITE_SIZE"), 0.0) * w_scale
    out["step_kernels"] = step
    out["step_hbm_bytes"] = sum(step.values())
    out["step_source_hash"] = step_source_hash()
    os.makedirs(os.path.dirname(PMC_FILE), exist_ok=True)
    with open(PMC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))
    return 0


def summarize_rocprof(path):
    """Summarise rocprofv3 output found under `path`: kernel stats (avg duration) and, when present,
    per-dispatch FETCH_SIZE / WRITE_SIZE averages per kernel."""
    stats = glob.glob(os.path.join(path, "**", "*kernel_stats.csv"), recursive=True)
    ctrs = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    for p in stats:
        print(f"# kernel stats: {os.path.relpath(p, path)}")
        with open(p) as f:
            rows = list(csv.DictReader(f))
        print("| kernel | calls | avg ns | min ns | max ns | total % |")
        print("|---|---|---|---|---|---|")
        for r in rows:
            nm = r.get("Name", "")
            short = nm.split("(")[0][:70]
            print(f"| {short} | {r.get('Calls')} | {r.get('AverageNs')} | {r.get('MinNs')} | {r.get('MaxNs')} | "
                  f"{float(r.get('Percentage', 0)):.2f} |")
    for p in ctrs:
        print(f"# counters: {os.path.relpath(p, path)}")
        agg = {}
        with open(p) as f:
            for r in csv.DictReader(f):
                key = (r.get("Kernel_Name", "").split("(")[0][:70], r.get("Counter_Name"))
                agg.setdefault(key, []).append(float(r.get("Counter_Value", 0)))
        print("| kernel | counter | dispatches | avg per dispatch |")
        print("|---|---|---|---|")
        for (k, c), v in sorted(agg.items()):
            print(f"| {k} | {c} | {len(v)} | {sum(v) / len(v):.1f} |")
    return 0


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="large", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--copies", type=int, default=3, help="input copies rotated across steps")
    ap.add_argument("--settle-ms", type=float, default=500.0,
                    help="untimed calls after the warm-up until this much wall time has passed since it began")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="wall time spent timing the CPU oracle on the host cores")
    ap.add_argument("--cpu1-seconds", type=float, default=4.0,
                    help="wall time spent timing the CPU oracle on one thread")
    ap.add_argument("--skip-cpu-baseline", action="store_true", help="no oracle run (profiling runs)")
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="do not create the library's kernel events (profiling runs: the profiler times the kernels)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--pooled-parity", metavar="NAMES",
                    help="comma-separated workloads (tiny,mid,large,ragged,tree_near,tree_rule,tree_walk): "
                         "GPU against the oracle over many seeds")
    ap.add_argument("--pool-seeds", type=int, default=None, help="seeds per workload for --pooled-parity")
    ap.add_argument("--summarize-rocprof", metavar="DIR")
    ap.add_argument("--write-pmc", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write the committed PMC traffic file from four rocprofv3 --pmc output folders")
    args = ap.parse_args()
    if args.summarize_rocprof:
        return summarize_rocprof(args.summarize_rocprof)
    if args.write_pmc:
        return write_pmc(args.write_pmc, args.workload)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: only one GPU is measured here; the verify step shards over requests with no "
              "communication, so N GPUs each run this same single-GPU step. Run with --gpus 1.", file=sys.stderr)
        return 2
    if args.copy_calibration:
        return copy_calibration(args)
    if args.pooled_parity:
        return run_pooled(args)
    if args.workload in CACHE_WORKLOADS:
        return run_cache_bench(args)
    return run_bench(args)


if __name__ == "__main__":
    sys.exit(main())
