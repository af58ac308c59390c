"""Seeded synthetic inputs for the speculative-decoding verify path.

Serves both sides (the HIP path's tests/bench and the CPU oracle) and holds
none of the verification arithmetic. Every value is a pure function of
(seed, stream, row, column) through Philox4x32-10 in ``gen.c``.

Workloads (names used by tests and the bench):

=========  =====================================================================
tiny       B=8, gamma=4, V=256, fp32; target ~ N(0, sd 2); draft = target + N(0, 0.7); T=1.0
mid        B=64, gamma=5, V=32000, fp32; target ~ N(0, sd 3) + 8 on 20 distinct ids per row;
           draft = target + N(0, 0.5); T=0.8
large      B=256, gamma=5, V=128256, bf16; target = 2.5 * Student-t(3); draft = target + N(0, 1.0); T=1.0
tree       B=32, 64 nodes (root + 4 + 16 + 43, depth 3), V=152064, bf16; target ~ N(0, sd 3);
           draft row of node v = target row of parent(v) + N(0, 0.7); T=1.0
ragged     B=1024, gamma_b ~ U{1..8}, V=151936, bf16; target ~ N(0, sd 3); draft = target + N(0, sigma_b),
           sigma_b ~ U[0.2, 2.0]; 256 requests (seeded permutation) greedy T=0, the rest T ~ U(0.5, 1.2)
kv         KV commit after a B=256, gamma=5 verify step: R=256 rows (32 layers x 8 KV heads) of E=256
           bytes (head dim 128, bf16) per position; S=4 sinks + W=1020 ring slots; lengths ~ U[0, 4096);
           accepted drafts = leading successes of 5 Bernoulli(0.8) trials; keys/values random bytes
window     draft-KV window: B=256, W=2048, block 128, future offset K=5; lengths ~ U{0..40960};
           full block table [256, 320] of distinct block ids
=========  =====================================================================

Draft tokens are drawn from softmax(draft row / T) of the *stored* draft row
(Gumbel-max), greedy requests take the draft argmax. Uniforms are float32 on
the 2^-24 grid of [0, 1 - 2^-24]. bf16 logits are returned as uint16 bit
patterns (round-to-nearest-even from fp32).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libinputgen.so")

S_TOKENS, S_UACC, S_USAMP, S_GAMMA, S_SIGMA, S_TEMP, S_PERM, S_TREE = 4, 5, 6, 7, 8, 9, 10, 11
S_KV, S_LEN, S_ACC, S_TABLE = 12, 13, 14, 15
DIST_NORMAL, DIST_T3 = 0, 1

_lib = None


def _compiler():
    """gcc, or with SPECVERIFY_SANITIZE=1 ROCm's clang with AddressSanitizer and UndefinedBehaviorSanitizer
    (the same runtime as the sanitized host code of the HIP library, so one process can load both)."""
    if os.environ.get("SPECVERIFY_SANITIZE") == "1":
        return ["/opt/rocm/llvm/bin/clang", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                "-fno-omit-frame-pointer", "-shared-libsan", "-g"]
    return ["gcc"]


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(_compiler() + ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-pthread", _SRC,
                                      "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P, I, U64, U32, I64, D = (ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_uint32,
                                  ctypes.c_int64, ctypes.c_double)
        lib.ig_philox4x32_10.argtypes = [P, P, P]
        lib.ig_uniform24.argtypes = [U64, U32, I64, P, I]
        lib.ig_uniform53.argtypes = [U64, U32, I64, P, I]
        lib.ig_normal.argtypes = [U64, U32, I64, P, I]
        lib.ig_words.argtypes = [U64, U32, I64, P, I]
        lib.ig_logit_rows.argtypes = [U64, I, D, I, D, I64, I, P, P, P, I, P, I]
        lib.ig_logit_rows.restype = I
        lib.ig_sample_tokens.argtypes = [U64, U32, I64, I, I, P, P, P, P, I]
        lib.ig_sample_tokens.restype = I
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _nt(n=None):
    return int(n) if n else max(1, min(16, os.cpu_count() or 1))


def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(ctr, np.uint32)
    k = np.ascontiguousarray(key, np.uint32)
    o = np.empty(4, np.uint32)
    _load().ig_philox4x32_10(_p(c), _p(k), _p(o))
    return o


def uniform24(seed, stream, n):
    out = np.empty(int(n), np.float32)
    _load().ig_uniform24(seed, stream, int(n), _p(out), _nt())
    return out


def uniform53(seed, stream, n):
    out = np.empty(int(n), np.float64)
    _load().ig_uniform53(seed, stream, int(n), _p(out), _nt())
    return out


def normal(seed, stream, n):
    out = np.empty(int(n), np.float64)
    _load().ig_normal(seed, stream, int(n), _p(out), _nt())
    return out


def words(seed, stream, n):
    """n raw uint32 words (Philox4x32-10 outputs in counter order)."""
    n = int(n)
    out = np.empty(4 * ((n + 3) // 4), np.uint32)
    _load().ig_words(seed, stream, out.size // 4, _p(out), _nt())
    return out[:n]


def random_bytes(seed, stream, shape):
    n = int(np.prod(shape))
    return words(seed, stream, (n + 3) // 4).view(np.uint8)[:n].reshape(shape)


def acceptance_counts(seed, B, gamma, alpha):
    """Accepted drafts per request under a fixed per-position acceptance rate alpha: the number of
    leading successes among gamma Bernoulli(alpha) trials (0..gamma)."""
    if gamma == 0:
        return np.zeros(B, np.int32)
    ok = uniform53(seed, S_ACC, B * gamma).reshape(B, gamma) < alpha
    first_fail = np.where(ok.all(axis=1), gamma, np.argmin(ok, axis=1))
    return first_fail.astype(np.int32)


def kv_inputs(B, gamma, R, E, S, W, seed, *, alpha=0.8, len_hi=None):
    """One KV commit step: staged keys and values [B, gamma+1, R, E] (random bytes), lengths
    uniform in [0, len_hi) (default 4*(S+W): filling caches and wrapped rings), and accepted
    counts from acceptance_counts."""
    len_hi = 4 * (S + W) if len_hi is None else len_hi
    return {"k_new": random_bytes(seed, S_KV, (B, gamma + 1, R, E)),
            "v_new": random_bytes(seed + 1, S_KV, (B, gamma + 1, R, E)),
            "lengths": np.minimum(uniform53(seed, S_LEN, B) * len_hi, len_hi - 1).astype(np.int32),
            "num_accepted": acceptance_counts(seed, B, gamma, alpha),
            "sink": S, "window": W, "gamma": gamma, "rows": R, "row_bytes": E}


def window_inputs(B, W, block, K, full_cols, seed, *, len_hi=None):
    """One draft-window step: lengths uniform in [0, len_hi] (default the full table's tokens) and a
    full block table [B, full_cols] of distinct block ids (a seeded permutation, from 1)."""
    len_hi = full_cols * block if len_hi is None else len_hi
    perm = np.argsort(words(seed, S_TABLE, B * full_cols), kind="stable")
    return {"seq_lens": np.minimum(uniform53(seed, S_LEN, B) * (len_hi + 1), len_hi).astype(np.int32),
            "block_table": (perm.reshape(B, full_cols) + 1).astype(np.int32),
            "window": W, "block_size": block, "future_offset": K}


def logit_rows(seed, V, src_row, *, dist=DIST_NORMAL, scale=1.0, n_spikes=0, spike_height=0.0,
               noise_sd=None, noise_row=None, dtype="f32"):
    """Rows of synthetic logits; see gen.c for the exact recipe."""
    src = np.ascontiguousarray(src_row, np.int64)
    n = src.shape[0]
    sd = None if noise_sd is None else np.ascontiguousarray(np.broadcast_to(noise_sd, (n,)), np.float64)
    nr = None if noise_row is None else np.ascontiguousarray(noise_row, np.int64)
    out = np.empty((n, V), np.float32 if dtype == "f32" else np.uint16)
    rc = _load().ig_logit_rows(seed, dist, float(scale), int(n_spikes), float(spike_height), n, int(V), _p(src),
                               _p(sd), _p(nr), 0 if dtype == "f32" else 1, _p(out), _nt())
    if rc != 0:
        raise ValueError("ig_logit_rows: bad arguments")
    return out


def sample_tokens(seed, rows, T_per_row, row_key, stream=S_TOKENS):
    """Draw one token per row from softmax(row / T) (Gumbel-max); T == 0 -> lowest argmax."""
    rows = np.ascontiguousarray(rows)
    V = rows.shape[-1]
    n = rows.size // V
    T = np.ascontiguousarray(np.broadcast_to(np.asarray(T_per_row, np.float32), (n,)))
    key = np.ascontiguousarray(row_key, np.int64)
    out = np.empty(n, np.int32)
    dt = 0 if rows.dtype == np.float32 else 1
    rc = _load().ig_sample_tokens(seed, stream, n, int(V), dt, _p(rows), _p(T), _p(key), _p(out), _nt())
    if rc != 0:
        raise ValueError("ig_sample_tokens: bad arguments")
    return out


# ---------------------------------------------------------------------------
# Workload recipes


def chain_inputs(B, gamma, V, seed, *, dtype="f32", dist=DIST_NORMAL, scale=1.0, n_spikes=0,
                 spike_height=0.0, noise_sd=0.7, temperature=1.0):
    """Dense chain batch: target [B, g+1, V], draft [B, g, V], tokens/u_accept [B, g], u_sample [B, g+1]."""
    T = np.array(np.broadcast_to(np.asarray(temperature, np.float32), (B,)), dtype=np.float32)
    sd = np.broadcast_to(np.asarray(noise_sd, np.float64), (B,))
    trow = np.arange(B * (gamma + 1), dtype=np.int64)
    target = logit_rows(seed, V, trow, dist=dist, scale=scale, n_spikes=n_spikes, spike_height=spike_height,
                        dtype=dtype)
    b = np.repeat(np.arange(B), gamma)
    i = np.tile(np.arange(gamma), B)
    src = (b * (gamma + 1) + i).astype(np.int64)
    drow = np.arange(B * gamma, dtype=np.int64)
    draft = logit_rows(seed, V, src, dist=dist, scale=scale, n_spikes=n_spikes, spike_height=spike_height,
                       noise_sd=sd[b], noise_row=drow, dtype=dtype)
    tokens = sample_tokens(seed, draft, T[b], drow)
    return dict(
        target=target.reshape(B, gamma + 1, V),
        draft=draft.reshape(B, gamma, V),
        draft_tokens=tokens.reshape(B, gamma),
        u_accept=uniform24(seed, S_UACC, B * gamma).reshape(B, gamma),
        u_sample=uniform24(seed, S_USAMP, B * (gamma + 1)).reshape(B, gamma + 1),
        temperature=T,
    )


def ragged_inputs(B, gamma_lo, gamma_hi, V, seed, *, dtype="bf16", dist=DIST_NORMAL, scale=3.0, sigma_lo=0.2,
                  sigma_hi=2.0, n_greedy=0, t_lo=0.5, t_hi=1.2):
    """Packed ragged batch with per-request gamma_b, sigma_b and temperature."""
    ug = uniform53(seed, S_GAMMA, B)
    gam = (gamma_lo + np.floor(ug * (gamma_hi - gamma_lo + 1))).astype(np.int64)
    gam = np.minimum(gam, gamma_hi)
    cu = np.zeros(B + 1, np.int64)
    cu[1:] = np.cumsum(gam)
    sig = sigma_lo + (sigma_hi - sigma_lo) * uniform53(seed, S_SIGMA, B)
    T = (t_lo + (t_hi - t_lo) * uniform53(seed, S_TEMP, B)).astype(np.float32)
    if n_greedy:
        order = np.argsort(uniform53(seed, S_PERM, B), kind="stable")
        T[order[:n_greedy]] = 0.0
    total = int(cu[-1])
    # target row of request b, position i: cu[b] + b + i ; draft row: cu[b] + i
    tb = np.repeat(np.arange(B), gam + 1)
    trow = np.arange(total + B, dtype=np.int64)
    target = logit_rows(seed, V, trow, dist=dist, scale=scale, dtype=dtype)
    db = np.repeat(np.arange(B), gam)
    dpos = np.arange(total) - cu[db]
    src = (cu[db] + db + dpos).astype(np.int64)
    drow = np.arange(total, dtype=np.int64)
    draft = logit_rows(seed, V, src, dist=dist, scale=scale, noise_sd=sig[db], noise_row=drow, dtype=dtype)
    tokens = sample_tokens(seed, draft, T[db], drow)
    del tb
    return dict(
        target=target, draft=draft, draft_tokens=tokens, cu_gamma=cu.astype(np.int32),
        u_accept=uniform24(seed, S_UACC, total), u_sample=uniform24(seed, S_USAMP, total + B),
        temperature=T, gamma_max=int(gamma_hi), total_draft=total,
    )


def tree_structure(B, seed, fanout=(4, 4, 3), n_nodes=64):
    """BFS token trees: root, fanout[0] children, fanout[1] children each, then up to fanout[2]
    children per depth-2 node until n_nodes nodes; which depth-2 nodes get fewer is seeded."""
    parents = np.empty((B, n_nodes), np.int32)
    for b in range(B):
        par = [-1]
        level = [0]
        for d, f in enumerate(fanout):
            nxt = []
            if d < len(fanout) - 1:
                counts = [f] * len(level)
            else:
                room = n_nodes - len(par)
                counts = [f] * len(level)
                short = f * len(level) - room
                if short > 0:
                    keys = uniform53(seed, S_TREE, (b + 1) * len(level))[b * len(level):]
                    for k in np.argsort(keys, kind="stable")[:short]:
                        counts[k] -= 1
            for p, c in zip(level, counts):
                for _ in range(c):
                    nxt.append(len(par))
                    par.append(p)
            level = nxt
        if len(par) != n_nodes:
            raise ValueError("fanout does not produce n_nodes nodes")
        parents[b] = par
    return parents


def tree_inputs(B, V, seed, *, n_nodes=64, fanout=(4, 4, 3), dtype="bf16", scale=3.0, noise_sd=0.7,
                temperature=1.0, iid_draft=False):
    """Token-tree batch: target [B, N, V], draft [B, N-1, V] (row v-1 belongs to node v)."""
    N = n_nodes
    parents = tree_structure(B, seed, fanout, N)
    depth = np.zeros((B, N), np.int32)
    for v in range(1, N):
        depth[:, v] = depth[np.arange(B), parents[:, v]] + 1
    T = np.array(np.broadcast_to(np.asarray(temperature, np.float32), (B,)), dtype=np.float32)
    target = logit_rows(seed, V, np.arange(B * N, dtype=np.int64), scale=scale, dtype=dtype)
    b = np.repeat(np.arange(B), N - 1)
    v = np.tile(np.arange(1, N), B)
    drow = np.arange(B * (N - 1), dtype=np.int64)
    if iid_draft:
        draft = logit_rows(seed, V, B * N + drow, scale=scale, dtype=dtype)
    else:
        src = (b * N + parents[b, v]).astype(np.int64)
        draft = logit_rows(seed, V, src, scale=scale, noise_sd=noise_sd, noise_row=drow, dtype=dtype)
    tok = sample_tokens(seed, draft, T[b], drow)
    tokens = np.zeros((B, N), np.int32)
    tokens[:, 1:] = tok.reshape(B, N - 1)
    return dict(
        target=target.reshape(B, N, V), draft=draft.reshape(B, N - 1, V), node_tokens=tokens, parents=parents,
        u_accept=uniform24(seed, S_UACC, B * N).reshape(B, N),
        u_sample=uniform24(seed, S_USAMP, B * N).reshape(B, N),
        temperature=T, max_depth=int(depth.max()),
    )


def near_identical_trees(B, V, seed, *, dtype, noise_sd):
    """Token trees (21 nodes: 4 children of the root, 4 under each, one under each of those) whose
    draft rows lie within noise_sd of their parent's target row, T = 1. The first child of every
    node, and every second sibling after it, gets an acceptance uniform of 0.999, so most of them
    are rejected and the residual they leave (about the rows' total variation) is small."""
    d = tree_inputs(B, V, seed, n_nodes=21, fanout=(4, 4, 1), dtype=dtype, noise_sd=noise_sd)
    ua = d["u_accept"].copy()
    par = d["parents"]
    for b in range(par.shape[0]):
        for v in range(1, par.shape[1]):
            p = int(par[b, v])
            first = min(c for c in range(1, par.shape[1]) if par[b, c] == p)
            if v == first or (v - first) % 2 == 1:
                ua[b, v] = 0.999
    d["u_accept"] = ua
    return d


WORKLOADS = {
    "tiny": dict(kind="chain", B=8, gamma=4, V=256, dtype="f32", scale=2.0, noise_sd=0.7, temperature=1.0,
                 seed=1),
    "mid": dict(kind="chain", B=64, gamma=5, V=32000, dtype="f32", scale=3.0, n_spikes=20, spike_height=8.0,
                noise_sd=0.5, temperature=0.8, seed=2),
    "large": dict(kind="chain", B=256, gamma=5, V=128256, dtype="bf16", dist=DIST_T3, scale=2.5,
                  noise_sd=1.0, temperature=1.0, seed=3),
    "tree": dict(kind="tree", B=32, V=152064, dtype="bf16", scale=3.0, noise_sd=0.7, temperature=1.0, seed=4),
    "ragged": dict(kind="ragged", B=1024, gamma_lo=1, gamma_hi=8, V=151936, dtype="bf16", scale=3.0,
                   sigma_lo=0.2, sigma_hi=2.0, n_greedy=256, t_lo=0.5, t_hi=1.2, seed=5),
    "kv": dict(kind="kv", B=256, gamma=5, R=256, E=256, S=4, W=1020, alpha=0.8, seed=6),
    "window": dict(kind="window", B=256, W=2048, block=128, K=5, full_cols=320, seed=7),
}


def make(name, seed=None, **overrides):
    """Build a named workload (optionally with another seed or smaller sizes)."""
    spec = dict(WORKLOADS[name])
    spec.update(overrides)
    kind = spec.pop("kind")
    s = spec.pop("seed") if seed is None else seed
    spec.pop("seed", None)
    if kind == "chain":
        return chain_inputs(spec.pop("B"), spec.pop("gamma"), spec.pop("V"), s, **spec)
    if kind == "ragged":
        return ragged_inputs(spec.pop("B"), spec.pop("gamma_lo"), spec.pop("gamma_hi"), spec.pop("V"), s, **spec)
    if kind == "tree":
        return tree_inputs(spec.pop("B"), spec.pop("V"), s, **spec)
    if kind == "kv":
        return kv_inputs(spec.pop("B"), spec.pop("gamma"), spec.pop("R"), spec.pop("E"), spec.pop("S"),
                         spec.pop("W"), s, **spec)
    if kind == "window":
        return window_inputs(spec.pop("B"), spec.pop("W"), spec.pop("block"), spec.pop("K"), spec.pop("full_cols"),
                             s, **spec)
    raise KeyError(kind)
